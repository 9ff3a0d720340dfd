/* Drives the host-side checks of the C ABI (include/kda.h) in a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: size functions, null /
 * misaligned pointers, bad sizes, undersized saved buffers and workspaces,
 * unsupported configurations and the static workspace's limit.  Every call
 * here fails its checks before any HIP call, with fake device addresses that
 * are never dereferenced.  Prints "abi checks ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/kda.h"

static int failures = 0;
#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            fprintf(stderr, "check failed at line %d: %s (last error: %s)\n",        \
                    __LINE__, #cond, kda_last_error());                              \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

#define FAKE ((void*)(uintptr_t)(1u << 20))

int main(void) {
    kda_config cfg;
    kda_config_init(&cfg, 32, 128, 128);
    cfg.in_dtype = KDA_BF16;
    const int64_t T = 4 * 8192;
    const int32_t N = 4;
    const size_t saved = kda_saved_size(&cfg, T, N);
    const size_t wsb = kda_bwd_workspace_size(&cfg, T, N);
    CHECK(saved > 0 && wsb > 0 && kda_fwd_workspace_size(&cfg, T, N) == 0);
    CHECK(kda_saved_size(NULL, T, N) == 0 && kda_saved_size(&cfg, -1, N) == 0 && kda_saved_size(&cfg, T, 0) == 0);

    /* forward: each case fails its checks */
    CHECK(kda_fwd(NULL, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0, NULL) ==
          KDA_ERR_INVALID_ARG);
    CHECK(kda_fwd(&cfg, T, N, NULL, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0, NULL) ==
          KDA_ERR_INVALID_ARG);
    CHECK(strstr(kda_last_error(), "q") != NULL);
    CHECK(kda_fwd(&cfg, T, N, (char*)FAKE + 2, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0,
                  NULL) == KDA_ERR_INVALID_ARG);
    CHECK(kda_fwd(&cfg, T + 1, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0, NULL) ==
          KDA_ERR_INVALID_ARG);
    CHECK(kda_fwd(&cfg, (int64_t)1 << 31, 1, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0,
                  NULL) == KDA_ERR_INVALID_ARG);
    cfg.flags = KDA_FLAG_SAVE_FOR_BWD;
    CHECK(kda_fwd(&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, FAKE, saved - 1, NULL, 0, NULL) ==
          KDA_ERR_WORKSPACE);
    CHECK(kda_fwd_static(&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL) ==
          KDA_ERR_INVALID_ARG);
    cfg.flags = 1u << 7;
    CHECK(kda_fwd(&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0, NULL) ==
          KDA_ERR_INVALID_ARG);
    cfg.flags = 0;
    cfg.dk = 96;
    CHECK(kda_fwd(&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0, NULL) ==
          KDA_ERR_UNSUPPORTED);
    cfg.dk = 128;
    cfg.chunk = 32;
    CHECK(kda_fwd(&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL, 0, NULL) ==
          KDA_ERR_UNSUPPORTED);
    cfg.chunk = 64;

    /* the long-sequence split needs a workspace; the static one has a limit */
    {
        kda_config c1;
        kda_config_init(&c1, 16, 128, 128);
        c1.in_dtype = KDA_BF16;
        const size_t need = kda_fwd_workspace_size(&c1, (int64_t)1 << 20, 1);
        CHECK(need > 0 && need <= KDA_STATIC_WORKSPACE_BYTES);
        CHECK(kda_fwd(&c1, (int64_t)1 << 20, 1, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, FAKE,
                      need - 1, NULL) == KDA_ERR_WORKSPACE);
        kda_config c2;
        kda_config_init(&c2, 1, 128, 64);
        c2.in_dtype = KDA_BF16;
        int64_t t2 = ((int64_t)(1 << 23) - 127 - 1) * 64;
        t2 -= t2 % 127;
        CHECK(kda_fwd_workspace_size(&c2, t2, 127) > KDA_STATIC_WORKSPACE_BYTES);
        CHECK(kda_fwd_static(&c2, t2, 127, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, NULL, NULL, 0, NULL) ==
              KDA_ERR_WORKSPACE);
        CHECK(strstr(kda_last_error(), "static workspace") != NULL);
    }

    /* backward and its stages */
    kda_status (*bwd[3])(const kda_config*, int64_t, int32_t, const void*, const void*, const void*, const void*,
                         const void*, const int32_t*, const float*, const void*, size_t, const void*, const float*,
                         void*, void*, void*, void*, void*, float*, void*, size_t,
                         void*) = {kda_bwd, kda_bwd_scan, kda_bwd_grads};
    for (int i = 0; i < 3; ++i) {
        CHECK(bwd[i](&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, saved, FAKE, NULL, FAKE, FAKE, FAKE,
                     FAKE, FAKE, NULL, FAKE, wsb - 1, NULL) == KDA_ERR_WORKSPACE);
        CHECK(bwd[i](&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, saved - 1, FAKE, NULL, FAKE, FAKE,
                     FAKE, FAKE, FAKE, NULL, FAKE, wsb, NULL) == KDA_ERR_WORKSPACE);
        CHECK(bwd[i](&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, NULL, saved, FAKE, NULL, FAKE, FAKE, FAKE,
                     FAKE, FAKE, NULL, FAKE, wsb, NULL) == KDA_ERR_INVALID_ARG);
        CHECK(bwd[i](&cfg, T, N, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, saved, NULL, NULL, FAKE, FAKE, FAKE,
                     FAKE, FAKE, NULL, FAKE, wsb, NULL) == KDA_ERR_INVALID_ARG);
    }

    /* decode */
    CHECK(kda_decode(&cfg, -1, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, NULL) == KDA_ERR_INVALID_ARG);
    CHECK(kda_decode(&cfg, 8, FAKE, FAKE, FAKE, FAKE, FAKE, (float*)FAKE + 64, (float*)FAKE, FAKE, NULL) ==
          KDA_ERR_INVALID_ARG);

    /* status strings */
    for (int s = 0; s <= 5; ++s) CHECK(kda_status_string((kda_status)s) != NULL);
    CHECK(kda_version() > 0);

    if (failures) {
        fprintf(stderr, "%d abi checks failed\n", failures);
        return 1;
    }
    printf("abi checks ok\n");
    return 0;
}
