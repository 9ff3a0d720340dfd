// kda_api.hip -- the C ABI declared in include/kda.h.
//
// Validates every argument on the host before any HIP call, sizes the saved
// and workspace buffers, and hands the work to the kernel launchers.  The
// library allocates nothing.  Its only global state is the thread-local error
// text and, for kda_fwd_static, one static device workspace per GPU with the
// table of its device addresses.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

#define KDA_TRY_(x)                      \
    do {                                 \
        kda_status _s = (x);             \
        if (_s != KDA_OK) return _s;     \
    } while (0)

namespace {

thread_local char g_err[256] = "";

kda_status fail(kda_status s, const char* fmt, const char* what = "") {
    snprintf(g_err, sizeof g_err, fmt, what);
    return s;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Saved per-chunk states and state gradients: fp32 [dk][dv] for fp32 inputs;
// fp16 with a power-of-two scale per 16-column group for bf16 inputs (the fp16
// kernels hold them as fp16-safe scaled values already), blocked by those 16
// columns ([dv/16][dk][16]) so that each wave's save is contiguous.
size_t state_elem_bytes(const kda_config* c) { return c->in_dtype == KDA_BF16 ? 2 : 4; }

// The scales of the fp16 saves: one fp32 per (slot, head, 16-column group).
size_t scale_bytes(const kda_config* c, int64_t T, int32_t N) {
    if (c->in_dtype != KDA_BF16) return 0;
    return (size_t)kda::num_slots(T, N) * c->H * (c->dv / 16) * sizeof(float);
}

// Config check shared by every entry point.  Returns KDA_OK or a status with
// the reason left in g_err.
// Everything but the chunk kernels' dtype/dim restriction (the decode step has none).
kda_status check_config_common(const kda_config* c) {
    if (!c) return fail(KDA_ERR_INVALID_ARG, "config is NULL%s");
    if (c->H < 1) return fail(KDA_ERR_INVALID_ARG, "H must be >= 1%s");
    if ((c->dk != 64 && c->dk != 128) || (c->dv != 64 && c->dv != 128))
        return fail(KDA_ERR_UNSUPPORTED, "dk and dv must be 64 or 128%s");
    if (c->chunk != kda::kChunk && !((c->flags & KDA_FLAG_STAGED) && (c->chunk == 16 || c->chunk == 32)))
        return fail(KDA_ERR_UNSUPPORTED, "chunk must be 64 (16 or 32 only with KDA_FLAG_STAGED)%s");
    if ((c->in_dtype != KDA_F32 && c->in_dtype != KDA_BF16) ||
        (c->out_dtype != KDA_F32 && c->out_dtype != KDA_BF16))
        return fail(KDA_ERR_INVALID_ARG, "unknown dtype%s");
    if (!(c->l2_eps >= 0.f) || !isfinite(c->l2_eps)) return fail(KDA_ERR_INVALID_ARG, "l2_eps must be finite and >= 0%s");
    if (!isfinite(c->scale)) return fail(KDA_ERR_INVALID_ARG, "scale must be finite%s");
    if (c->flags & ~(KDA_FLAG_SAVE_FOR_BWD | KDA_FLAG_SEQUENTIAL | KDA_FLAG_STAGED))
        return fail(KDA_ERR_INVALID_ARG, "unknown flag bits%s");
    return KDA_OK;
}

// Config check shared by the chunked entry points.
kda_status check_config(const kda_config* c) { return check_config_common(c); }

// One launch covers at most 2^32 - 1 work-items along x (the dispatch packet's
// grid size is a 32-bit count of work-items).
bool grid_fits(int64_t workgroups, int threads) {
    return workgroups >= 0 && workgroups * threads <= (int64_t)UINT32_MAX;
}

kda_status check_sizes(const kda_config* c, int64_t T, int32_t N, const int32_t* cu) {
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(KDA_ERR_INVALID_ARG, "total_tokens must be in [0, 2^31)%s");
    if (N < 1) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 1%s");
    if (!cu && (T % N) != 0)
        return fail(KDA_ERR_INVALID_ARG, "cu_seqlens is NULL but total_tokens is not a multiple of num_seqs%s");
    if (!grid_fits((int64_t)N * c->H * (c->dv / kda::kSlice), kda::kWideThreads) ||
        !grid_fits(kda::num_slots(T, N) * c->H, kda::kWideThreads) ||
        !grid_fits((T / c->chunk + N) * c->H, kda::kWideThreads))
        return fail(KDA_ERR_UNSUPPORTED, "num_seqs, H or total_tokens too large for one launch%s");
    // the kernels address a chunk's rows with 32-bit offsets from a 64-bit base
    if ((int64_t)kda::kChunk * c->H * (c->dk > c->dv ? c->dk : c->dv) >= ((int64_t)1 << 31))
        return fail(KDA_ERR_UNSUPPORTED, "H too large%s");
    return KDA_OK;
}

kda_status need_ptr(const void* p, const char* name) {
    if (!p) return fail(KDA_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return KDA_OK;
}

kda_status opt_ptr(const void* p, const char* name) {
    if (p && !aligned16(p)) return fail(KDA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return KDA_OK;
}

// Per-chunk U (forward) and dU (reverse scan), fp16, 64 x dv per (slot, head) in
// MFMA fragment order (ufrag in kda_f16.h) (bf16 inputs): the bf16 chunk-gradient
// kernel reads them instead of recomputing both.
size_t chunk_u_bytes(const kda_config* c, int64_t T, int32_t N) {
    if (c->in_dtype != KDA_BF16) return 0;
    return (size_t)kda::num_slots(T, N) * c->H * kda::kChunk * c->dv * 2;
}

struct SavedLayout {
    size_t states, nq, nk, u, scale, total;
};

SavedLayout saved_layout(const kda_config* c, int64_t T, int32_t N) {
    SavedLayout s;
    const size_t st = (size_t)kda::num_slots(T, N) * c->H * c->dk * c->dv * state_elem_bytes(c);
    const size_t nrm = (size_t)T * c->H * sizeof(float);
    s.states = 0;
    s.nq = align256(st);
    s.nk = s.nq + align256(nrm);
    s.u = s.nk + align256(nrm);
    s.scale = s.u + align256(chunk_u_bytes(c, T, N));
    s.total = s.scale + align256(scale_bytes(c, T, N));
    return s;
}

// ---------------------------------------------------------------- two-level forward
// Few long sequences leave most compute units idle in the one-pass forward
// (one workgroup per sequence, head and value slice).  Then every document is
// split into segments (see kda_split.hip).  The plan depends on the config and
// the sizes only, so the workspace size is a pure host function.
constexpr int64_t kSplitMaxChains = 128;   // split only below this many (sequence, head, slice) chains
constexpr int64_t kSplitTargetWGs = 1024;  // aim for this many workgroups in the per-segment passes
constexpr int64_t kMinSegment = 4096;      // tokens; shorter segments spend more on maps than they save

struct SplitPlan {
    bool on;
    int32_t seg_len, P;   // segment length (multiple of the chunk) and segment capacity
    size_t seg_cu, doc_seg, sf_dst, maps, s_in, total;   // workspace offsets
};

SplitPlan split_plan(const kda_config* c, int64_t T, int32_t N) {
    SplitPlan s;
    memset(&s, 0, sizeof s);
    if (c->in_dtype != KDA_BF16 || (c->flags & (KDA_FLAG_SAVE_FOR_BWD | KDA_FLAG_SEQUENTIAL | KDA_FLAG_STAGED)) ||
        N < 1 || T < 1)
        return s;
    const int64_t chains = (int64_t)N * c->H * (c->dv / kda::kSlice);
    if (chains >= kSplitMaxChains) return s;
    const int64_t avg = T / N;
    const int64_t per_doc = (kSplitTargetWGs + chains - 1) / chains;
    int64_t L = (avg + per_doc - 1) / per_doc;
    L = (L + kda::kChunk - 1) / kda::kChunk * kda::kChunk;
    if (L < kMinSegment) L = kMinSegment;
    if (avg < 2 * L) return s;
    const int64_t P = T / L + N;
    if (P * c->H * ((c->dk + c->dv) / kda::kSlice) >= ((int64_t)1 << 31)) return s;
    s.on = true;
    s.seg_len = (int32_t)L;
    s.P = (int32_t)P;
    s.seg_cu = 0;
    s.doc_seg = align256((size_t)(P + 1) * 4);
    s.sf_dst = s.doc_seg + align256((size_t)(N + 1) * 4);
    s.maps = s.sf_dst + align256((size_t)P * 4);
    s.s_in = s.maps + align256((size_t)P * c->H * c->dk * (c->dk + c->dv) * sizeof(float));
    s.total = s.s_in + align256((size_t)P * c->H * c->dk * c->dv * sizeof(float));
    return s;
}

// dL/dS at the end of every chunk (state type), then dU of every chunk, the
// scales of both (bf16 inputs), then one flag per chunk and head (decay past
// the factorised kernels' range).
size_t bwd_dst_bytes(const kda_config* c, int64_t T, int32_t N) {
    return align256((size_t)kda::num_slots(T, N) * c->H * c->dk * c->dv * state_elem_bytes(c));
}
size_t bwd_flag_bytes(const kda_config* c, int64_t T, int32_t N) {
    return align256((size_t)kda::num_slots(T, N) * c->H * sizeof(int32_t));
}

// The staged forward's workspace: the eleven fp32 stage buffers of
// kda_stage, each [slots, H, ...] (slots = T / chunk + N) and 256-byte
// aligned, in enum order.
size_t stage_bytes(const kda_config* c, int64_t T, int32_t N, int stage) {
    const size_t C = c->chunk, dk = c->dk, dv = c->dv;
    const size_t sh = (size_t)(T / c->chunk + N) * c->H * sizeof(float);   // chunk slots x heads
    switch (stage) {
        case KDA_STAGE_G: case KDA_STAGE_W: case KDA_STAGE_QG: case KDA_STAGE_KTIL: return align256(sh * C * dk);
        case KDA_STAGE_AKK: case KDA_STAGE_AQK: case KDA_STAGE_T: return align256(sh * C * C);
        case KDA_STAGE_UT: case KDA_STAGE_U: return align256(sh * C * dv);
        case KDA_STAGE_S_IN: return align256(sh * dk * dv);
        case KDA_STAGE_GAMC: return align256(sh * dk);
        default: return 0;
    }
}
size_t stage_offset(const kda_config* c, int64_t T, int32_t N, int stage) {
    size_t off = 0;
    for (int i = 0; i < stage; ++i) off += stage_bytes(c, T, N, i);
    return off;
}

// Every argument check of kda_fwd except the workspace's.
kda_status fwd_check(const kda_config* cfg, int64_t T, int32_t N, const void* q, const void* k, const void* v,
                     const void* g, const void* beta, const int32_t* cu, const float* s0, const void* o,
                     const float* sfinal, const void* saved, size_t saved_bytes) {
    KDA_TRY_(check_config(cfg));
    KDA_TRY_(check_sizes(cfg, T, N, cu));
    if (T > 0) {
        KDA_TRY_(need_ptr(q, "q"));
        KDA_TRY_(need_ptr(k, "k"));
        KDA_TRY_(need_ptr(v, "v"));
        KDA_TRY_(need_ptr(g, "g"));
        KDA_TRY_(need_ptr(beta, "beta"));
        KDA_TRY_(need_ptr(o, "o"));
    }
    KDA_TRY_(opt_ptr(cu, "cu_seqlens"));
    KDA_TRY_(opt_ptr(s0, "initial_state"));
    KDA_TRY_(opt_ptr(sfinal, "final_state"));
    if ((cfg->flags & KDA_FLAG_STAGED) && (cfg->flags & KDA_FLAG_SAVE_FOR_BWD))
        return fail(KDA_ERR_UNSUPPORTED, "KDA_FLAG_STAGED does not fill the saved buffer%s");
    if (cfg->flags & KDA_FLAG_SAVE_FOR_BWD) {
        KDA_TRY_(need_ptr(saved, "saved"));
        if (saved_bytes < kda_saved_size(cfg, T, N)) return fail(KDA_ERR_WORKSPACE, "saved buffer too small%s");
    }
    return KDA_OK;
}

// The forward's launches, after every check; `workspace` holds at least
// kda_fwd_workspace_size() bytes.
kda_status fwd_launch(const kda_config* cfg, int64_t T, int32_t N, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const int32_t* cu, const float* s0, void* o,
                      float* sfinal, void* saved, void* workspace, hipStream_t st) {
    const bool save = (cfg->flags & KDA_FLAG_SAVE_FOR_BWD) != 0;
    kda::FwdParams p;
    memset(&p, 0, sizeof p);
    p.q = q; p.k = k; p.v = v; p.g = g; p.b = beta;
    p.cu = cu; p.s0 = s0; p.o = o; p.sfinal = sfinal;
    if (save) {
        const SavedLayout L = saved_layout(cfg, T, N);
        char* base = (char*)saved;
        p.st_saved = base + L.states;
        p.nq_saved = (float*)(base + L.nq);
        p.nk_saved = (float*)(base + L.nk);
        p.u_saved = chunk_u_bytes(cfg, T, N) ? (void*)(base + L.u) : nullptr;
        p.sv_scale = scale_bytes(cfg, T, N) ? (float*)(base + L.scale) : nullptr;
    }
    p.T = T; p.N = N; p.H = cfg->H; p.dv = cfg->dv;
    p.seqlen = cu ? 0 : (int32_t)(T / N);
    p.eps = cfg->l2_eps; p.scale = cfg->scale;
    p.nslices = cfg->dv / kda::kSlice;
    const SplitPlan sp = split_plan(cfg, T, N);
    hipError_t e = hipSuccess;
    if (cfg->flags & KDA_FLAG_STAGED) {
        kda::StagedParams sp2;
        memset(&sp2, 0, sizeof sp2);
        sp2.q = q; sp2.k = k; sp2.v = v; sp2.g = g; sp2.b = beta;
        sp2.cu = cu; sp2.s0 = s0; sp2.o = o; sp2.sfinal = sfinal;
        float** dst[KDA_STAGE_COUNT] = {&sp2.G, &sp2.Akk, &sp2.Aqk, &sp2.Tm, &sp2.W, &sp2.Ut,
                                        &sp2.U, &sp2.Sin, &sp2.QG, &sp2.Ktil, &sp2.GamC};
        for (int i = 0; i < KDA_STAGE_COUNT; ++i) *dst[i] = (float*)((char*)workspace + stage_offset(cfg, T, N, i));
        sp2.T = T; sp2.N = N; sp2.H = cfg->H; sp2.dv = cfg->dv;
        sp2.seqlen = p.seqlen;
        sp2.eps = cfg->l2_eps; sp2.scale = cfg->scale;
        if (T > 0) e = kda::launch_fwd_staged(sp2, cfg->in_dtype, cfg->out_dtype, cfg->dk, cfg->chunk, st);
    } else if (!sp.on) {
        e = kda::launch_fwd(p, cfg->in_dtype, cfg->out_dtype, cfg->dk, save, st);
    } else {
        char* ws = (char*)workspace;
        int32_t* seg_cu = (int32_t*)(ws + sp.seg_cu);
        int32_t* doc_seg = (int32_t*)(ws + sp.doc_seg);
        int32_t* sf_dst = (int32_t*)(ws + sp.sf_dst);
        float* maps = (float*)(ws + sp.maps);
        float* s_in = (float*)(ws + sp.s_in);
        kda::SegParams sg = {cu, seg_cu, doc_seg, sf_dst, T, N, p.seqlen, sp.seg_len, sp.P};
        e = kda::launch_segments(sg, st);
        if (e == hipSuccess) {   // every segment's [M | B] from the zero state
            kda::FwdParams pm = p;
            pm.cu = seg_cu; pm.N = sp.P; pm.seqlen = 0;
            pm.s0 = nullptr; pm.o = nullptr; pm.sfinal = maps; pm.sf_dst = nullptr;
            pm.nslices = (cfg->dk + cfg->dv) / kda::kSlice;
            pm.map_slices = cfg->dk / kda::kSlice;
            e = kda::launch_fwd_maps(pm, cfg->dk, st);
        }
        if (e == hipSuccess) {   // the state entering every segment
            kda::CarryParams cp = {doc_seg, s0, maps, s_in, N, cfg->H, cfg->dv, cfg->dv / kda::kCarryCols};
            e = kda::launch_carry(cp, cfg->dk, st);
        }
        if (e == hipSuccess) {   // the segments from their entering states
            kda::FwdParams pc = p;
            pc.cu = seg_cu; pc.N = sp.P; pc.seqlen = 0;
            pc.s0 = s_in; pc.sf_dst = sf_dst;
            e = kda::launch_fwd(pc, cfg->in_dtype, cfg->out_dtype, cfg->dk, false, st);
        }
    }
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

// ---------------------------------------------------------- static workspace
// kda_fwd_static's workspace: one array per GPU, placed by the code object
// loader, held until the process ends.  Host code never passes `scratch`
// itself (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[KDA_STATIC_WORKSPACE_BYTES];
// the host check of a call's workspace against the array uses the array's own size
constexpr size_t kStaticWorkspaceBytes = sizeof(scratch);
static_assert(kStaticWorkspaceBytes == KDA_STATIC_WORKSPACE_BYTES, "static workspace size");

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];

kda_status static_workspace(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_UNSUPPORTED, "device index out of range%s");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "hipGetSymbolAddress of the static workspace failed: %s",
                                         hipGetErrorString(e));
        if (!ptr) return fail(KDA_ERR_HIP, "the static workspace has no device address%s");
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return KDA_OK;
}

}  // namespace

#define KDA_TRY(x) KDA_TRY_(x)

extern "C" {

void kda_config_init(kda_config* cfg, int32_t H, int32_t dk, int32_t dv) {
    if (!cfg) return;
    memset(cfg, 0, sizeof *cfg);
    cfg->H = H;
    cfg->dk = dk;
    cfg->dv = dv;
    cfg->chunk = kda::kChunk;
    cfg->in_dtype = KDA_F32;
    cfg->out_dtype = KDA_F32;
    cfg->l2_eps = 1e-6f;
    cfg->scale = 1.0f;
    cfg->flags = 0;
}

size_t kda_saved_size(const kda_config* cfg, int64_t T, int32_t N) {
    if (check_config(cfg) != KDA_OK || T < 0 || N < 1) return 0;
    return saved_layout(cfg, T, N).total;
}

size_t kda_fwd_workspace_size(const kda_config* cfg, int64_t T, int32_t N) {
    if (check_config(cfg) != KDA_OK || T < 0 || N < 1) return 0;
    if (cfg->flags & KDA_FLAG_STAGED) return stage_offset(cfg, T, N, KDA_STAGE_COUNT);
    return split_plan(cfg, T, N).total;
}

size_t kda_stage_offset(const kda_config* cfg, int64_t T, int32_t N, int32_t stage) {
    if (check_config(cfg) != KDA_OK || T < 0 || N < 1 || stage < 0 || stage > KDA_STAGE_COUNT) return 0;
    return stage_offset(cfg, T, N, stage);
}

size_t kda_bwd_workspace_size(const kda_config* cfg, int64_t T, int32_t N) {
    if (check_config(cfg) != KDA_OK || T < 0 || N < 1) return 0;
    return bwd_dst_bytes(cfg, T, N) + align256(chunk_u_bytes(cfg, T, N)) + align256(scale_bytes(cfg, T, N)) +
           bwd_flag_bytes(cfg, T, N);
}

kda_status kda_fwd(const kda_config* cfg, int64_t T, int32_t N, const void* q, const void* k,
                   const void* v, const void* g, const void* beta, const int32_t* cu,
                   const float* s0, void* o, float* sfinal, void* saved, size_t saved_bytes,
                   void* workspace, size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    KDA_TRY(fwd_check(cfg, T, N, q, k, v, g, beta, cu, s0, o, sfinal, saved, saved_bytes));
    KDA_TRY(opt_ptr(workspace, "workspace"));
    const size_t ws_need = kda_fwd_workspace_size(cfg, T, N);
    if (workspace_bytes < ws_need) return fail(KDA_ERR_WORKSPACE, "workspace too small%s");
    if (ws_need > 0) KDA_TRY(need_ptr(workspace, "workspace"));
    return fwd_launch(cfg, T, N, q, k, v, g, beta, cu, s0, o, sfinal, saved, workspace, (hipStream_t)stream);
}

kda_status kda_fwd_static(const kda_config* cfg, int64_t T, int32_t N, const void* q, const void* k,
                          const void* v, const void* g, const void* beta, const int32_t* cu,
                          const float* s0, void* o, float* sfinal, void* saved, size_t saved_bytes,
                          void* stream) {
    g_err[0] = 0;
    KDA_TRY(fwd_check(cfg, T, N, q, k, v, g, beta, cu, s0, o, sfinal, saved, saved_bytes));
    const size_t ws_need = kda_fwd_workspace_size(cfg, T, N);
    if (ws_need > kStaticWorkspaceBytes) {
        snprintf(g_err, sizeof g_err,
                 "the call needs %zu bytes of workspace, above the static workspace's %zu: call kda_fwd",
                 ws_need, kStaticWorkspaceBytes);
        return KDA_ERR_WORKSPACE;
    }
    void* ws = nullptr;
    if (ws_need > 0) KDA_TRY(static_workspace(&ws));
    return fwd_launch(cfg, T, N, q, k, v, g, beta, cu, s0, o, sfinal, saved, ws, (hipStream_t)stream);
}

kda_status kda_decode(const kda_config* cfg, int32_t N, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* state_in, float* state_out, void* o,
                      void* stream) {
    g_err[0] = 0;
    KDA_TRY(check_config_common(cfg));
    if (N < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0%s");
    if (!grid_fits((int64_t)N * cfg->H * (cfg->dv / kda::kSlice), kda::kThreads))
        return fail(KDA_ERR_UNSUPPORTED, "num_seqs * H too large for one launch%s");
    if (N > 0) {
        KDA_TRY(need_ptr(q, "q"));
        KDA_TRY(need_ptr(k, "k"));
        KDA_TRY(need_ptr(v, "v"));
        KDA_TRY(need_ptr(g, "g"));
        KDA_TRY(need_ptr(beta, "beta"));
        KDA_TRY(need_ptr(state_out, "state_out"));
        KDA_TRY(need_ptr(o, "o"));
    }
    KDA_TRY(opt_ptr(state_in, "state_in"));
    if (state_in && state_in != state_out) {
        const size_t bytes = (size_t)N * cfg->H * cfg->dk * cfg->dv * sizeof(float);
        const char *a = (const char*)state_in, *b = (const char*)state_out;
        if (a < b + bytes && b < a + bytes)
            return fail(KDA_ERR_INVALID_ARG, "state_in and state_out overlap without being equal%s");
    }
    kda::DecodeParams p;
    memset(&p, 0, sizeof p);
    p.q = q; p.k = k; p.v = v; p.g = g; p.b = beta;
    p.s_in = state_in; p.s_out = state_out; p.o = o;
    p.N = N; p.H = cfg->H; p.dv = cfg->dv;
    p.eps = cfg->l2_eps; p.scale = cfg->scale;
    p.nslices = cfg->dv / kda::kSlice;
    hipError_t e = kda::launch_decode(p, cfg->in_dtype, cfg->out_dtype, cfg->dk, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

static kda_status bwd_call(int stages, const kda_config* cfg, int64_t T, int32_t N, const void* q,
                           const void* k, const void* v, const void* g, const void* beta, const int32_t* cu,
                           const float* s0, const void* saved, size_t saved_bytes, const void* dO,
                           const float* dSf, void* dq,
                           void* dk, void* dv, void* dg, void* dbeta, float* dS0, void* workspace,
                           size_t workspace_bytes, void* stream) {
    g_err[0] = 0;
    KDA_TRY(check_config(cfg));
    if (cfg->chunk != kda::kChunk) return fail(KDA_ERR_UNSUPPORTED, "the backward runs chunks of 64 only%s");
    KDA_TRY(check_sizes(cfg, T, N, cu));
    if (T > 0) {
        KDA_TRY(need_ptr(q, "q"));
        KDA_TRY(need_ptr(k, "k"));
        KDA_TRY(need_ptr(v, "v"));
        KDA_TRY(need_ptr(g, "g"));
        KDA_TRY(need_ptr(beta, "beta"));
        KDA_TRY(need_ptr(dO, "dO"));
        KDA_TRY(need_ptr(dq, "dq"));
        KDA_TRY(need_ptr(dk, "dk"));
        KDA_TRY(need_ptr(dv, "dv"));
        KDA_TRY(need_ptr(dg, "dg"));
        KDA_TRY(need_ptr(dbeta, "dbeta"));
    }
    KDA_TRY(need_ptr(saved, "saved"));
    if (saved_bytes < kda_saved_size(cfg, T, N)) return fail(KDA_ERR_WORKSPACE, "saved buffer too small%s");
    KDA_TRY(opt_ptr(cu, "cu_seqlens"));
    KDA_TRY(opt_ptr(s0, "initial_state"));
    KDA_TRY(opt_ptr(dSf, "dS_final"));
    KDA_TRY(opt_ptr(dS0, "d_initial_state"));
    const size_t need = kda_bwd_workspace_size(cfg, T, N);
    if (need > 0) KDA_TRY(need_ptr(workspace, "workspace"));
    if (workspace_bytes < need) return fail(KDA_ERR_WORKSPACE, "workspace too small%s");

    kda::BwdParams p;
    memset(&p, 0, sizeof p);
    const SavedLayout L = saved_layout(cfg, T, N);
    const char* base = (const char*)saved;
    p.q = q; p.k = k; p.v = v; p.g = g; p.b = beta; p.cu = cu;
    p.st_saved = base + L.states;
    p.nq_saved = (const float*)(base + L.nq);
    p.nk_saved = (const float*)(base + L.nk);
    p.dO = dO; p.dS_final = dSf;
    p.dst_saved = workspace;
    if (chunk_u_bytes(cfg, T, N)) {
        p.u_saved = (const void*)(base + L.u);
        p.du_ws = (void*)((char*)workspace + bwd_dst_bytes(cfg, T, N));
        p.sv_scale = (const float*)(base + L.scale);
        p.ds_scale = (float*)((char*)workspace + bwd_dst_bytes(cfg, T, N) + align256(chunk_u_bytes(cfg, T, N)));
    }
    p.chunk_flags = (int32_t*)((char*)workspace + bwd_dst_bytes(cfg, T, N) + align256(chunk_u_bytes(cfg, T, N)) +
                               align256(scale_bytes(cfg, T, N)));
    p.dq = dq; p.dk = dk; p.dv_out = dv; p.dg = dg; p.db = dbeta; p.dS0 = dS0;
    p.T = T; p.N = N; p.H = cfg->H; p.dv = cfg->dv;
    p.seqlen = cu ? 0 : (int32_t)(T / N);
    p.eps = cfg->l2_eps; p.scale = cfg->scale;
    p.nslices = cfg->dv / kda::kSlice;
    (void)s0;
    hipError_t e = kda::launch_bwd(p, cfg->in_dtype, cfg->out_dtype, cfg->dk, stages, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

#define KDA_BWD_ARGS                                                                                   \
    const kda_config *cfg, int64_t T, int32_t N, const void *q, const void *k, const void *v, const void *g, \
        const void *beta, const int32_t *cu, const float *s0, const void *saved, size_t saved_bytes,      \
        const void *dO,                                                                                   \
        const float *dSf, void *dq, void *dk, void *dv, void *dg, void *dbeta, float *dS0, void *workspace, \
        size_t workspace_bytes, void *stream
#define KDA_BWD_PASS cfg, T, N, q, k, v, g, beta, cu, s0, saved, saved_bytes, dO, dSf, dq, dk, dv, dg, dbeta, dS0, workspace, \
                     workspace_bytes, stream

kda_status kda_bwd(KDA_BWD_ARGS) { return bwd_call(kda::kBwdScan | kda::kBwdGrads, KDA_BWD_PASS); }
kda_status kda_bwd_scan(KDA_BWD_ARGS) { return bwd_call(kda::kBwdScan, KDA_BWD_PASS); }
kda_status kda_bwd_grads(KDA_BWD_ARGS) { return bwd_call(kda::kBwdGrads, KDA_BWD_PASS); }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
        case KDA_ERR_WORKSPACE: return "workspace or saved buffer too small";
        case KDA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_err; }

int32_t kda_version(void) { return 100; }

}  // extern "C"
