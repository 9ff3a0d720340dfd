/*
 * kda.h -- C ABI of libkda: Kimi Delta Attention (KDA) chunked forward and
 * backward on one AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The pages describe KDA in words: per head, a gated
 * matrix-valued state is read and written token by token in place of attention
 * over all past keys and values ("TorchTitan Ascend open source: Kimi K3.1 Pro
 * adaptation and training practice", jinguxun.com news 11080097, section
 * "Kimi K3.1 Pro model structure").  libkda implements the gated delta rule as
 * that recurrence.  For each document and head, with S a dk x dv fp32 state:
 *
 *     qh_t = scale * q_t / sqrt(|q_t|^2 + eps),  kh_t = k_t / sqrt(|k_t|^2 + eps)
 *     beta_t = sigmoid(b_t),   alpha_t = exp(g_t)          (g_t <= 0, per key channel)
 *     S_t  = (I - beta_t kh_t kh_t^T) Diag(alpha_t) S_{t-1} + beta_t kh_t v_t^T
 *     o_t  = S_t^T qh_t
 *
 * The work is organised as intra-chunk processing plus inter-chunk state
 * passing, with the Q/K normalisation, the beta transform and the gating fused
 * into the forward, and the backward reusing the statistics and states the
 * forward saved (same page, section "KDA pre/post-processing fusion"; also
 * "Ascend implements LoRA training of Kimi K3.1 Pro", jinguxun.com news
 * 11045563, section "KDA: big fused forward and backward").  Packed sequences
 * with document boundaries are supported through cu_seqlens (page 11080097,
 * section "Kimi K3.1 Pro Ascend training adaptation").  The chunking changes
 * only rounding, never the result.
 *
 * Conventions for every entry point.
 *  - Layouts (row-major, contiguous, token-major packed):
 *      q, k, g : [total_tokens, H, dk]      v, o, dO : [total_tokens, H, dv]
 *      beta    : [total_tokens, H]          (the logit b; sigmoid is applied inside)
 *      states  : [num_seqs, H, dk, dv] fp32 (dk is the outer index)
 *      cu_seqlens : [num_seqs + 1] int32 in device memory; cu[0] = 0,
 *                   non-decreasing, cu[num_seqs] = total_tokens.  NULL means
 *                   num_seqs equal sequences of total_tokens / num_seqs tokens.
 *  - All pointers except the config are device pointers (hipMalloc'ed or
 *    equivalent), 16-byte aligned, and owned by the caller.  Inputs are read
 *    only; outputs are fully overwritten.  The library never allocates, frees,
 *    synchronises or changes the current device, and keeps no global state
 *    apart from kda_fwd_static's workspace: every other entry point is
 *    re-entrant.  All work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL is the null stream).
 *  - Errors.  Arguments are validated on the host BEFORE any HIP call; a bad
 *    argument returns KDA_ERR_INVALID_ARG / KDA_ERR_UNSUPPORTED /
 *    KDA_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *    KDA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation.  kda_last_error() returns a thread-local description of
 *    the last failure.  No exception crosses this boundary.
 *  - cu_seqlens contents live on the device and are not checked on the host.
 *    A malformed cu_seqlens (decreasing, or last entry != total_tokens) is
 *    undefined behaviour; the kernels clamp every document to
 *    [0, total_tokens) so it cannot address memory outside the buffers.
 *  - Supported: dk, dv in {64, 128}; chunk = 64 (16 and 32 as well for the
 *    staged forward, KDA_FLAG_STAGED); in_dtype, out_dtype in
 *    {KDA_F32, KDA_BF16}; H >= 1 with 64 * H * max(dk, dv) < 2^31 (the
 *    kernels address a chunk's rows with 32-bit offsets); total_tokens < 2^31;
 *    one launch covers at most 2^32 - 1 work-items, so num_seqs * H * dv/64
 *    and (total_tokens/64 + num_seqs) * H stay below 2^23 (kda_decode:
 *    num_seqs * H * dv/64 below 2^24).  Outside these, KDA_ERR_UNSUPPORTED.
 *  - Gates: any g <= 0 (decay alpha in (0, 1]).  The matrix-core kernels
 *    factor the decay between two tokens of a chunk against a reference
 *    point; a chunk in which some channel decays past that factorisation's
 *    fp32 range (a per-chunk sum of g below about -60 per channel, or a
 *    16-token block below about -9.7 in the bf16 forward) runs through the
 *    recurrence token by token in the forward and the reverse scan, and its
 *    gradients through a kernel that forms the decay of every token pair
 *    directly.  The result is the same up to rounding; such chunks are slower.
 *    fp32 inputs at dk = 128 take those kernels for every chunk.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer   */
    KDA_ERR_UNSUPPORTED = 2, /* valid but not implemented (dk, dv, chunk...) */
    KDA_ERR_WORKSPACE = 3,   /* workspace or saved buffer too small          */
    KDA_ERR_HIP = 4          /* a HIP runtime call or launch failed          */
} kda_status;

typedef enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* kda_config.flags */
#define KDA_FLAG_SAVE_FOR_BWD 1u /* forward also fills `saved` for kda_bwd */
#define KDA_FLAG_SEQUENTIAL 2u   /* forward: never split long sequences into segments */
#define KDA_FLAG_STAGED 4u       /* forward: the staged correctness path, every stage
                                    written to the workspace (see kda_stage) */

typedef struct kda_config {
    int32_t H;         /* heads                                        */
    int32_t dk;        /* key / query head dim (64 or 128)             */
    int32_t dv;        /* value head dim (64 or 128)                   */
    int32_t chunk;     /* chunk length: 64 (16, 32 with KDA_FLAG_STAGED) */
    int32_t in_dtype;  /* kda_dtype of q, k, v, g, beta, dO            */
    int32_t out_dtype; /* kda_dtype of o, dq, dk, dv, dg, dbeta        */
    float l2_eps;      /* eps inside the L2 norm (1e-6 by default)     */
    float scale;       /* multiplies the normalised query (1.0)        */
    uint32_t flags;    /* KDA_FLAG_*                                   */
} kda_config;

/* Fill *cfg with defaults: chunk 64, eps 1e-6, scale 1, fp32/fp32, no flags. */
void kda_config_init(kda_config* cfg, int32_t H, int32_t dk, int32_t dv);

/* Sizes in bytes (pure host functions; 0 for an invalid config).
 * kda_saved_size: the buffer kda_fwd fills under KDA_FLAG_SAVE_FOR_BWD and
 * kda_bwd reads: per-chunk entering states, the per-token q/k norms (fp32)
 * and, for bf16 inputs, each chunk's pseudo-values U = T beta v - W S; for
 * bf16 inputs the states and U are fp16, each (chunk, head, 16 value columns)
 * scaled by a power of two kept beside them in fp32, for fp32 inputs the
 * states are fp32.
 * kda_fwd_workspace_size / kda_bwd_workspace_size: scratch for one call (the
 * backward's holds dL/dS at the end of every chunk and, for bf16 inputs, each
 * chunk's dL/dU, stored like the saved states; the forward's is non-zero only
 * when it splits long sequences, see kda_fwd, or under KDA_FLAG_STAGED, where
 * it holds the stages of kda_stage). */
size_t kda_saved_size(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs);
size_t kda_fwd_workspace_size(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs);
size_t kda_bwd_workspace_size(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs);

/* The staged forward (KDA_FLAG_STAGED on kda_fwd).  The chunk form of the
 * pages' intra-chunk processing plus inter-chunk state passing ("TorchTitan
 * Ascend open source: Kimi K3.1 Pro adaptation and training practice", section
 * "KDA pre/post-processing fusion"), run as two launches that write every
 * intermediate to the workspace: first every chunk in parallel (G, Akk, Aqk,
 * T, W, Ut and the scan's operands), then the state pass per document (U, o,
 * the entering states).  Plain fp32 arithmetic with the decay of every token
 * pair formed directly, so any g <= 0; slow; meant as a cross-check of the
 * fused kernels, stage by stage.  o and final_state are as from kda_fwd.
 * KDA_FLAG_SAVE_FOR_BWD with it returns KDA_ERR_UNSUPPORTED; the other entry
 * points ignore the flag.  Under this flag alone cfg->chunk may also be 16 or
 * 32 (C below), for chunk-size invariance checks: the chunking changes only
 * rounding.
 *
 * Each stage is an fp32 array indexed [slot][head][...], slots = total_tokens
 * / C + num_seqs, where chunk j of document n (tokens cu[n] + C j ..) has slot
 * floor(cu[n] / C) + n + j; a chunk's rows (and Akk/Aqk/T columns) past its
 * document's end are zero, and slots no chunk maps to are left unwritten.
 * Shapes below are for C = 64; for another C read C for 64.  With G the in-chunk inclusive
 * cumsum of g, qh, kh the normalised q (times scale) and k, E_rs =
 * exp(G_r - G_s) per channel: */
typedef enum kda_stage {
    KDA_STAGE_G = 0,    /* [64][dk] G                                              */
    KDA_STAGE_AKK = 1,  /* [64][64] beta_r sum_c kh_r kh_s E_rs for s < r, else 0  */
    KDA_STAGE_AQK = 2,  /* [64][64] sum_c qh_r kh_s E_rs for s <= r, else 0        */
    KDA_STAGE_T = 3,    /* [64][64] (I + Akk)^-1                                   */
    KDA_STAGE_W = 4,    /* [64][dk] T (beta kh exp(G))                             */
    KDA_STAGE_UT = 5,   /* [64][dv] T (beta v)                                     */
    KDA_STAGE_U = 6,    /* [64][dv] Ut - W S_in                                    */
    KDA_STAGE_S_IN = 7, /* [dk][dv] the state entering the chunk                   */
    KDA_STAGE_QG = 8,   /* [64][dk] qh exp(G)                                      */
    KDA_STAGE_KTIL = 9, /* [64][dk] kh exp(G_C - G), G_C = G of the chunk's last row */
    KDA_STAGE_GAMC = 10, /* [dk]    exp(G_C)                                       */
    KDA_STAGE_COUNT = 11
} kda_stage;

/* Byte offset of `stage` in the workspace of a KDA_FLAG_STAGED forward
 * (stage = KDA_STAGE_COUNT gives the total, which equals
 * kda_fwd_workspace_size under the flag).  Pure host function; 0 for an
 * invalid config or stage. */
size_t kda_stage_offset(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs, int32_t stage);

/* Forward.  o: [total_tokens, H, dv] in out_dtype.  initial_state: fp32
 * [num_seqs, H, dk, dv] or NULL (zero state; every document starts from its
 * own entry, never from the previous document).  final_state: fp32
 * [num_seqs, H, dk, dv] or NULL.  saved: required iff flags has
 * KDA_FLAG_SAVE_FOR_BWD, else ignored; saved_bytes is its size, and a
 * buffer smaller than kda_saved_size() returns KDA_ERR_WORKSPACE.  workspace
 * may be NULL when kda_fwd_workspace_size() is 0.
 *
 * Long sequences.  With bf16 inputs, no KDA_FLAG_SAVE_FOR_BWD and no
 * KDA_FLAG_SEQUENTIAL, when there are few (sequence, head) chains for the
 * GPU and the documents are long (the test is on cfg, total_tokens and
 * num_seqs only), every document is cut into segments: each segment's affine
 * map S_out = M S_in + B is computed in parallel, the maps are composed per
 * document in fp32, and the segments are rerun from their entering states.
 * The chunk boundaries do not move, so only rounding differs from the
 * one-pass forward.  The workspace (kda_fwd_workspace_size bytes) then holds
 * the segment bounds, the maps and the entering states ("Large models on
 * Ascend: from adaptation challenges to efficient training", ruibaoantu.com
 * 9569846, section 2: the KDA recurrence spread over many compute units). */
kda_status kda_fwd(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs, const void* q,
                   const void* k, const void* v, const void* g, const void* beta,
                   const int32_t* cu_seqlens, const float* initial_state, void* o,
                   float* final_state, void* saved, size_t saved_bytes, void* workspace,
                   size_t workspace_bytes, void* stream);

/* kda_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, checks and results are those of kda_fwd;
 * when the call needs a workspace (the long-sequence split), it uses a static
 * device array of KDA_STATIC_WORKSPACE_BYTES that the library holds on every
 * GPU it runs on until the process ends (one copy per GPU, found once per
 * device on its first use here).  A call whose kda_fwd_workspace_size()
 * exceeds that returns KDA_ERR_WORKSPACE and enqueues nothing.  Every call on
 * one GPU shares that GPU's array: calls on one GPU that can overlap (other
 * host threads, or work on other streams still in flight) race and must be
 * ordered by the caller.  The array needs no clearing: every byte a call reads
 * is written by that call first.  No hipMalloc, hipFree or other allocating
 * call is made. */
#define KDA_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
kda_status kda_fwd_static(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs, const void* q,
                          const void* k, const void* v, const void* g, const void* beta,
                          const int32_t* cu_seqlens, const float* initial_state, void* o,
                          float* final_state, void* saved, size_t saved_bytes, void* stream);

/* Backward of kda_fwd for the loss <dO, o> + <dS_final, final_state>.
 * Takes the same inputs as the forward plus `saved` (filled by a forward with
 * KDA_FLAG_SAVE_FOR_BWD on the same inputs; saved_bytes is its size, checked
 * against kda_saved_size() as in kda_fwd), dO ([total_tokens, H, dv],
 * in_dtype) and dS_final (fp32 [num_seqs, H, dk, dv] or NULL = 0).
 * Outputs, all in out_dtype: dq, dk, dg [total_tokens, H, dk] (gradients with
 * respect to the RAW q and k, through the L2 norm, and to g, the log-decay);
 * dv [total_tokens, H, dv]; dbeta [total_tokens, H] (with respect to the
 * logit b).  d_initial_state: fp32 [num_seqs, H, dk, dv] or NULL.
 * workspace: kda_bwd_workspace_size() bytes. */
kda_status kda_bwd(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs, const void* q,
                   const void* k, const void* v, const void* g, const void* beta,
                   const int32_t* cu_seqlens, const float* initial_state, const void* saved,
                   size_t saved_bytes, const void* dO, const float* dS_final, void* dq, void* dk, void* dv, void* dg,
                   void* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                   void* stream);

/* The two stages of kda_bwd, for callers that schedule or time them apart:
 * kda_bwd_scan runs the reverse state-gradient scan (it writes d_initial_state
 * and fills the workspace with dL/dS at the end of every chunk and, for bf16
 * inputs, each chunk's dL/dU); kda_bwd_grads runs the chunk-parallel gradients
 * from that workspace (it writes dq, dk, dv, dg, dbeta).  Both take exactly
 * kda_bwd's arguments and check them the same way.  kda_bwd_scan followed by
 * kda_bwd_grads on one stream, with the same arguments and the same workspace,
 * equals kda_bwd; the workspace must not be changed in between.  (Stage split:
 * "state-gradient propagation" and the Q/K gradients of "TorchTitan Ascend
 * open source: Kimi K3.1 Pro adaptation and training practice", section
 * "KDA pre/post-processing fusion".) */
kda_status kda_bwd_scan(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs, const void* q,
                        const void* k, const void* v, const void* g, const void* beta,
                        const int32_t* cu_seqlens, const float* initial_state, const void* saved,
                        size_t saved_bytes, const void* dO, const float* dS_final, void* dq, void* dk, void* dv, void* dg,
                        void* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                        void* stream);
kda_status kda_bwd_grads(const kda_config* cfg, int64_t total_tokens, int32_t num_seqs, const void* q,
                         const void* k, const void* v, const void* g, const void* beta,
                         const int32_t* cu_seqlens, const float* initial_state, const void* saved,
                         size_t saved_bytes, const void* dO, const float* dS_final, void* dq, void* dk, void* dv, void* dg,
                         void* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Decode step: one token per sequence on a resident state (serving).  For
 * every sequence n and head h it applies one step of the recurrence above to
 * the state entering the token and returns that token's output, reading and
 * writing the state once (the pages report KDA inside the serving frameworks
 * with prefill and decode run apart: "Moore Threads добавила поддержку Kimi
 * K3.1 Pro на GPU MTT S5000", lt.allworld.media 191952736, section
 * "Поддержка в фреймворках и новые возможности").  A run of calls over the
 * tokens of a sequence equals kda_fwd on that sequence up to rounding.
 *   q, k, g : [num_seqs, H, dk]   v : [num_seqs, H, dv]   beta : [num_seqs, H]
 *             (in_dtype; one token per sequence; beta is the logit)
 *   state_in  : fp32 [num_seqs, H, dk, dv], or NULL for the zero state
 *   state_out : fp32 [num_seqs, H, dk, dv], the state after the token; it may
 *               be state_in itself (in-place update) but must not otherwise
 *               overlap it (KDA_ERR_INVALID_ARG)
 *   o         : [num_seqs, H, dv] in out_dtype
 * cfg->chunk and cfg->flags are checked as for kda_fwd but not used; fp32
 * inputs are supported for dk = 64 and 128.  num_seqs = 0 enqueues nothing. */
kda_status kda_decode(const kda_config* cfg, int32_t num_seqs, const void* q, const void* k, const void* v,
                      const void* g, const void* beta, const float* state_in, float* state_out, void* o,
                      void* stream);

/* Static description of a status code. */
const char* kda_status_string(kda_status s);
/* Thread-local description of the last failure on this thread ("" if none). */
const char* kda_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
