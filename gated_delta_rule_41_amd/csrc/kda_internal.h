// kda_internal.h -- host-side interface between the C ABI (kda_api.hip) and
// the kernel launchers.  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;      // tokens per chunk
constexpr int kSlice = 64;      // value columns per forward / reverse-scan workgroup
constexpr int kCarryCols = 16;  // value columns per segment-carry workgroup
constexpr int kThreads = 256;   // 4 wave64 per workgroup
constexpr int kWideThreads = 512;   // 8 wave64: four state waves + four prep waves (bf16 kernels)

// Transposed operand tile [row c][64 chunk positions] without padding, each
// 16-byte group XOR-swizzled with (c ^ c>>3) & 7, so that A-fragment reads (16
// consecutive rows) and writes from the prep layout (rows 8 apart) spread over
// the LDS banks.  `pos` is the position inside the row (perm32 order).
__device__ __forceinline__ int kt_off(int c, int pos) {
    return c * kChunk + ((((pos >> 3) ^ (c ^ (c >> 3))) & 7) << 3) + (pos & 7);
}

// kt_off of the A fragments a lane (qg, cl) reads: row 16m + cl, positions
// 32kk + 8qg..+7, for compile-time m (0..7) and kk (0..1).  The swizzle group is
// g0 ^ ((4kk ^ 2m) & 7) with g0 = (qg ^ cl ^ (cl >> 3)) & 7 a lane constant, so
// four lane values and an immediate row offset cover every (m, kk).
struct KtFrag {
    int b[4];   // b[x] = 64 cl + ((g0 ^ 2x) << 3)
    __device__ __forceinline__ KtFrag(int qg, int cl) {
        const int g0 = (qg ^ cl ^ (cl >> 3)) & 7;
#pragma unroll
        for (int x = 0; x < 4; ++x) b[x] = kChunk * cl + ((g0 ^ (2 * x)) << 3);
    }
    __device__ __forceinline__ int at(int m, int kk) const { return b[(((4 * kk) ^ (2 * m)) & 7) >> 1] + 16 * kChunk * m; }
};

// Per-chunk state slots: chunk j of sequence n uses slot floor(cu[n]/64) + n + j.
// The map is collision-free and bounded by floor(T/64) + N (see kda_api.hip).
inline int64_t num_slots(int64_t T, int32_t N) { return T / kChunk + N; }

// The sequence that owns state slot `slot` (the inverse of the map above).
__device__ __forceinline__ int slot_owner(const int32_t* cu, int N, int seqlen, int64_t slot) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t start = cu ? (int64_t)cu[mid] : (int64_t)mid * seqlen;
        if (start / kChunk + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* b;
    const int32_t* cu;   // device [N+1] or nullptr (equal sequences of `seqlen`)
    const float* s0;     // [N,H,dk,dv] or nullptr
    void* o;             // [T,H,dv] out dtype
    float* sfinal;       // [N,H,dk,dv] or nullptr
    // Saves for the backward (or nullptr).  fp32 inputs: states fp32.  bf16
    // inputs: states and U in fp16, scaled by 2^-e per (slot, head, 16-column
    // group), with 2^e in sv_scale.
    void* st_saved;      // the state entering every chunk: fp32 [slots,H,dk,dv], or (bf16
                         // inputs) fp16 blocked by 16 value columns [slots,H,dv/16,dk,16]
    float* nq_saved;     // [H,T] (head-major) or nullptr
    float* nk_saved;     // [H,T] (head-major) or nullptr
    void* u_saved;       // [slots,H,64*dv] fp16 in fragment order (ufrag): U of every chunk (bf16 inputs)
    float* sv_scale;     // [slots,H,dv/16] fp32: 2^e of the saved state and U (bf16 inputs)
    const int32_t* sf_dst;   // per sequence: row of sfinal to write, or -1 to skip; nullptr = itself
    int64_t T;
    int32_t N, H, dv, seqlen;
    float eps, scale;
    int32_t nslices;     // dv / kSlice (segment maps: (dk + dv) / kSlice)
    int32_t map_slices;  // segment maps: the first dk / kSlice slices carry M, the rest B
};

// Segment split of long sequences for the two-level forward (bf16 inputs).
struct SegParams {
    const int32_t* cu;   // documents [N+1] (device) or nullptr: N equal sequences of seqlen
    int32_t* seg_cu;     // [P+1] segment token bounds; unused trailing segments are empty at T
    int32_t* doc_seg;    // [N+1] first segment of every document (doc_seg[N] = segments used)
    int32_t* sf_dst;     // [P] document whose final state segment j ends, or -1
    int64_t T;
    int32_t N, seqlen, seg_len, P;
};
struct CarryParams {
    const int32_t* doc_seg;
    const float* s0;     // [N,H,dk,dv] or nullptr
    const float* maps;   // [P,H,dk,dk+dv]: [M | B] of every segment
    float* s_in;         // [P,H,dk,dv]: the state entering every segment
    int32_t N, H, dv, nslices;   // nslices = dv / kCarryCols
};

// The staged forward (KDA_FLAG_STAGED): inputs as FwdParams, and the stage
// buffers it writes, all fp32, indexed by (slot * H + head), C the chunk:
//   G, W, QG, Ktil [., C, dk]    Akk, Aqk, Tm [., C, C]      Ut, U [., C, dv]
//   Sin [., dk, dv]              GamC [., dk]
struct StagedParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* b;
    const int32_t* cu;
    const float* s0;
    void* o;
    float* sfinal;
    float *G, *Akk, *Aqk, *Tm, *W, *Ut, *U, *Sin, *QG, *Ktil, *GamC;
    int64_t T;
    int32_t N, H, dv, seqlen;
    float eps, scale;
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* b;
    const int32_t* cu;
    const void* st_saved;    // forward-entering state of every chunk (format as in FwdParams)
    const float* nq_saved;
    const float* nk_saved;
    const void* dO;          // [T,H,dv] in dtype
    const float* dS_final;   // [N,H,dk,dv] or nullptr
    void* dst_saved;         // workspace: dL/dS at the END of every chunk (layout of st_saved)
                             // (fp32 for fp32 inputs; fp16 scaled by ds_scale for bf16 inputs)
    const void* u_saved;     // forward's U of every chunk [slots,H,64*dv] fp16, fragment order (bf16 inputs)
    void* du_ws;             // workspace: dU of every chunk, the same layout (bf16 inputs)
    const float* sv_scale;   // [slots,H,dv/16]: 2^e of the saved state and U (bf16 inputs)
    float* ds_scale;         // workspace [slots,H,dv/16]: 2^e of dS1 and dU (bf16 inputs)
    int32_t* chunk_flags;    // workspace [slots,H]: 1 where the chunk's decay passes the factorised
                             // range (written by the reverse scan, read by the pair-exact kernel)
    void* dq;
    void* dk;
    void* dv_out;
    void* dg;
    void* db;
    float* dS0;              // [N,H,dk,dv] or nullptr
    int64_t T;
    int32_t N, H, dv, seqlen;
    float eps, scale;
    int32_t nslices;
};

struct DecodeParams {
    const void* q;       // [N,H,dk] one token per sequence
    const void* k;
    const void* v;       // [N,H,dv]
    const void* g;
    const void* b;       // [N,H]
    const float* s_in;   // [N,H,dk,dv] or nullptr (zero state)
    float* s_out;        // [N,H,dk,dv]; may equal s_in
    void* o;             // [N,H,dv] out dtype
    int32_t N, H, dv;
    float eps, scale;
    int32_t nslices;     // dv / kSlice
};

// in_dtype / out_dtype: 0 = fp32, 1 = bf16 (kda_dtype values).
hipError_t launch_fwd(const FwdParams& p, int in_dtype, int out_dtype, int dk, bool save,
                      hipStream_t stream);
// Backward stages (bit mask): the reverse state scan, then the chunk-parallel gradients.
constexpr int kBwdScan = 1, kBwdGrads = 2;
hipError_t launch_bwd(const BwdParams& p, int in_dtype, int out_dtype, int dk, int stages, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int in_dtype, int out_dtype, int dk, hipStream_t stream);
// Two-level forward pieces (bf16 inputs): segment split, segment maps, carry scan.
hipError_t launch_segments(const SegParams& p, hipStream_t stream);
hipError_t launch_fwd_maps(const FwdParams& p, int dk, hipStream_t stream);
// bf16 inputs: the fused forward with fp16 matrix-core operands (kda_fwd16.hip).
hipError_t launch_fwd16(const FwdParams& p, int out_dtype, int dk, bool save, hipStream_t stream);
hipError_t launch_fwd16_maps(const FwdParams& p, int dk, hipStream_t stream);
// bf16 inputs: the reverse state-gradient scan with fp16 matrix-core operands (kda_scan16.hip).
hipError_t launch_scan16(const BwdParams& p, int dk, hipStream_t stream);
hipError_t launch_carry(const CarryParams& p, int dk, hipStream_t stream);
hipError_t launch_fwd_staged(const StagedParams& p, int in_dtype, int out_dtype, int dk, int chunk, hipStream_t stream);
// Kernels without the chunk-start gate factorisation (kda_exact.hip): the
// forward and the reverse scan token by token, and the chunk gradients with
// the decay of every token pair formed directly (only_unsafe: only chunks whose
// decay passes the factorised kernels' range; the others are left as they are).
hipError_t launch_fwd_token(const FwdParams& p, int in_dtype, int out_dtype, int dk, bool save, hipStream_t stream);
hipError_t launch_bwd_scan_token(const BwdParams& p, int in_dtype, int dk, hipStream_t stream);
hipError_t launch_bwd_exact(const BwdParams& p, int in_dtype, int out_dtype, int dk, bool only_unsafe,
                            hipStream_t stream);

}  // namespace kda
