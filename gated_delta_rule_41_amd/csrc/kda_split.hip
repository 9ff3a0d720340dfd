// kda_split.hip -- the two-level forward for long sequences (bf16 inputs).
//
// A chain (sequence, head) is sequential over its chunks, so a few long
// sequences leave most compute units idle.  The map of one chunk on the state
// is affine, S_out = M S_in + B, with M = Diag(Gam_C) - Ktil^T W and
// B = Ktil^T Ut in the notation of the chunked form, and so is the map of any
// run of chunks.  The pages spread the KDA recurrence over many compute units
// and hide its dependency latency by pipelining ("Large models on Ascend: from
// adaptation challenges to efficient training", section 2, the compute side),
// and list context parallelism among the supported parallel modes
// ("TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
// practice", section "Kimi K3.1 Pro Ascend training adaptation"); splitting a
// long sequence into segments whose maps are composed is the single-GPU form of
// both.  On one GPU:
//
//   1. split every document into segments of seg_len tokens (a multiple of the
//      chunk), on the device, from cu_seqlens       (kda_segments_kernel)
//   2. every segment's [M | B] from the zero state: the fused forward kernel
//      in its map mode, all segments in parallel     (kda_fwd.hip)
//   3. per document, the state entering every segment: S_0 = initial state,
//      S_{j+1} = M_j S_j + B_j, in fp32              (kda_carry_kernel)
//   4. the fused forward over the segments, each from its entering state,
//      writing o and, for the last segment of a document, its final state
//
// Steps 2 and 4 each fill the GPU; step 3 is dk x dk x dv fp32 work per
// segment.  The chunk boundaries are those of the one-pass forward, so the
// result differs from it only by rounding.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// One workgroup: per-document segment counts max(1, ceil(len / seg_len)),
// their exclusive prefix sum (doc_seg), and the segment bounds.
__global__ __launch_bounds__(kThreads) void kda_segments_kernel(SegParams p) {
    __shared__ int32_t wsum[kThreads / 64];
    __shared__ int32_t carry;
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < p.N; base += kThreads) {
        const int n = base + tid;
        int64_t a = 0, z = 0;
        int cnt = 0;
        if (n < p.N) {
            seq_bounds(p.cu, n, p.seqlen, p.T, a, z);
            const int64_t len = z - a;
            cnt = len > 0 ? (int)((len + p.seg_len - 1) / p.seg_len) : 1;
        }
        // inclusive scan of cnt over the workgroup
        int x = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (l >= d) x += y;
        }
        if (l == 63) wsum[w] = x;
        __syncthreads();
        int off = carry;
        for (int i = 0; i < w; ++i) off += wsum[i];
        const int first = off + x - cnt;
        if (n < p.N) {
            p.doc_seg[n] = first;
            for (int s = 0; s < cnt; ++s) {
                const int j = first + s;
                if (j < p.P) {
                    const int64_t sa = a + (int64_t)s * p.seg_len;
                    p.seg_cu[j] = (int32_t)sa;
                    p.sf_dst[j] = s == cnt - 1 ? n : -1;
                }
            }
        }
        __syncthreads();
        if (tid == kThreads - 1) carry = off + x;
        __syncthreads();
    }
    const int used = carry < p.P ? carry : p.P;
    if (tid == 0) p.doc_seg[p.N] = used;
    // the end of every used segment is the start of the next; unused ones are empty at T
    for (int j = used + tid; j <= p.P; j += kThreads) {
        p.seg_cu[j] = (int32_t)p.T;
        if (j < p.P) p.sf_dst[j] = -1;
    }
}

hipError_t launch_segments(const SegParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(kda_segments_kernel, dim3(1), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// One workgroup per (document, head, 16-wide value slice): walks the
// document's segments in order, writing the state entering each and applying
// S <- M S + B.  The slice of S (dk x 16) and M (dk x dk) sit in LDS; thread
// (r, c) computes row r = tid / TPR, columns c*CPT .. c*CPT + CPT - 1.  Narrow
// slices put dv/16 workgroups on every (document, head), so that the few
// sequential chains of a long-context call spread over more compute units.
template <int DK>
__global__ __launch_bounds__(kThreads) void kda_carry_kernel(CarryParams p) {
    constexpr int TPR = kThreads / DK;     // threads per state row (2 or 4)
    constexpr int CPT = kCarryCols / TPR;  // columns per thread (8 or 4)
    constexpr int PM = DK + 4;             // padded row stride of M in LDS (16-byte rows)
    __shared__ float sS[DK][kCarryCols];
    __shared__ __attribute__((aligned(16))) float sM[DK][PM];
    const int tid = threadIdx.x;
    const int nh = blockIdx.x / p.nslices, slice = blockIdx.x % p.nslices;
    const int n = nh / p.H, h = nh % p.H;
    const int dv = p.dv, ldm = DK + dv;
    const int r = tid / TPR, c0 = (tid % TPR) * CPT;
    const int col = slice * kCarryCols + c0;    // value column of the thread's first output
    const int j0 = p.doc_seg[n], j1 = p.doc_seg[n + 1];

    float x[CPT];
    const float* s0 = p.s0 ? p.s0 + ((int64_t)n * p.H + h) * DK * dv + (int64_t)r * dv + col : nullptr;
#pragma unroll
    for (int c = 0; c < CPT; ++c) x[c] = s0 ? s0[c] : 0.f;
    for (int j = j0; j < j1; ++j) {
        float* si = p.s_in + ((int64_t)j * p.H + h) * DK * dv + (int64_t)r * dv + col;
#pragma unroll
        for (int c = 0; c < CPT; c += 4) *reinterpret_cast<f32x4*>(si + c) = f32x4{x[c], x[c + 1], x[c + 2], x[c + 3]};
        if (j + 1 == j1) break;   // the last segment's own map is not needed
        const float* mp = p.maps + ((int64_t)j * p.H + h) * DK * ldm;
#pragma unroll
        for (int c = 0; c < CPT; ++c) sS[r][c0 + c] = x[c];
        for (int e = tid; e < DK * DK / 4; e += kThreads) {
            const int rr = e / (DK / 4), cc = 4 * (e % (DK / 4));
            *reinterpret_cast<f32x4*>(&sM[rr][cc]) = *reinterpret_cast<const f32x4*>(mp + (int64_t)rr * ldm + cc);
        }
        const float* bp = mp + (int64_t)r * ldm + DK + col;
#pragma unroll
        for (int c = 0; c < CPT; c += 4) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(bp + c);
            x[c] = b[0]; x[c + 1] = b[1]; x[c + 2] = b[2]; x[c + 3] = b[3];
        }
        __syncthreads();
        for (int k = 0; k < DK; ++k) {
            const float m = sM[r][k];
#pragma unroll
            for (int c = 0; c < CPT; ++c) x[c] = fmaf(m, sS[k][c0 + c], x[c]);
        }
        __syncthreads();
    }
}

hipError_t launch_carry(const CarryParams& p, int dk, hipStream_t stream) {
    const int blocks = p.N * p.H * p.nslices;
    if (blocks == 0) return hipSuccess;
    if (dk == 128)
        hipLaunchKernelGGL(kda_carry_kernel<128>, dim3(blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(kda_carry_kernel<64>, dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda
