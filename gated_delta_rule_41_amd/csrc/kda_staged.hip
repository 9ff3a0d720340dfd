// kda_staged.hip -- the staged forward (KDA_FLAG_STAGED): the correctness path
// that writes every intermediate of the chunk form out, so that a parity
// failure of the fused kernels can be traced to a stage.
//
// The chunk form follows the intra-chunk processing plus inter-chunk state
// passing that the pages describe ("TorchTitan Ascend open source: Kimi K3.1
// Pro adaptation and training practice", section "KDA pre/post-processing
// fusion"; "Ascend implements LoRA training of Kimi K3.1 Pro", section "KDA:
// big fused forward and backward").  Per (document, head) and chunk of C rows
// (C = 64, or 16 or 32 for chunk-size invariance checks; fewer rows at a
// document's end), with G the in-chunk inclusive cumsum of g
// and E_rs = exp(G_r - G_s) per channel (s <= r, so E <= 1 for g <= 0):
//
//   Akk[r,s] = beta_r sum_c kh_r kh_s E_rs (s < r)    Aqk[r,s] = sum_c qh_r kh_s E_rs (s <= r)
//   T = (I + Akk)^-1       W = T (beta kh exp(G))      Ut = T (beta v)
//   U = Ut - W S           O = (qh exp(G)) S + Aqk U
//   S <- Diag(exp(G_C)) S + Ktil^T U,   Ktil_r = kh_r exp(G_C - G_r)
//
// Two launches: kda_staged_intra_kernel, one workgroup per (chunk slot, head),
// everything that does not depend on the state (G, norms, Akk, Aqk, T, W, Ut
// and the scan's operands exp(G) qh, Ktil, exp(G_C)); then
// kda_staged_scan_kernel, one workgroup per (document, head, 64 value
// columns), the state in LDS, walking the chunks in order (U, O, S).  Plain
// fp32 FMA throughout (no matrix cores) with every pair decay formed
// directly, so the path holds for any g <= 0.  Not tuned: it exists to be
// compared stage by stage with a chunked reference.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace staged {

constexpr int PR = 128 + 1;        // row stride of the [C][<= 128] fp32 tiles (odd: rows spread over banks)

// The document that owns chunk slot `slot` for chunk length C (slots as in
// the fused kernels: floor(start / C) + document + chunk index).
__device__ __forceinline__ int owner(const int32_t* cu, int N, int seqlen, int64_t slot, int C) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int64_t start = cu ? (int64_t)cu[mid] : (int64_t)mid * seqlen;
        if (start / C + mid <= slot) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <typename T, int DK, int C>
__global__ __launch_bounds__(kThreads) void kda_staged_intra_kernel(StagedParams p) {
    constexpr int PA = C + 1;          // row stride of the [C][C] tiles
    constexpr int TPR = kThreads / C;  // threads per row for the norms (4, 8 or 16)
    __shared__ float bufG[C * PR];     // G
    __shared__ float bufK[C * PR];     // kh, later beta v
    __shared__ float bufQ[C * PR];     // qh, later beta kh exp(G)
    __shared__ float sA[C * PA];       // Akk
    __shared__ float sT[C * PA];       // T
    __shared__ float sbeta[C];
    const int tid = threadIdx.x;
    const int H = p.H, dv = p.dv;
    const int64_t slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int n = owner(p.cu, p.N, p.seqlen, slot, C);
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int64_t jc = slot - (t0 / C + n);
    const int64_t c0 = t0 + jc * C;
    if (jc < 0 || c0 >= t1) return;   // unused slot (uniform across the workgroup)
    const int L = (int)((t1 - c0) < C ? (t1 - c0) : C);
    const int64_t rsk = (int64_t)H * DK, rsv = (int64_t)H * dv;
    const T* qc = reinterpret_cast<const T*>(p.q) + c0 * rsk + (int64_t)h * DK;
    const T* kc = reinterpret_cast<const T*>(p.k) + c0 * rsk + (int64_t)h * DK;
    const T* gc = reinterpret_cast<const T*>(p.g) + c0 * rsk + (int64_t)h * DK;
    const T* vc = reinterpret_cast<const T*>(p.v) + c0 * rsv + (int64_t)h * dv;
    const T* bc = reinterpret_cast<const T*>(p.b) + c0 * H + h;
    const int64_t bi = slot * H + h;
    float* stG = p.G + bi * C * DK;
    float* stAkk = p.Akk + bi * C * C;
    float* stAqk = p.Aqk + bi * C * C;
    float* stT = p.Tm + bi * C * C;
    float* stW = p.W + bi * C * DK;
    float* stUt = p.Ut + bi * C * dv;
    float* stQG = p.QG + bi * C * DK;
    float* stKt = p.Ktil + bi * C * DK;
    float* stGC = p.GamC + bi * DK;

    // G: one thread per channel walks the rows (rows past the end add g = 0)
    if (tid < DK) {
        float a = 0.f;
        for (int r = 0; r < C; ++r) {
            a += r < L ? to_f32(gc[r * rsk + tid]) : 0.f;
            bufG[r * PR + tid] = a;
        }
    }
    // the L2 norms: TPR adjacent threads per row
    {
        const int r = tid / TPR, part = tid % TPR;
        float sq = 0.f, sk = 0.f;
        for (int c = part; c < DK; c += TPR) {
            const float qv = r < L ? to_f32(qc[r * rsk + c]) : 0.f;
            const float kv = r < L ? to_f32(kc[r * rsk + c]) : 0.f;
            sq += qv * qv;
            sk += kv * kv;
            bufQ[r * PR + c] = qv;
            bufK[r * PR + c] = kv;
        }
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) {
            sq += __shfl_xor(sq, m);
            sk += __shfl_xor(sk, m);
        }
        const float iq = p.scale / sqrtf(sq + p.eps), ik = 1.f / sqrtf(sk + p.eps);
        for (int c = part; c < DK; c += TPR) {
            bufQ[r * PR + c] *= iq;
            bufK[r * PR + c] *= ik;
        }
        if (part == 0) sbeta[r] = r < L ? 1.f / (1.f + expf(-to_f32(bc[(int64_t)r * H]))) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < C * DK; e += kThreads) {
        const int r = e / DK, c = e % DK;
        stG[e] = r < L ? bufG[r * PR + c] : 0.f;
    }
    // Akk and Aqk with the decay of every token pair
    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, s = e % C;
        float akk = 0.f, aqk = 0.f;
        if (s <= r && r < L) {
            for (int c = 0; c < DK; ++c) {
                const float ks = bufK[s * PR + c] * expf(bufG[r * PR + c] - bufG[s * PR + c]);
                akk += bufK[r * PR + c] * ks;
                aqk += bufQ[r * PR + c] * ks;
            }
        }
        akk = s < r ? sbeta[r] * akk : 0.f;
        sA[r * PA + s] = akk;
        stAkk[e] = akk;
        stAqk[e] = aqk;
    }
    __syncthreads();
    // T = (I + Akk)^-1: thread j owns column j (forward substitution down it)
    if (tid < C) {
        const int j = tid;
        for (int r = 0; r < C; ++r) {
            float t = r == j ? 1.f : 0.f;
            for (int s = j; s < r; ++s) t -= sA[r * PA + s] * sT[s * PA + j];
            sT[r * PA + j] = t;
        }
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += kThreads) {
        const int r = e / C, s = e % C;
        stT[e] = r < L ? sT[r * PA + s] : 0.f;
    }
    // the scan's operands; beta kh exp(G) replaces qh
    for (int e = tid; e < C * DK; e += kThreads) {
        const int r = e / DK, c = e % DK;
        const float gr = bufG[r * PR + c], eg = expf(gr);
        const float kh = bufK[r * PR + c];
        stQG[e] = r < L ? bufQ[r * PR + c] * eg : 0.f;
        stKt[e] = r < L ? kh * expf(bufG[(C - 1) * PR + c] - gr) : 0.f;
        bufQ[r * PR + c] = sbeta[r] * kh * eg;
    }
    if (tid < DK) stGC[tid] = expf(bufG[(C - 1) * PR + tid]);
    __syncthreads();
    // W = T (beta kh exp(G)); beta v replaces kh
    for (int e = tid; e < C * DK; e += kThreads) {
        const int r = e / DK, c = e % DK;
        float acc = 0.f;
        for (int s = 0; s <= r; ++s) acc += sT[r * PA + s] * bufQ[s * PR + c];
        stW[e] = r < L ? acc : 0.f;
    }
    for (int e = tid; e < C * dv; e += kThreads) {
        const int r = e / dv, j = e % dv;
        bufK[r * PR + j] = r < L ? sbeta[r] * to_f32(vc[r * rsv + j]) : 0.f;
    }
    __syncthreads();
    // Ut = T (beta v)
    for (int e = tid; e < C * dv; e += kThreads) {
        const int r = e / dv, j = e % dv;
        float acc = 0.f;
        for (int s = 0; s <= r; ++s) acc += sT[r * PA + s] * bufK[s * PR + j];
        stUt[e] = r < L ? acc : 0.f;
    }
}

template <typename TO, int DK, int C>
__global__ __launch_bounds__(kThreads) void kda_staged_scan_kernel(StagedParams p) {
    constexpr int SW = kSlice, PS = SW + 1;
    __shared__ float sS[DK * PS];   // this slice of the state [c][j]
    __shared__ float sU[C * PS];    // U of the chunk [r][j]
    const int tid = threadIdx.x;
    const int H = p.H, dv = p.dv, nsl = dv / SW;
    const int chain = blockIdx.x / nsl, slice = blockIdx.x % nsl;
    const int n = chain / H, h = chain % H;
    const int j0 = slice * SW;
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int nch = (int)((t1 - t0 + C - 1) / C);
    const int64_t sb = ((int64_t)n * H + h) * DK * dv;
    for (int e = tid; e < DK * SW; e += kThreads) {
        const int c = e / SW, j = e % SW;
        sS[c * PS + j] = p.s0 ? p.s0[sb + (int64_t)c * dv + j0 + j] : 0.f;
    }
    __syncthreads();
    TO* op = reinterpret_cast<TO*>(p.o);
    for (int ic = 0; ic < nch; ++ic) {
        const int64_t c0 = t0 + (int64_t)ic * C;
        const int L = (int)((t1 - c0) < C ? (t1 - c0) : C);
        const int64_t bi = (t0 / C + n + ic) * H + h;
        const float* W = p.W + bi * C * DK;
        const float* QG = p.QG + bi * C * DK;
        const float* Kt = p.Ktil + bi * C * DK;
        const float* GC = p.GamC + bi * DK;
        const float* Aqk = p.Aqk + bi * C * C;
        const float* Ut = p.Ut + bi * C * dv;
        float* U = p.U + bi * C * dv;
        float* Sin = p.Sin + bi * DK * dv;
        for (int e = tid; e < DK * SW; e += kThreads) {
            const int c = e / SW, j = e % SW;
            Sin[(int64_t)c * dv + j0 + j] = sS[c * PS + j];
        }
        // U = Ut - W S
        for (int e = tid; e < C * SW; e += kThreads) {
            const int r = e / SW, j = e % SW;
            float acc = Ut[r * dv + j0 + j];
            for (int c = 0; c < DK; ++c) acc -= W[r * DK + c] * sS[c * PS + j];
            const float u = r < L ? acc : 0.f;
            sU[r * PS + j] = u;
            U[r * dv + j0 + j] = u;
        }
        __syncthreads();
        // O = (qh exp(G)) S + Aqk U
        for (int e = tid; e < C * SW; e += kThreads) {
            const int r = e / SW, j = e % SW;
            if (r < L) {
                float acc = 0.f;
                for (int c = 0; c < DK; ++c) acc += QG[r * DK + c] * sS[c * PS + j];
                for (int s = 0; s <= r; ++s) acc += Aqk[r * C + s] * sU[s * PS + j];
                op[(c0 + r) * H * (int64_t)dv + (int64_t)h * dv + j0 + j] = from_f32<TO>(acc);
            }
        }
        __syncthreads();
        // S <- Diag(exp(G_C)) S + Ktil^T U (each element read and written by one thread)
        for (int e = tid; e < DK * SW; e += kThreads) {
            const int c = e / SW, j = e % SW;
            float acc = GC[c] * sS[c * PS + j];
            for (int s = 0; s < L; ++s) acc += Kt[s * DK + c] * sU[s * PS + j];
            sS[c * PS + j] = acc;
        }
        __syncthreads();
    }
    if (p.sfinal) {
        for (int e = tid; e < DK * SW; e += kThreads) {
            const int c = e / SW, j = e % SW;
            p.sfinal[sb + (int64_t)c * dv + j0 + j] = sS[c * PS + j];
        }
    }
}

template <typename T, typename TO, int DK, int C>
hipError_t launch_c(const StagedParams& p, hipStream_t s) {
    const int64_t intra = (p.T / C + p.N) * p.H;   // chunk slots x heads
    const int64_t scan = (int64_t)p.N * p.H * (p.dv / kSlice);
    if (intra > 0)
        hipLaunchKernelGGL((kda_staged_intra_kernel<T, DK, C>), dim3((unsigned)intra), dim3(kThreads), 0, s, p);
    if (scan > 0)
        hipLaunchKernelGGL((kda_staged_scan_kernel<TO, DK, C>), dim3((unsigned)scan), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T, typename TO, int DK>
hipError_t launch_typed(const StagedParams& p, int chunk, hipStream_t s) {
    if (chunk == 16) return launch_c<T, TO, DK, 16>(p, s);
    if (chunk == 32) return launch_c<T, TO, DK, 32>(p, s);
    return launch_c<T, TO, DK, 64>(p, s);
}

}  // namespace staged

hipError_t launch_fwd_staged(const StagedParams& p, int in_dtype, int out_dtype, int dk, int chunk, hipStream_t s) {
    const bool bin = in_dtype != 0, bout = out_dtype != 0;
    if (dk == 128) {
        if (bin) return bout ? staged::launch_typed<bf16, bf16, 128>(p, chunk, s) : staged::launch_typed<bf16, float, 128>(p, chunk, s);
        return bout ? staged::launch_typed<float, bf16, 128>(p, chunk, s) : staged::launch_typed<float, float, 128>(p, chunk, s);
    }
    if (bin) return bout ? staged::launch_typed<bf16, bf16, 64>(p, chunk, s) : staged::launch_typed<bf16, float, 64>(p, chunk, s);
    return bout ? staged::launch_typed<float, bf16, 64>(p, chunk, s) : staged::launch_typed<float, float, 64>(p, chunk, s);
}

}  // namespace kda
