// kda_decode.hip -- one-token KDA step on a resident state, for serving.
//
// In decoding the KDA layers carry their per-head state from token to token
// and each new token costs one recurrent update (the pages report KDA support
// inside the serving frameworks and prefill/decode-separated deployments:
// "Moore Threads добавила поддержку Kimi K3.1 Pro на GPU MTT S5000", section
// "Поддержка в фреймворках и новые возможности", the Huawei Ascend inference
// adaptation).  For one token of one (sequence, head), with S the dk x dv fp32
// state entering the token:
//
//     S' = Diag(alpha) S                       alpha = exp(g)
//     p  = S'^T kh,   r = S'^T qh              (two reductions over dk)
//     u  = beta (v - p)
//     S  <- S' + kh u^T                        (the delta-rule write)
//     o  = S^T qh = r + (kh . qh) u
//
// which is the recurrence of the forward taken one token at a time.  The step
// reads and writes the state once and touches a few hundred bytes of token
// inputs, so it is bound by HBM traffic on the state: 2 * dk * dv * 4 bytes per
// (sequence, head).  No matrix unit is involved: two column reductions and a
// rank-1 update are vector work.
//
// One workgroup (4 waves) per (sequence, head, 64-wide value slice).  Thread
// (tr, tc), tr = tid / 16, tc = tid % 16, holds state rows tr + 16 j
// (j < dk / 16) and value columns 4 tc .. 4 tc + 3 of the slice in registers:
// the loads of a wave cover four 256-byte row segments.  All state loads are
// issued first; the token's norms and gates are computed while they are in
// flight.  The state is streamed (each byte read once and written once per
// step), so its loads and stores are nontemporal: they do not displace other
// data from the caches.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__device__ __forceinline__ float wave_sum(float v) {
    // butterfly over the 64 lanes: every lane ends with the same bits
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <typename T, typename TO, int DK>
__global__ __launch_bounds__(kThreads) void kda_decode_kernel(DecodeParams p) {
    constexpr int RPT = DK / 16;            // state rows per thread
    __shared__ float sqh[DK], skh[DK], sal[DK];
    __shared__ float spart[3][4];           // per-wave partial sums: |q|^2, |k|^2, q.k
    __shared__ f32x4 sred[2][4][16];        // per-wave partial p and r, per column group

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int tc = tid & 15, tr = tid >> 4;
    const int nh = blockIdx.x / p.nslices, slice = blockIdx.x % p.nslices;
    const int dv = p.dv;
    const int col = slice * kSlice + 4 * tc;
    const int64_t sbase = (int64_t)nh * DK * dv + col;

    f32x4 s[RPT];
    if (p.s_in) {
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            s[j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(p.s_in + sbase + (int64_t)(tr + 16 * j) * dv));
    } else {
#pragma unroll
        for (int j = 0; j < RPT; ++j) s[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const T* qp = reinterpret_cast<const T*>(p.q) + (int64_t)nh * DK;
    const T* kp = reinterpret_cast<const T*>(p.k) + (int64_t)nh * DK;
    const T* gp = reinterpret_cast<const T*>(p.g) + (int64_t)nh * DK;
    const T* vp = reinterpret_cast<const T*>(p.v) + (int64_t)nh * dv + col;
    const float b = to_f32(reinterpret_cast<const T*>(p.b)[nh]);
    float vv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(vp[e]);

    float qx = 0.f, kx = 0.f;
    if (tid < DK) {
        qx = to_f32(qp[tid]);
        kx = to_f32(kp[tid]);
        sal[tid] = __expf(to_f32(gp[tid]));
    }
    {
        const float a = wave_sum(qx * qx), c = wave_sum(kx * kx), d = wave_sum(qx * kx);
        if (l == 0) { spart[0][w] = a; spart[1][w] = c; spart[2][w] = d; }
    }
    __syncthreads();
    float sumq = 0.f, sumk = 0.f, sumqk = 0.f;
#pragma unroll
    for (int i = 0; i < DK / 64; ++i) { sumq += spart[0][i]; sumk += spart[1][i]; sumqk += spart[2][i]; }
    const float rq = p.scale / sqrtf(sumq + p.eps), rk = 1.f / sqrtf(sumk + p.eps);
    const float kq = sumqk * rq * rk;                      // kh . qh
    const float beta = 1.f / (1.f + __expf(-b));
    if (tid < DK) { sqh[tid] = qx * rq; skh[tid] = kx * rk; }
    __syncthreads();

    // S' = Diag(alpha) S and this thread's share of the two reductions
    f32x4 pp = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i = tr + 16 * j;
        s[j] *= sal[i];
        pp += skh[i] * s[j];
        rr += sqh[i] * s[j];
    }
    // lanes tc, tc+16, tc+32, tc+48 of a wave share the column group
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pp[e] += __shfl_xor(pp[e], 16, 64);
        pp[e] += __shfl_xor(pp[e], 32, 64);
        rr[e] += __shfl_xor(rr[e], 16, 64);
        rr[e] += __shfl_xor(rr[e], 32, 64);
    }
    if (l < 16) { sred[0][w][tc] = pp; sred[1][w][tc] = rr; }
    __syncthreads();
    f32x4 pc = sred[0][0][tc], rc = sred[1][0][tc];
#pragma unroll
    for (int i = 1; i < 4; ++i) { pc += sred[0][i][tc]; rc += sred[1][i][tc]; }

    f32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = beta * (vv[e] - pc[e]);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i = tr + 16 * j;
        s[j] += skh[i] * u;
        __builtin_nontemporal_store(s[j], reinterpret_cast<f32x4*>(p.s_out + sbase + (int64_t)i * dv));
    }
    if (tr == 0) {
        TO* op = reinterpret_cast<TO*>(p.o) + (int64_t)nh * dv + col;
#pragma unroll
        for (int e = 0; e < 4; ++e) op[e] = from_f32<TO>(rc[e] + kq * u[e]);
    }
}

template <typename T, typename TO>
static hipError_t launch_decode_t(const DecodeParams& p, int dk, hipStream_t stream) {
    const int blocks = p.N * p.H * p.nslices;
    if (blocks == 0) return hipSuccess;
    if (dk == 128)
        hipLaunchKernelGGL((kda_decode_kernel<T, TO, 128>), dim3(blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_decode_kernel<T, TO, 64>), dim3(blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, int in_dtype, int out_dtype, int dk, hipStream_t stream) {
    if (in_dtype == 1)
        return out_dtype == 1 ? launch_decode_t<bf16, bf16>(p, dk, stream) : launch_decode_t<bf16, float>(p, dk, stream);
    return out_dtype == 1 ? launch_decode_t<float, bf16>(p, dk, stream) : launch_decode_t<float, float>(p, dk, stream);
}

}  // namespace kda
