// kda_exact.hip -- KDA kernels that evaluate every gate decay without the
// chunk-start factorisation (see kda_token.h for why it is needed):
//
//   kda_fwd_token_kernel       forward, token by token (fp32 inputs at dk = 128)
//   kda_bwd_scan_token_kernel  reverse state-gradient scan, token by token
//                              (fp32 inputs at dk = 128)
//   kda_bwd_exact_kernel       chunk gradients with exp(G_r - G_s) formed for
//                              every token pair: every chunk for fp32 inputs at
//                              dk = 128; for the other configurations it runs
//                              after the factorised gradient kernel and rewrites
//                              the chunks whose decay passes kExactBelow.
//
// The chunk gradients follow the chunk form of the intra-chunk / inter-chunk
// organisation the pages describe ("TorchTitan Ascend open source: Kimi K3.1
// Pro adaptation and training practice", section "KDA pre/post-processing
// fusion"): with G the in-chunk cumulative sum of g, Gam = exp(G), E_rs =
// exp(G_r - G_s) per channel (r >= s, so E <= 1),
//
//   Akk[r,s] = beta_r sum_c kh_r kh_s E_rs  (s < r),  Aqk[r,s] = sum_c qh_r kh_s E_rs  (s <= r)
//   T = (I + Akk)^-1,  U = T (beta v - (beta kh Gam) S0),  O = (qh Gam) S0 + Aqk U
//   S1 = Diag(Gam_C) S0 + Ktil^T U,  Ktil_r = kh_r exp(G_C - G_r)
//
// and their reverse mode from S0 (saved by the forward) and dS1 = dL/dS1 (from
// the reverse scan).  Every factor that multiplies a key or query row is a
// decay between two tokens, at most 1, so nothing overflows for any g <= 0.
// The arithmetic is plain fp32 FMA (no matrix cores): this path is the
// correctness path for inputs outside the factorised kernels' range.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_token.h"

namespace kda {
namespace ex {

// ---------------------------------------------------------------- token forward
template <typename T, typename TO, int DK, bool SAVE>
__global__ __launch_bounds__(kThreads) void kda_fwd_token_kernel(FwdParams p) {
    constexpr int NMB = DK / 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, qg = l >> 4, cl = l & 15;
    int chain, slice;
    map_block(blockIdx.x, p.N * p.H, p.nslices, chain, slice);
    const int n = chain / p.H, h = chain % p.H;
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int dv = p.dv, H = p.H;
    const int col = slice * kSlice + 16 * w + cl;
    const TokSrc<T> src = {reinterpret_cast<const T*>(p.q), reinterpret_cast<const T*>(p.k),
                           reinterpret_cast<const T*>(p.g), reinterpret_cast<const T*>(p.b),
                           reinterpret_cast<const T*>(p.v), H, h, dv, col, qg, p.eps, p.scale};
    const int64_t sbase = ((int64_t)n * H + h) * DK * dv;
    f32x4 S[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mb][i] = p.s0 ? p.s0[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + col] : 0.f;
    TO* op = reinterpret_cast<TO*>(p.o);
    int64_t slot = t0 / kChunk + n;
    for (int64_t c0 = t0; c0 < t1; c0 += kChunk, ++slot) {
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);
        if (SAVE) {
            float* st = reinterpret_cast<float*>(p.st_saved) + (slot * H + h) * (int64_t)DK * dv;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[(int64_t)(16 * mb + 4 * qg + i) * dv + col] = S[mb][i];
        }
        token_fwd<T, TO, DK>(S, src, c0, L, op, SAVE ? p.nq_saved + (int64_t)h * p.T : nullptr,
                             SAVE ? p.nk_saved + (int64_t)h * p.T : nullptr, slice == 0 && tid == 0);
    }
    if (p.sfinal) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.sfinal[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + col] = S[mb][i];
    }
}

// ---------------------------------------------------------------- token reverse scan
template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void kda_bwd_scan_token_kernel(BwdParams p) {
    constexpr int NMB = DK / 16;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, qg = l >> 4, cl = l & 15;
    int chain, slice;
    map_block(blockIdx.x, p.N * p.H, p.nslices, chain, slice);
    const int n = chain / p.H, h = chain % p.H;
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int dv = p.dv, H = p.H;
    const int col = slice * kSlice + 16 * w + cl;
    const TokSrc<T> src = {reinterpret_cast<const T*>(p.q), reinterpret_cast<const T*>(p.k),
                           reinterpret_cast<const T*>(p.g), reinterpret_cast<const T*>(p.b),
                           reinterpret_cast<const T*>(p.dO), H, h, dv, col, qg, p.eps, p.scale};
    const int64_t sbase = ((int64_t)n * H + h) * DK * dv;
    f32x4 R[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            R[mb][i] = p.dS_final ? p.dS_final[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + col] : 0.f;
    float* dst = reinterpret_cast<float*>(p.dst_saved);
    const int64_t nchunks = (t1 - t0 + kChunk - 1) / kChunk;
    for (int64_t jc = nchunks - 1; jc >= 0; --jc) {
        const int64_t c0 = t0 + jc * kChunk;
        const int64_t slot = t0 / kChunk + n + jc;
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);
        float* out = dst + (slot * H + h) * (int64_t)DK * dv;   // dL/dS at the end of the chunk
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(int64_t)(16 * mb + 4 * qg + i) * dv + col] = R[mb][i];
        token_bwd<T, DK>(R, src, c0, L);
    }
    if (p.dS0) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.dS0[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + col] = R[mb][i];
    }
}

// ---------------------------------------------------------------- pair-exact chunk gradients
constexpr int kExactThreads = 512;

template <int DK>
struct ExactLds {
    static constexpr int PD = DK + 4;        // row stride of the [64][DK] tiles
    static constexpr int NRG = DK == 128 ? 16 : 32;   // row groups of the key-side tile
    float q[kChunk * PD];     // qh = scale q / |q|
    float k[kChunk * PD];     // kh = k / |k|
    float G[kChunk * PD];     // inclusive in-chunk cumulative sum of g (natural log)
    float T[kChunk * kChunk]; // Akk, then T = (I + Akk)^-1  ([r][s])
    // 8192 floats shared by phases: [Aqk | U quarter | dU quarter] during the
    // value quarters; dW [64][DK]; then [dT | Y] and [dAkk | dAqk]
    float R[8192];
    float beta[kChunk], nq[kChunk], nk[kChunk], db[kChunk];
    float gc[DK], dgc[DK];
    float red[NRG * DK];      // per row group: sum of dKtil * Ktil over its rows
    int list[kExactThreads];  // flagged items of the current round
    int nlist;
};

// One chunk (state slot `slot`, head h) of the pair-exact gradients.  Every
// thread of the workgroup calls it; it leaves through its end or through the
// uniform early return for an unused slot.
template <typename T, typename TO, int DK, int DV>
__device__ void exact_chunk(const BwdParams& p, ExactLds<DK>& sm, int64_t slot, int h) {
    typedef ExactLds<DK> LY;
    constexpr int PD = LY::PD;
    constexpr int C = kChunk;
    // key-side tile: rows rA .. rA + RA - 1, channels cA .. cA + 3
    constexpr int NCG = DK / 4;                     // channel groups of 4
    constexpr int RA = C * NCG / kExactThreads;     // 4 (dk 128) or 2 (dk 64)
    static_assert(C / RA == LY::NRG, "row groups");
    const int tid = threadIdx.x;
    const int rgA = tid / NCG, rA = RA * rgA, cA = 4 * (tid % NCG);
    // 64 x 64 tile: rows rB, rB + 1; columns sB .. sB + 3
    const int rB = 2 * (tid >> 4), sB = 4 * (tid & 15);
    // 64 x 32 value-quarter tile: row rQ, columns cQ .. cQ + 3
    const int rQ = tid >> 3, cQ = 4 * (tid & 7);

    const int H = p.H;
    const int n = slot_owner(p.cu, p.N, p.seqlen, slot);
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int64_t jc = slot - (t0 / kChunk + n);
    const int64_t c0 = t0 + jc * kChunk;
    if (jc < 0 || c0 >= t1) return;   // unused slot (uniform)
    const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);

    const T* __restrict__ qg_ = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kg_ = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ gg_ = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ vg_ = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ dog = reinterpret_cast<const T*>(p.dO);
    const T* __restrict__ bg_ = reinterpret_cast<const T*>(p.b);
    // S0 and dS1: fp32 for fp32 inputs; for bf16 inputs fp16 scaled by 2^-e per
    // 16-column group, with 2^e in sv_scale / ds_scale.  ld4 returns row c,
    // columns j .. j + 3 (j a multiple of 4, so one group).
    const int64_t sbase = (slot * H + h) * (int64_t)DK * DV;
    auto ld4 = [&](const void* base, const float* scale, int c, int j) -> f32x4 {
        if constexpr (std::is_same<T, bf16>::value) {
            typedef _Float16 h4v __attribute__((ext_vector_type(4)));
            // fp16 states are blocked by 16 value columns: [dv/16][dk][16]
            const h4v x = *reinterpret_cast<const h4v*>(reinterpret_cast<const _Float16*>(base) + sbase +
                                                        (int64_t)((j >> 4) * DK + c) * 16 + (j & 15));
            return __builtin_convertvector(x, f32x4) * scale[(slot * H + h) * (DV / 16) + (j >> 4)];
        } else {
            (void)scale;
            return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + sbase + (int64_t)c * DV + j);
        }
    };
    auto ldS0 = [&](int c, int j) { return ld4(p.st_saved, p.sv_scale, c, j); };
    auto ldS1 = [&](int c, int j) { return ld4(p.dst_saved, p.ds_scale, c, j); };
    auto krow = [&](int r) { return (c0 + r) * H + h; };   // token-row index into [T, H]

    // ================= phase 0: rows, norms, gate sums =================
    {
        constexpr int CP = DK / 8;
        const int r = tid >> 3, part = tid & 7, c_0 = CP * part;
        float qv[CP], kv[CP], gv[CP];
        if (r < L) {
            const int64_t base = krow(r) * DK + c_0;
#pragma unroll
            for (int j = 0; j < CP; j += 4) {
                float a[4], b[4], g[4];
                gload<T, 4>(a, qg_ + base + j);
                gload<T, 4>(b, kg_ + base + j);
                gload<T, 4>(g, gg_ + base + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) { qv[j + e] = a[e]; kv[j + e] = b[e]; gv[j + e] = g[e]; }
            }
        } else {
#pragma unroll
            for (int j = 0; j < CP; ++j) { qv[j] = 0.f; kv[j] = 0.f; gv[j] = 0.f; }
        }
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < CP; ++j) { sq += qv[j] * qv[j]; sk += kv[j] * kv[j]; }
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) { sq += __shfl_xor(sq, m); sk += __shfl_xor(sk, m); }
        const float nq = sqrtf(sq + p.eps), nk = sqrtf(sk + p.eps);
        const float aq = p.scale / nq, ak = 1.f / nk;
#pragma unroll
        for (int j = 0; j < CP; ++j) {
            sm.q[r * PD + c_0 + j] = qv[j] * aq;
            sm.k[r * PD + c_0 + j] = kv[j] * ak;
            sm.G[r * PD + c_0 + j] = gv[j];
        }
        if (part == 0) {
            sm.beta[r] = r < L ? 1.f / (1.f + fast_exp(-gload1(bg_ + krow(r)))) : 0.f;
            sm.nq[r] = nq;
            sm.nk[r] = nk;
        }
        // dGam_C = sum over value columns of S0 * dS1, per key channel
        constexpr int TPC = kExactThreads / DK, VPT = DV / TPC;
        const int c = tid / TPC, v_0 = VPT * (tid % TPC);
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < VPT; j += 4) {
            const f32x4 a = ldS0(c, v_0 + j);
            const f32x4 b = ldS1(c, v_0 + j);
            d += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
        }
#pragma unroll
        for (int m = 1; m < TPC; m <<= 1) d += __shfl_xor(d, m);
        if (tid % TPC == 0) sm.dgc[c] = d;
    }
    __syncthreads();
    if (tid < DK) {
        float a = 0.f;
        for (int r = 0; r < C; ++r) {
            a += sm.G[r * PD + tid];
            sm.G[r * PD + tid] = a;
        }
        sm.gc[tid] = a;
    }
    __syncthreads();

    // ================= phase 1: Akk (-> T) and Aqk (-> R[0:4096]) =================
    float* const A2 = sm.R;
    float* const Uq = sm.R + 4096;
    float* const DUq = sm.R + 6144;
    {
        float kk[2][4], qk[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) { kk[i][j] = 0.f; qk[i][j] = 0.f; }
        if (sB <= rB + 1) {
            #pragma unroll 1
            for (int c = 0; c < DK; c += 4) {
                f32x4 kr[2], qr[2], gr[2], ks[4], gs[4];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    kr[i] = *reinterpret_cast<const f32x4*>(&sm.k[(rB + i) * PD + c]);
                    qr[i] = *reinterpret_cast<const f32x4*>(&sm.q[(rB + i) * PD + c]);
                    gr[i] = *reinterpret_cast<const f32x4*>(&sm.G[(rB + i) * PD + c]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ks[j] = *reinterpret_cast<const f32x4*>(&sm.k[(sB + j) * PD + c]);
                    gs[j] = *reinterpret_cast<const f32x4*>(&sm.G[(sB + j) * PD + c]);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // pairs above the diagonal take exponent 0; their sums are discarded
                        const bool low = sB + j <= rB + i;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float ex = fast_exp(low ? gr[i][e] - gs[j][e] : 0.f);
                            const float kx = ks[j][e] * ex;
                            kk[i][j] += kr[i][e] * kx;
                            qk[i][j] += qr[i][e] * kx;
                        }
                    }
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = rB + i;
            const float b = sm.beta[r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = sB + j;
                sm.T[r * C + s] = s < r ? b * kk[i][j] : 0.f;
                A2[r * C + s] = s <= r ? qk[i][j] : 0.f;
            }
        }
    }
    __syncthreads();

    // ================= phase 2: T = (I + Akk)^-1 by columns (into Uq..DUq, then sm.T) =================
    {
        float* const Tt = sm.R + 4096;   // [r][j], 4096 floats over the two quarter buffers
        if (tid < C) {
            const int j = tid;
            for (int r = 0; r < C; ++r) {
                float x;
                if (r < j) x = 0.f;
                else if (r == j) x = 1.f;
                else {
                    float acc = 0.f;
                    for (int s = j; s < r; ++s) acc += sm.T[r * C + s] * Tt[s * C + j];
                    x = -acc;
                }
                Tt[r * C + j] = x;
            }
        }
        __syncthreads();
        for (int e = tid; e < C * C; e += kExactThreads) sm.T[e] = Tt[e];
        __syncthreads();
    }

    // ================= phase 3: value quarters =================
    float dQG[RA][4], dW[RA][4], dKt[RA][4];   // key-side tile accumulators
    float dT1[2][4], dAqk[2][4];               // 64 x 64 tile accumulators
    float dbv = 0.f;                           // value part of dbeta for row rQ (partial over columns)
#pragma unroll
    for (int i = 0; i < RA; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) { dQG[i][e] = 0.f; dW[i][e] = 0.f; dKt[i][e] = 0.f; }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) { dT1[i][j] = 0.f; dAqk[i][j] = 0.f; }

    TO* const dvo = reinterpret_cast<TO*>(p.dv_out);
    for (int v0 = 0; v0 < DV; v0 += 32) {
        // X = beta v - (beta kh Gam) S0  (row rQ, columns v0 + cQ ..)
        {
            float x[4];
            const float b = sm.beta[rQ];
            if (rQ < L) {
                float vv[4];
                gload<T, 4>(vv, vg_ + krow(rQ) * DV + v0 + cQ);
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = b * vv[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = 0.f;
            }
            #pragma unroll 1
            for (int c = 0; c < DK; ++c) {
                const float kgv = b * sm.k[rQ * PD + c] * fast_exp(sm.G[rQ * PD + c]);
                const f32x4 s0 = ldS0(c, v0 + cQ);
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] -= kgv * s0[j];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) Uq[rQ * 32 + cQ + j] = x[j];
        }
        __syncthreads();
        // U = T X
        {
            float u[4] = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll 1
            for (int s = 0; s <= rQ; ++s) {
                const float t = sm.T[rQ * C + s];
                const f32x4 xv = *reinterpret_cast<const f32x4*>(&Uq[s * 32 + cQ]);
#pragma unroll
                for (int j = 0; j < 4; ++j) u[j] += t * xv[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j) Uq[rQ * 32 + cQ + j] = u[j];
            // this quarter of dO
            if (rQ < L) {
                float dd[4];
                gload<T, 4>(dd, dog + krow(rQ) * DV + v0 + cQ);
#pragma unroll
                for (int j = 0; j < 4; ++j) DUq[rQ * 32 + cQ + j] = dd[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) DUq[rQ * 32 + cQ + j] = 0.f;
            }
        }
        __syncthreads();
        // dAqk += dO U^T;  dQG += dO S0^T
        #pragma unroll 1
        for (int j = 0; j < 32; j += 4) {
            f32x4 dor[2], us[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) dor[i] = *reinterpret_cast<const f32x4*>(&DUq[(rB + i) * 32 + j]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) us[jj] = *reinterpret_cast<const f32x4*>(&Uq[(sB + jj) * 32 + j]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    dAqk[i][jj] += dor[i][0] * us[jj][0] + dor[i][1] * us[jj][1] + dor[i][2] * us[jj][2] +
                                   dor[i][3] * us[jj][3];
        }
        #pragma unroll 1
        for (int j = 0; j < 32; j += 4) {
            f32x4 dor[RA], s0[4];
#pragma unroll
            for (int i = 0; i < RA; ++i) dor[i] = *reinterpret_cast<const f32x4*>(&DUq[(rA + i) * 32 + j]);
#pragma unroll
            for (int e = 0; e < 4; ++e) s0[e] = ldS0(cA + e, v0 + j);
#pragma unroll
            for (int i = 0; i < RA; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dQG[i][e] += dor[i][0] * s0[e][0] + dor[i][1] * s0[e][1] + dor[i][2] * s0[e][2] + dor[i][3] * s0[e][3];
        }
        // dU = Aqk^T dO + Ktil dS1  (row rQ)
        {
            float du[4] = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll 1
            for (int t = rQ; t < C; ++t) {
                const float a = A2[t * C + rQ];
                const f32x4 d = *reinterpret_cast<const f32x4*>(&DUq[t * 32 + cQ]);
#pragma unroll
                for (int j = 0; j < 4; ++j) du[j] += a * d[j];
            }
            #pragma unroll 1
            for (int c = 0; c < DK; ++c) {
                const float kt = sm.k[rQ * PD + c] * fast_exp(sm.gc[c] - sm.G[rQ * PD + c]);
                const f32x4 d1 = ldS1(c, v0 + cQ);
#pragma unroll
                for (int j = 0; j < 4; ++j) du[j] += kt * d1[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 4; ++j) DUq[rQ * 32 + cQ + j] = du[j];
        }
        __syncthreads();
        // dBV = T^T dU: dv = beta dBV, dbeta += v . dBV
        {
            float d[4] = {0.f, 0.f, 0.f, 0.f};
            #pragma unroll 1
            for (int t = rQ; t < C; ++t) {
                const float a = sm.T[t * C + rQ];
                const f32x4 x = *reinterpret_cast<const f32x4*>(&DUq[t * 32 + cQ]);
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] += a * x[j];
            }
            if (rQ < L) {
                float vv[4];
                gload<T, 4>(vv, vg_ + krow(rQ) * DV + v0 + cQ);
                const float b = sm.beta[rQ];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    dvo[krow(rQ) * DV + v0 + cQ + j] = from_f32<TO>(b * d[j]);
                    dbv += vv[j] * d[j];
                }
            }
        }
        // dW -= dU S0^T;  dKt += U dS1^T
        #pragma unroll 1
        for (int j = 0; j < 32; j += 4) {
            f32x4 dur[RA], ur[RA], s0[4], d1[4];
#pragma unroll
            for (int i = 0; i < RA; ++i) {
                dur[i] = *reinterpret_cast<const f32x4*>(&DUq[(rA + i) * 32 + j]);
                ur[i] = *reinterpret_cast<const f32x4*>(&Uq[(rA + i) * 32 + j]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0[e] = ldS0(cA + e, v0 + j);
                d1[e] = ldS1(cA + e, v0 + j);
            }
#pragma unroll
            for (int i = 0; i < RA; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dW[i][e] -= dur[i][0] * s0[e][0] + dur[i][1] * s0[e][1] + dur[i][2] * s0[e][2] + dur[i][3] * s0[e][3];
                    dKt[i][e] += ur[i][0] * d1[e][0] + ur[i][1] * d1[e][1] + ur[i][2] * d1[e][2] + ur[i][3] * d1[e][3];
                }
        }
        __syncthreads();
        // beta v of this quarter replaces U
        {
            const float b = sm.beta[rQ];
            if (rQ < L) {
                float vv[4];
                gload<T, 4>(vv, vg_ + krow(rQ) * DV + v0 + cQ);
#pragma unroll
                for (int j = 0; j < 4; ++j) Uq[rQ * 32 + cQ + j] = b * vv[j];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) Uq[rQ * 32 + cQ + j] = 0.f;
            }
        }
        __syncthreads();
        // dT1 += dU (beta v)^T
        #pragma unroll 1
        for (int j = 0; j < 32; j += 4) {
            f32x4 dur[2], bv[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) dur[i] = *reinterpret_cast<const f32x4*>(&DUq[(rB + i) * 32 + j]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) bv[jj] = *reinterpret_cast<const f32x4*>(&Uq[(sB + jj) * 32 + j]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    dT1[i][jj] += dur[i][0] * bv[jj][0] + dur[i][1] * bv[jj][1] + dur[i][2] * bv[jj][2] +
                                  dur[i][3] * bv[jj][3];
        }
        __syncthreads();
    }

    // ================= phase 4: dT, dKG, dAkk =================
    float* const DW = sm.R;   // [64][DK]
#pragma unroll
    for (int i = 0; i < RA; ++i)
        *reinterpret_cast<f32x4*>(&DW[(rA + i) * DK + cA]) = f32x4{dW[i][0], dW[i][1], dW[i][2], dW[i][3]};
    __syncthreads();
    float dT[2][4], dKG[RA][4];
    {
        // dT = dT1 + dW (beta kh Gam)^T
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dT[i][jj] = dT1[i][jj];
        #pragma unroll 1
        for (int c = 0; c < DK; c += 4) {
            f32x4 dwr[2], kgs[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) dwr[i] = *reinterpret_cast<const f32x4*>(&DW[(rB + i) * DK + c]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int s = sB + jj;
                const f32x4 kv = *reinterpret_cast<const f32x4*>(&sm.k[s * PD + c]);
                const f32x4 gv = *reinterpret_cast<const f32x4*>(&sm.G[s * PD + c]);
                const float b = sm.beta[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) kgs[jj][e] = b * kv[e] * fast_exp(gv[e]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    dT[i][jj] += dwr[i][0] * kgs[jj][0] + dwr[i][1] * kgs[jj][1] + dwr[i][2] * kgs[jj][2] +
                                 dwr[i][3] * kgs[jj][3];
        }
        // dKG = T^T dW (the direct part; the Akk part is added pair by pair below)
#pragma unroll
        for (int i = 0; i < RA; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) dKG[i][e] = 0.f;
        #pragma unroll 1
        for (int t = rA; t < C; ++t) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&DW[t * DK + cA]);
#pragma unroll
            for (int i = 0; i < RA; ++i) {
                const float a = sm.T[t * C + rA + i];
#pragma unroll
                for (int e = 0; e < 4; ++e) dKG[i][e] += a * x[e];
            }
        }
    }
    __syncthreads();
    float* const M1 = sm.R;          // [64][64]
    float* const M2 = sm.R + 4096;   // [64][64]
#pragma unroll
    for (int i = 0; i < 2; ++i)
        *reinterpret_cast<f32x4*>(&M1[(rB + i) * C + sB]) = f32x4{dT[i][0], dT[i][1], dT[i][2], dT[i][3]};
    __syncthreads();
    {
        // Y = T^T dT
        float y[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) y[i][jj] = 0.f;
        #pragma unroll 1
        for (int t = rB; t < C; ++t) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&M1[t * C + sB]);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float a = sm.T[t * C + rB + i];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) y[i][jj] += a * x[jj];
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<f32x4*>(&M2[(rB + i) * C + sB]) = f32x4{y[i][0], y[i][1], y[i][2], y[i][3]};
    }
    __syncthreads();
    {
        // dAkk = -strict(Y T^T); dAqk kept lower (incl. diagonal)
        float a[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) a[i][jj] = 0.f;
        #pragma unroll 1
        for (int t = 0; t < C; t += 4) {
            f32x4 yr[2], ts[4];
#pragma unroll
            for (int i = 0; i < 2; ++i) yr[i] = *reinterpret_cast<const f32x4*>(&M2[(rB + i) * C + t]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ts[jj] = *reinterpret_cast<const f32x4*>(&sm.T[(sB + jj) * C + t]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    a[i][jj] += yr[i][0] * ts[jj][0] + yr[i][1] * ts[jj][1] + yr[i][2] * ts[jj][2] + yr[i][3] * ts[jj][3];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = rB + i;
            f32x4 x, z;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int s = sB + jj;
                x[jj] = s < r ? -a[i][jj] : 0.f;
                z[jj] = s <= r ? dAqk[i][jj] : 0.f;
            }
            *reinterpret_cast<f32x4*>(&M1[r * C + sB]) = x;   // dAkk
            *reinterpret_cast<f32x4*>(&M2[r * C + sB]) = z;   // dAqk
        }
    }
    __syncthreads();

    // ================= phase 5: per-row / per-channel gradients =================
    float dqh[RA][4], dkh[RA][4], dG[RA][4], dbk[RA];
    float qo[RA][4], ko[RA][4], go[RA][4], bo[RA];
    float redp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RA; ++i) {
        const int r = rA + i;
        bo[i] = sm.beta[r];
        dbk[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = cA + e;
            qo[i][e] = sm.q[r * PD + c];
            ko[i][e] = sm.k[r * PD + c];
            go[i][e] = sm.G[r * PD + c];
            const float gam = fast_exp(go[i][e]);
            const float ekt = fast_exp(sm.gc[c] - go[i][e]);
            dqh[i][e] = dQG[i][e] * gam;
            dkh[i][e] = bo[i] * gam * dKG[i][e] + dKt[i][e] * ekt;
            dG[i][e] = dQG[i][e] * qo[i][e] * gam + dKG[i][e] * bo[i] * ko[i][e] * gam - dKt[i][e] * ko[i][e] * ekt;
            dbk[i] += dKG[i][e] * ko[i][e] * gam;
            redp[e] += dKt[i][e] * ko[i][e] * ekt;
        }
    }
    // row side of the Akk / Aqk terms: for row r, sums over s <= r
    #pragma unroll 1
    for (int s = 0; s < rA + RA; ++s) {
        const f32x4 ks = *reinterpret_cast<const f32x4*>(&sm.k[s * PD + cA]);
        const f32x4 gs = *reinterpret_cast<const f32x4*>(&sm.G[s * PD + cA]);
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int r = rA + i;
            const bool ok = s <= r;
            const float a = ok ? M1[r * C + s] : 0.f;   // dAkk (0 on the diagonal)
            const float b = ok ? M2[r * C + s] : 0.f;   // dAqk
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kx = ks[e] * fast_exp(ok ? go[i][e] - gs[e] : 0.f);
                const float ak = a * kx, bk = b * kx;
                dkh[i][e] += bo[i] * ak;
                dqh[i][e] += bk;
                dG[i][e] += bo[i] * ko[i][e] * ak + qo[i][e] * bk;
                dbk[i] += ko[i][e] * ak;
            }
        }
    }
    // column side: for column s, sums over r >= s
    #pragma unroll 1
    for (int r = rA; r < C; ++r) {
        const f32x4 kr = *reinterpret_cast<const f32x4*>(&sm.k[r * PD + cA]);
        const f32x4 qr = *reinterpret_cast<const f32x4*>(&sm.q[r * PD + cA]);
        const f32x4 gr = *reinterpret_cast<const f32x4*>(&sm.G[r * PD + cA]);
        const float br = sm.beta[r];
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int s = rA + i;
            const bool ok = r >= s;
            const float a = ok ? M1[r * C + s] * br : 0.f;
            const float b = ok ? M2[r * C + s] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float t = (a * kr[e] + b * qr[e]) * fast_exp(ok ? gr[e] - go[i][e] : 0.f);
                dkh[i][e] += t;
                dG[i][e] -= ko[i][e] * t;
            }
        }
    }

    // ================= phase 6: chain rule through the norms and the sigmoid; write =================
    // value part of dbeta: row rQ over the 8 lanes of its column groups
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) dbv += __shfl_xor(dbv, m);
    if ((tid & 7) == 0) sm.db[rQ] = dbv;
    __syncthreads();   // also: every read of sm.q above is done
    TO* const dqo = reinterpret_cast<TO*>(p.dq);
    TO* const dko = reinterpret_cast<TO*>(p.dk);
    TO* const dbo = reinterpret_cast<TO*>(p.db);
    {
        float sqd[RA], skd[RA];
        float qbar[RA][4];
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int r = rA + i;
            sqd[i] = 0.f;
            skd[i] = 0.f;
            if (r < L) {
                float qv[4];
                gload<T, 4>(qv, qg_ + krow(r) * DK + cA);
                const float inq = 1.f / sm.nq[r];
#pragma unroll
                for (int e = 0; e < 4; ++e) qbar[i][e] = qv[e] * inq;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) qbar[i][e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sqd[i] += qbar[i][e] * (p.scale * dqh[i][e]);
                skd[i] += ko[i][e] * dkh[i][e];
            }
        }
        // sums over the NCG lanes that share the rows (consecutive lanes)
#pragma unroll
        for (int m = 1; m < NCG; m <<= 1) {
#pragma unroll
            for (int i = 0; i < RA; ++i) {
                sqd[i] += __shfl_xor(sqd[i], m);
                skd[i] += __shfl_xor(skd[i], m);
                dbk[i] += __shfl_xor(dbk[i], m);
            }
        }
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int r = rA + i;
            if (r < L) {
                const float inq = 1.f / sm.nq[r], ink = 1.f / sm.nk[r];
                float xq[4], xk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    xq[e] = (p.scale * dqh[i][e] - qbar[i][e] * sqd[i]) * inq;
                    xk[e] = (dkh[i][e] - ko[i][e] * skd[i]) * ink;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dqo[krow(r) * DK + cA + e] = from_f32<TO>(xq[e]);
                    dko[krow(r) * DK + cA + e] = from_f32<TO>(xk[e]);
                }
                if (tid % NCG == 0)
                    dbo[krow(r)] = from_f32<TO>((dbk[i] + sm.db[r]) * sigmoid_deriv(gload1(bg_ + krow(r))));
            }
        }
    }
    // dg: reverse cumulative sum over the rows of dG, plus dL/dG_C on every row
    float* const DG = sm.q;   // [64][PD], qh is no longer read
#pragma unroll
    for (int i = 0; i < RA; ++i)
        *reinterpret_cast<f32x4*>(&DG[(rA + i) * PD + cA]) = f32x4{dG[i][0], dG[i][1], dG[i][2], dG[i][3]};
    *reinterpret_cast<f32x4*>(&sm.red[rgA * DK + cA]) = f32x4{redp[0], redp[1], redp[2], redp[3]};
    __syncthreads();
    if (tid < DK) {
        const int c = tid;
        float run = sm.dgc[c] * fast_exp(sm.gc[c]);
        for (int g = 0; g < LY::NRG; ++g) run += sm.red[g * DK + c];
        TO* const dgo = reinterpret_cast<TO*>(p.dg);
        for (int r = C - 1; r >= 0; --r) {
            run += DG[r * PD + c];
            if (r < L) dgo[krow(r) * DK + c] = from_f32<TO>(run);
        }
    }
}

// Persistent over the (slot, head) items b, b + G, b + 2G, ... of workgroup b
// (G = gridDim.x).  With only_unsafe, an item is processed only if the reverse
// scan flagged its chunk (decay past kExactBelow); the flags of up to 512
// items are read at once and the flagged ones listed in LDS, so a launch with
// no flagged chunk costs one round of flag reads.
template <typename T, typename TO, int DK, int DV>
__global__ __launch_bounds__(kExactThreads, 1) void kda_bwd_exact_kernel(BwdParams p, int only_unsafe, int64_t nitems) {
    __shared__ __attribute__((aligned(16))) ExactLds<DK> sm;
    const int tid = threadIdx.x;
    const int64_t G = gridDim.x;
    for (int64_t j0 = 0; (int64_t)blockIdx.x + j0 * G < nitems; j0 += kExactThreads) {
        if (tid == 0) sm.nlist = 0;
        __syncthreads();
        const int64_t item = (int64_t)blockIdx.x + (j0 + tid) * G;
        if (item < nitems && (!only_unsafe || p.chunk_flags[item] != 0)) sm.list[atomicAdd(&sm.nlist, 1)] = tid;
        __syncthreads();
        const int cnt = sm.nlist;
        for (int k = 0; k < cnt; ++k) {
            const int64_t it = (int64_t)blockIdx.x + (j0 + sm.list[k]) * G;
            exact_chunk<T, TO, DK, DV>(p, sm, it / p.H, (int)(it % p.H));
            __syncthreads();   // the next item reuses every LDS array
        }
    }
}

}  // namespace ex

// ---------------------------------------------------------------- launchers
// fp32 inputs only: these kernels save fp32 states (bf16 inputs save fp16 ones
// and take their token-by-token chunks inline, kda_fwd16.hip / kda_scan16.hip)
hipError_t launch_fwd_token(const FwdParams& p, int in_dtype, int out_dtype, int dk, bool save, hipStream_t s) {
    if (in_dtype != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
#define KDA_FWD_TOKEN(TO, DK)                                                                                    \
    do {                                                                                                         \
        if (save) hipLaunchKernelGGL((ex::kda_fwd_token_kernel<float, TO, DK, true>), grid, dim3(kThreads), 0, s, p);  \
        else hipLaunchKernelGGL((ex::kda_fwd_token_kernel<float, TO, DK, false>), grid, dim3(kThreads), 0, s, p);      \
    } while (0)
    if (out_dtype == 0) { if (dk == 128) KDA_FWD_TOKEN(float, 128); else KDA_FWD_TOKEN(float, 64); }
    else { if (dk == 128) KDA_FWD_TOKEN(bf16, 128); else KDA_FWD_TOKEN(bf16, 64); }
#undef KDA_FWD_TOKEN
    return hipGetLastError();
}

hipError_t launch_bwd_scan_token(const BwdParams& p, int in_dtype, int dk, hipStream_t s) {
    if (in_dtype != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if (dk == 128) hipLaunchKernelGGL((ex::kda_bwd_scan_token_kernel<float, 128>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((ex::kda_bwd_scan_token_kernel<float, 64>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T, typename TO>
static void launch_exact_t(const BwdParams& p, int dk, int ou, int64_t n, dim3 grid, hipStream_t s) {
    const dim3 block(ex::kExactThreads);
    if (dk == 128 && p.dv == 128) hipLaunchKernelGGL((ex::kda_bwd_exact_kernel<T, TO, 128, 128>), grid, block, 0, s, p, ou, n);
    else if (dk == 128) hipLaunchKernelGGL((ex::kda_bwd_exact_kernel<T, TO, 128, 64>), grid, block, 0, s, p, ou, n);
    else if (p.dv == 128) hipLaunchKernelGGL((ex::kda_bwd_exact_kernel<T, TO, 64, 128>), grid, block, 0, s, p, ou, n);
    else hipLaunchKernelGGL((ex::kda_bwd_exact_kernel<T, TO, 64, 64>), grid, block, 0, s, p, ou, n);
}

hipError_t launch_bwd_exact(const BwdParams& p, int in_dtype, int out_dtype, int dk, bool only_unsafe,
                            hipStream_t s) {
    const int64_t n = num_slots(p.T, p.N) * p.H;   // (slot, head) items
    if (n == 0) return hipSuccess;
    // one workgroup per compute unit (the kernel's LDS allows no more)
    const dim3 grid((unsigned)(n < 256 ? n : 256));
    const int ou = only_unsafe ? 1 : 0;
    if (in_dtype == 0) {
        if (out_dtype == 0) launch_exact_t<float, float>(p, dk, ou, n, grid, s);
        else launch_exact_t<float, bf16>(p, dk, ou, n, grid, s);
    } else {
        if (out_dtype == 0) launch_exact_t<bf16, float>(p, dk, ou, n, grid, s);
        else launch_exact_t<bf16, bf16>(p, dk, ou, n, grid, s);
    }
    return hipGetLastError();
}

}  // namespace kda
