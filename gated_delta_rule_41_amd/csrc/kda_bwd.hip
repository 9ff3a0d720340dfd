// kda_bwd.hip -- chunked KDA backward for gfx950.
//
// The pages ask the backward to reuse what the forward saved (normalisation
// statistics and states) and to join state-gradient propagation with the Q/K
// gradients ("TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and
// training practice", section "KDA pre/post-processing fusion").  Here:
//
//  B1  reverse state-gradient scan (kda_bwd_scan_kernel for fp32 inputs;
//      kda_bwd_scan16_kernel in kda_scan16.hip for bf16 inputs).  One
//      persistent workgroup per (sequence, head, 64-column value slice) walks
//      the chunks backwards with dL/dS (dk x 64, fp32) resident in MFMA
//      accumulators:
//          dU  = Aqk^T dO + Ktil dS1
//          dS0 = Diag(Gam_C) dS1 + (qh Gam)^T dO - W^T dU
//      and writes dS1 (dL/dS at the end of every chunk) and dU for B2.
//  B2  chunk-parallel gradients (kda_bwd_grads_kernel; kda_bwd_chunk_f32_kernel
//      for fp32 inputs).  One workgroup per (chunk, head) recomputes the
//      chunk's Akk and T, reads the saved entering state S0, U, dS1 and dU, and
//      forms dq, dk, dv, dg, dbeta.
//
// Chunk equations (G the in-chunk cumulative log-decay, Gam = exp(G)):
//   QG = qh Gam, KG = beta kh Gam, KI = kh / Gam, Ktil = kh Gam_C / Gam
//   Akk = strict(KG KI^T), Aqk = lower(QG KI^T), T = (I + Akk)^{-1}
//   W = T KG, U = T beta v - W S0, O = QG S0 + Aqk U,
//   S1 = Diag(Gam_C) S0 + Ktil^T U
// and their reverse-mode derivatives (dAkk = -strict(T^T dT T^T), ...).
#include <type_traits>

#include "kda_device.h"
#include "kda_f16.h"
#include "kda_internal.h"
#include "kda_token.h"

namespace kda {

// ============================================================================
// B1: reverse state-gradient scan
// ============================================================================
template <typename T, int DK>
struct __attribute__((aligned(32))) ScanSmem {
    static constexpr bool SPLIT = std::is_same<T, bf16>::value;
    static constexpr int PK = DK + 8;
    static constexpr int PC = kChunk + 8;
    static constexpr int RK = kChunk * PK;
    static constexpr int RT = DK * PC;
    static constexpr int RG = RK > RT ? RK : RT;
    T r0[RG];                  // qh*Gam [r][perm32(c)]        -> (qh*Gam)^T hi [c][perm32(r)]
    T r1[SPLIT ? RG : 16];     //   lo                           -> (qh*Gam)^T lo
    T r2[RG];                  // kh/Gam [r][perm32(c)]        -> Ktil hi [r][perm32(c)]
    T r3[SPLIT ? RG : 16];     //   lo                           -> Ktil lo
    T kg[RK];                  // beta*kh*Gam [r][perm32(c)]
    T wt[RT];                  // -W^T [c][perm32(r)]
    T aqt[kChunk * PC];        // Aqk^T [s][perm32(r)]
    T aqtl[SPLIT ? kChunk * PC : 16];
    T akk[kChunk * PC];        // strict(Akk) [r][s]
    T dot[kSlice * PC];        // dO^T (input values) [c][perm32(r)]
    float adiag[4][16][20];
    float tdiag[4][16][20];
    float gc[DK];
    float red[4][DK];
};

template <typename T, int DK>
__global__ __launch_bounds__(kThreads, 1) void kda_bwd_scan_kernel(BwdParams p) {
    __shared__ ScanSmem<T, DK> sm;
    typedef ScanSmem<T, DK> SM;
    constexpr bool SPLIT = SM::SPLIT;
    constexpr int PK = SM::PK;
    constexpr int PC = SM::PC;
    constexpr int CPL = DK / 16;
    constexpr int VPL = kSlice / 16;
    constexpr int NKB = DK / 32;
    constexpr int NMB = DK / 16;
    constexpr int NWB = DK / 64;
    typedef typename V8<T>::t V8T;
    typedef typename V4<T>::t V4T;

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, qg = l >> 4, cl = l & 15;
    int chain, slice;
    map_block(blockIdx.x, p.N * p.H, p.nslices, chain, slice);
    const int n = chain / p.H, h = chain % p.H;
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int dv = p.dv, H = p.H;
    const int dv0 = slice * kSlice;
    const int vcol = dv0 + 16 * w + cl;

    const T* __restrict__ qp = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kp = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ gp = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bp = reinterpret_cast<const T*>(p.b);
    const T* __restrict__ dop = reinterpret_cast<const T*>(p.dO);
    float* __restrict__ dst = reinterpret_cast<float*>(p.dst_saved);

    const int64_t sbase = ((int64_t)n * H + h) * DK * dv;
    f32x4 dS[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[mb][i] = p.dS_final ? p.dS_final[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + vcol] : 0.f;

    float rq[4][CPL], rk[4][CPL], rg[4][CPL], rdo[4][VPL], rb[4];
    auto load_chunk = [&](int64_t c0) {
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * qg + i;
            if (r < L) {
                const int64_t tok = c0 + r;
                const int64_t rowk = (tok * H + h) * DK + CPL * cl;
                gload<T, CPL>(rq[i], qp + rowk);
                gload<T, CPL>(rk[i], kp + rowk);
                gload<T, CPL>(rg[i], gp + rowk);
                gload<T, VPL>(rdo[i], dop + (tok * H + h) * dv + dv0 + VPL * cl);
                rb[i] = gload1(bp + tok * H + h);
            } else {
#pragma unroll
                for (int e = 0; e < CPL; ++e) { rq[i][e] = 0.f; rk[i][e] = 0.f; rg[i][e] = 0.f; }
#pragma unroll
                for (int e = 0; e < VPL; ++e) rdo[i][e] = 0.f;
                rb[i] = 0.f;
            }
        }
    };
    const int64_t nchunks = (t1 - t0 + kChunk - 1) / kChunk;
    if (nchunks > 0) load_chunk(t0 + (nchunks - 1) * kChunk);
    // Aqk^T blocks above the diagonal of the (s, r) tile are never written.
    for (int e = tid; e < kChunk * PC; e += kThreads) {
        sm.aqt[e] = from_f32<T>(0.f);
        if constexpr (SPLIT) sm.aqtl[e] = from_f32<T>(0.f);
    }

    for (int64_t jc = nchunks - 1; jc >= 0; --jc) {
        const int64_t c0 = t0 + jc * kChunk;
        const int64_t slot = t0 / kChunk + n + jc;
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);

        // ================= prep =================
        float nq[4], nk[4], beta[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) { sq += rq[i][e] * rq[i][e]; sk += rk[i][e] * rk[i][e]; }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) { sq += __shfl_xor(sq, m); sk += __shfl_xor(sk, m); }
            nq[i] = sqrtf(sq + p.eps);
            nk[i] = sqrtf(sk + p.eps);
            const int r = 16 * w + 4 * qg + i;
            beta[i] = (r < L) ? 1.f / (1.f + fast_exp(-rb[i])) : 0.f;
        }
        float G[4][CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { a += rg[i][e]; G[i][e] = a; }
            const float tot = a;
            float s = tot, x;
            x = __shfl_up(s, 16);
            if (qg >= 1) s += x;
            x = __shfl_up(s, 32);
            if (qg >= 2) s += x;
            const float excl = s - tot;
#pragma unroll
            for (int i = 0; i < 4; ++i) G[i][e] += excl;
            if (qg == 3) sm.red[w][CPL * cl + e] = s;
        }
        __syncthreads();
        float GC[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int c = CPL * cl + e;
            float a = 0.f, tot = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const float x = sm.red[ww][c];
                if (ww < w) a += x;
                tot += x;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) G[i][e] += a;
            GC[e] = tot;
        }
        if (w == 0 && qg == 0) {
#pragma unroll
            for (int e = 0; e < CPL; ++e) sm.gc[CPL * cl + e] = fast_exp(GC[e]);
        }
        {
            // decay past the factorised range: the transposed recurrence token by
            // token (every wave holds every channel's sum, so the branch is uniform)
            bool tok = false, exact = false;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                tok |= !(GC[e] >= kTokenBelow);
                exact |= !(GC[e] >= kExactBelow);
            }
            const bool xexact = __builtin_amdgcn_ballot_w64(exact) != 0;
            if (slice == 0 && tid == 0) p.chunk_flags[slot * H + h] = xexact ? 1 : 0;
            if (__builtin_amdgcn_ballot_w64(tok) != 0) {
                if (jc > 0) load_chunk(c0 - kChunk);
                float* out = dst + (slot * H + h) * (int64_t)DK * dv;
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) out[(int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = dS[mb][i];
                const TokSrc<T> src = {qp, kp, gp, bp, dop, H, h, dv, vcol, qg, p.eps, p.scale};
                token_bwd<T, DK>(dS, src, c0, L);
                __syncthreads();
                continue;
            }
        }
        float qgv[CPL][4], ktv[CPL][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * qg + i;
            const float iq = p.scale / nq[i], ik = 1.f / nk[i];
#pragma unroll
            for (int e4 = 0; e4 < CPL; e4 += 4) {
                f32x4 vq, vk, vi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = e4 + j;
                    const float kh = rk[i][e] * ik;
                    const float gam = fast_exp(G[i][e]);
                    const float gin = fast_exp(-G[i][e]);
                    vq[j] = rq[i][e] * iq * gam;
                    vk[j] = beta[i] * kh * gam;
                    vi[j] = kh * gin;
                    qgv[e][i] = vq[j];
                    ktv[e][i] = kh * fast_exp(GC[e] - G[i][e]);
                }
                const int pc = perm32(CPL * cl + e4);
                sts4_split<T, SPLIT>(&sm.r0[r * PK + pc], &sm.r1[SPLIT ? r * PK + pc : 0], vq);
                sts4<T>(&sm.kg[r * PK + pc], vk);
                sts4_split<T, SPLIT>(&sm.r2[r * PK + pc], &sm.r3[SPLIT ? r * PK + pc : 0], vi);
            }
        }
        {
            const int pr = perm32(16 * w + 4 * qg);
#pragma unroll
            for (int e = 0; e < VPL; ++e) {
                f32x4 x = {rdo[0][e], rdo[1][e], rdo[2][e], rdo[3][e]};
                sts4<T>(&sm.dot[(VPL * cl + e) * PC + pr], x);   // exact: dO is an input value
            }
        }
        if (jc > 0) load_chunk(c0 - kChunk);
        __syncthreads();

        // ================= intra: Akk, Aqk^T =================
#pragma unroll
        for (int st = 0; st < 5; ++st) {
            const int it = w + 4 * st;
            const bool isqk = it >= 10;
            const int pi = isqk ? it - 10 : it;
            const int ib = pi >= 6 ? 3 : (pi >= 3 ? 2 : (pi >= 1 ? 1 : 0));
            const int jb = pi - (ib * (ib + 1)) / 2;
            const int ra = (16 * ib + cl) * PK + 8 * qg, rbk = (16 * jb + cl) * PK + 8 * qg;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (isqk) {
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) {
                    const V8T ah = lds8<T>(sm.r0 + ra + 32 * kk), bh = lds8<T>(sm.r2 + rbk + 32 * kk);
                    if constexpr (SPLIT)
                        acc = mma3<true>(acc, ah, lds8<T>(sm.r1 + ra + 32 * kk), bh, lds8<T>(sm.r3 + rbk + 32 * kk));
                    else
                        acc = mma_k32(acc, ah, bh);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk)
                    acc = mma_k32(acc, lds8<T>(sm.kg + ra + 32 * kk), lds8<T>(sm.r2 + rbk + 32 * kk));
            }
            const int s = 16 * jb + cl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ib + 4 * qg + i;
                if (isqk) {
                    const float val = s <= r ? acc[i] : 0.f;
                    const T hi = from_f32<T>(val);
                    sm.aqt[s * PC + perm32(r)] = hi;
                    if constexpr (SPLIT) sm.aqtl[s * PC + perm32(r)] = from_f32<T>(val - to_f32(hi));
                } else {
                    const float val = s < r ? acc[i] : 0.f;
                    sm.akk[r * PC + s] = from_f32<T>(val);
                    if (ib == jb) sm.adiag[ib][4 * qg + i][cl] = val;
                }
            }
        }
        __syncthreads();

        // ======== diagonal inverses; transposed / row-major scan tiles ========
        if (l < 16) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == l) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c) s -= sm.adiag[w][r][c] * x[c];
                x[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.tdiag[w][r][l] = x[r];
        }
        {
            const int pr = perm32(16 * w + 4 * qg);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                f32x4 x = {qgv[e][0], qgv[e][1], qgv[e][2], qgv[e][3]};
                sts4_split<T, SPLIT>(&sm.r0[(CPL * cl + e) * PC + pr], &sm.r1[SPLIT ? (CPL * cl + e) * PC + pr : 0], x);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * qg + i;
#pragma unroll
                for (int e4 = 0; e4 < CPL; e4 += 4) {
                    f32x4 x = {ktv[e4][i], ktv[e4 + 1][i], ktv[e4 + 2][i], ktv[e4 + 3][i]};
                    const int pc = perm32(CPL * cl + e4);
                    sts4_split<T, SPLIT>(&sm.r2[r * PK + pc], &sm.r3[SPLIT ? r * PK + pc : 0], x);
                }
            }
        }
        __syncthreads();

        // ======== blocked solve for W = (I + Akk)^{-1} beta kh Gam; store -W^T ========
        {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            V4T tii[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) tii[i] = pack4<T>(*reinterpret_cast<const f32x4*>(&sm.tdiag[i][cl][4 * qg]));
#pragma unroll
            for (int cb = 0; cb < NWB; ++cb) {
                const int nb = 16 * (w + 4 * cb);
                const int pc = perm32(nb + cl);
                f32x4 X[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 acc;
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = to_f32(sm.kg[(16 * i + 4 * qg + j) * PK + pc]);
#pragma unroll
                    for (int jp = 0; jp < i; ++jp)
                        acc = mma_k16(acc, neg4(lds4<T>(&sm.akk[(16 * i + cl) * PC + 16 * jp + 4 * qg])),
                                      pack4<T>(X[jp]));
                    X[i] = mma_k16(zero, tii[i], pack4<T>(acc));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) sts4<T>(&sm.wt[(nb + cl) * PC + perm32(16 * i + 4 * qg)], -X[i]);
            }
        }
        __syncthreads();

        // ================= reverse state-gradient step =================
        {
            float* out = dst + (slot * H + h) * (int64_t)DK * dv;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) out[(int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = dS[mb][i];
        }
        V8T dsh[NKB], dsl[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) split8<T, SPLIT>(dS[2 * kk], dS[2 * kk + 1], dsh[kk], dsl[kk]);
        V8T dof[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) dof[kk] = lds8<T>(sm.dot + (16 * w + cl) * PC + 32 * kk + 8 * qg);
        // dU = Aqk^T dO + Ktil dS1
        f32x4 dU[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ra = (16 * i + cl) * PC + 8 * qg;
#pragma unroll
            for (int kk = (i >> 1); kk < 2; ++kk) {
                acc = mma_k32(acc, lds8<T>(sm.aqt + ra + 32 * kk), dof[kk]);
                if constexpr (SPLIT) acc = mma_k32(acc, lds8<T>(sm.aqtl + ra + 32 * kk), dof[kk]);
            }
            const int rk2 = (16 * i + cl) * PK + 8 * qg;
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk)
                acc = mma3<SPLIT>(acc, lds8<T>(sm.r2 + rk2 + 32 * kk), lds8<T>(sm.r3 + (SPLIT ? rk2 + 32 * kk : 0)),
                                  dsh[kk], dsl[kk]);
            dU[i] = acc;
        }
        V8T duf[2];
        duf[0] = pack8<T>(dU[0], dU[1]);
        duf[1] = pack8<T>(dU[2], dU[3]);
        // dS0 = Diag(Gam_C) dS1 + (qh Gam)^T dO - W^T dU
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[16 * mb + 4 * qg]);
            f32x4 acc = dS[mb] * gcv;
            const int rt = (16 * mb + cl) * PC + 8 * qg;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                acc = mma_k32(acc, lds8<T>(sm.r0 + rt + 32 * kk), dof[kk]);
                if constexpr (SPLIT) acc = mma_k32(acc, lds8<T>(sm.r1 + rt + 32 * kk), dof[kk]);
                acc = mma_k32(acc, lds8<T>(sm.wt + rt + 32 * kk), duf[kk]);
            }
            dS[mb] = acc;
        }
        __syncthreads();
    }
    if (p.dS0) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.dS0[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = dS[mb][i];
    }
}

// ============================================================================
// B2: chunk-parallel gradients
// ============================================================================
// One workgroup per (chunk, head), full value width.  Operand tiles live in LDS
// in the orientation each product contracts over (8 contiguous elements per
// lane), written once per chunk; bf16 operands whose rounding shows in a
// gradient carry a lo tile and take three MFMAs.  The fp32 entering state S0
// and dS1 feed B fragments straight from global memory.  dU, dT and dW act as
// accumulator-resident B operands of the T^T products (perm32 layout of T^T).

__device__ __forceinline__ void st_blk(float* M, int ld, int m0, int n0, f32x4 x, int qg, int cl) {
#pragma unroll
    for (int i = 0; i < 4; ++i) M[(m0 + 4 * qg + i) * ld + n0 + cl] = x[i];
}


// Sixteen sums over the 16 lanes of each row group, one per lane: at each
// halving step a lane keeps the half of the remaining sums that its lane bit
// selects and adds its partner's copy of that half (the partner differs in that
// bit), so lane cl ends with the sum of v[cl].  v is used as scratch.
__device__ __forceinline__ float row16_scatter(float (&v)[16], int cl) {
    auto halve = [&](auto half, auto ctrl, int bit) {
        constexpr int hh = decltype(half)::value;
#pragma unroll
        for (int j = 0; j < hh; ++j) {
            const float keep = bit ? v[j + hh] : v[j];
            const float send = bit ? v[j] : v[j + hh];
            v[j] = keep + dpp<decltype(ctrl)::value>(send);
        }
    };
    halve(std::integral_constant<int, 8>{}, std::integral_constant<int, 0x140>{}, (cl >> 3) & 1);   // row_mirror
    halve(std::integral_constant<int, 4>{}, std::integral_constant<int, 0x141>{}, (cl >> 2) & 1);   // row_half_mirror
    halve(std::integral_constant<int, 2>{}, std::integral_constant<int, 0x4E>{}, (cl >> 1) & 1);    // quad_perm [2,3,0,1]
    halve(std::integral_constant<int, 1>{}, std::integral_constant<int, 0xB1>{}, cl & 1);           // quad_perm [1,0,3,2]
    return v[0];
}

// Slot layout of the chunk kernel's LDS (bytes).
template <typename T, int DK, int DV>
struct ChunkLds {
    static constexpr int PK = DK + 8, PV = DV + 8, PC = kChunk + 8, PF = kChunk + 4;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int RK = kChunk * PK * ES;          // [64][DK] tile
    static constexpr int RV = kChunk * PV * ES;          // [64][DV] tile
    static constexpr int CK = DK * PC * ES;              // [DK][64] tile
    static constexpr int CV = DV * PC * ES;              // [DV][64] tile
    static constexpr int RQ = kChunk * PC * ES;          // [64][64] tile
    static constexpr int FQ = kChunk * PF * 4;           // [64][64] fp32
    static constexpr int m2(int a, int b) { return a > b ? a : b; }
    static constexpr int SLOT0 = m2(m2(RK, RV), m2(CK, CV));
    static constexpr int SLOT1 = m2(SLOT0, m2(2 * RQ, FQ));
    static constexpr int SLOT = (SLOT1 + 255) & ~255;
    static constexpr int NSLOT = 8;
    static constexpr int QX = NSLOT * SLOT;              // one extra [64][64] tile
    static constexpr int SMALL = QX + ((RQ + 255) & ~255);
    // small arrays
    static constexpr int BETA = SMALL;                   // float[64]
    static constexpr int GC = BETA + 64 * 4;             // float[DK]
    static constexpr int DGC = GC + DK * 4;              // float[DK]
    static constexpr int RED = DGC + DK * 4;             // float[4][DK]
    static constexpr int DBV = RED + 4 * DK * 4;         // float[4][64]
    static constexpr int GW = DBV + 4 * 64 * 4;          // float[4][DK]: per-wave column sums of g
    static constexpr int SCL = GW + 4 * DK * 4;          // float[2][DV/16]: scales of S0 / dS1 (bf16 inputs)
    static constexpr int BYTES = SCL + 2 * (DV / 16) * 4;
    static_assert(BYTES <= 163840, "chunk kernel LDS");
};

// --- fragment helpers ------------------------------------------------------
// 8 fp32 values -> bf16 hi (and lo) fragments
__device__ __forceinline__ void cvt8(const float (&x)[8], bf16x8& hi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) hi[j] = (bf16)x[j];
}
__device__ __forceinline__ void cvt8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        hi[j] = (bf16)x[j];
        lo[j] = (bf16)(x[j] - (float)hi[j]);
    }
}
__device__ __forceinline__ void cvt8(const float (&x)[8], f32x8& hi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) hi[j] = x[j];
}
__device__ __forceinline__ void cvt8(const float (&x)[8], f32x8& hi, f32x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) { hi[j] = x[j]; lo[j] = 0.f; }
}
// 8 contiguous fp32 from global
__device__ __forceinline__ void gf8(float (&x)[8], const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
// 8 strided fp32 from global
__device__ __forceinline__ void gs8(float (&x)[8], const float* p, int ld) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = p[(int64_t)j * ld];
}
// 8 contiguous input elements from global as an operand fragment (exact)
__device__ __forceinline__ bf16x8 gin8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 gin8(const float* p) {
    f32x8 r;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
    return r;
}

// Store an accumulator block (rows m0+4qg+i, col n0+cl) into a tile.
// RM: row-major tile [m][n] (stride ld); else transposed tile [n][m].
template <typename T, bool SPLIT>
__device__ __forceinline__ void put_blk(T* hi, T* lo, int ld, int m0, int n0, f32x4 x, int qg, int cl, bool rm) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int o = rm ? (m0 + 4 * qg + i) * ld + n0 + cl : (n0 + cl) * ld + m0 + 4 * qg + i;
        const T h = from_f32<T>(x[i]);
        hi[o] = h;
        if constexpr (SPLIT) lo[o] = from_f32<T>(x[i] - to_f32(h));
    }
}
// Transposed store of 4 consecutive rows as one vector, tile [n][m] with m permuted by perm32.
template <typename T, bool SPLIT>
__device__ __forceinline__ void put_blk_tp(T* hi, T* lo, int ld, int m0, int n0, f32x4 x, int qg, int cl) {
    const int o = (n0 + cl) * ld + perm32(m0 + 4 * qg);
    sts4_split<T, SPLIT>(hi + o, lo + (SPLIT ? o : 0), x);
}

// N contiguous outputs from fp32 values, as 16-byte stores.
template <typename TO, int N>
__device__ __forceinline__ void store_row(TO* p, const float (&v)[N]) {
    if constexpr (N % 4 != 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) p[j] = from_f32<TO>(v[j]);
    } else if constexpr (sizeof(TO) == 4) {
#pragma unroll
        for (int j = 0; j < N; j += 4) *reinterpret_cast<f32x4*>(p + j) = f32x4{v[j], v[j + 1], v[j + 2], v[j + 3]};
    } else {
#pragma unroll
        for (int j = 0; j < N; j += 4)
            *reinterpret_cast<bf16x4*>(p + j) = pack4<bf16>(f32x4{v[j], v[j + 1], v[j + 2], v[j + 3]});
    }
}

// The A fragment (8 positions, perm32 order) of T^T at rows 16mb + cl and
// contraction block 32kk, read straight from the row-major T tile with the LDS
// transpose load (ds_read_b64_tr_b16: inside each row of 16 lanes, lane t
// receives element (t & 3) of the 8 bytes named by lanes 4k + (t >> 2),
// k = 0..3, as measured on gfx950): lane l names row 32kk + 16h + 4qg + (l >> 2),
// columns 16mb + 4(l & 3), so lane cl gets T[32kk + 16h + 4qg + j][16mb + cl].
__device__ __forceinline__ bf16x8 lds_trT(const bf16* tile, int ld, int mb, int kk, int qg, int cl) {
    typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
    const bf16* p0 = tile + (32 * kk + 4 * qg + (cl >> 2)) * ld + 16 * mb + 4 * (cl & 3);
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(const_cast<bf16*>(p0)));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(const_cast<bf16*>(p0 + 16 * ld)));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), 0, 1, 2, 3, 4, 5, 6, 7);
}

// ============================================================================
// B2 for bf16 inputs with 8 waves.
//
// Laid out for two waves per SIMD: every dk- or dv-wide output (64 rows x 16
// columns per block) belongs to wave w for column block w; the 64x64 products
// (Akk, T, dAqk, dT, dAkk) run on waves 0-3; the prep layout (q/k/g rows, the
// tiles written from them, the chain rule) gives wave w rows
// 16(w&3)..16(w&3)+15 and one half of the key columns, the two halves' row sums
// meeting in LDS.
// ============================================================================
template <typename TO, int DK, int DV>
__global__ __launch_bounds__(kWideThreads, 1) void kda_bwd_grads_kernel(BwdParams p) {
    typedef bf16 T;
    typedef ChunkLds<T, DK, DV> LY;
    __shared__ __attribute__((aligned(256))) char lds[LY::BYTES];
    constexpr bool SPLIT = true;
    constexpr int PK = LY::PK, PV = LY::PV, PC = LY::PC, PF = LY::PF;
    constexpr int CPH = DK / 32, VPH = DV / 32;   // key / value columns per lane (prep layout, half a row)
    constexpr int NKK = DK / 32, NKV = DV / 32;   // k32 steps over dk / dv
    typedef bf16x8 V8T;
    auto S = [&](int i) { return reinterpret_cast<T*>(lds + i * LY::SLOT); };
    auto Sh = [&](int i) { return reinterpret_cast<T*>(lds + i * LY::SLOT + LY::RQ); };   // second half
    auto Sf = [&](int i) { return reinterpret_cast<float*>(lds + i * LY::SLOT); };
    auto Sx = [&](int i) { return reinterpret_cast<_Float16*>(lds + i * LY::SLOT); };   // fp16 view
    T* const QX = reinterpret_cast<T*>(lds + LY::QX);
    float* const sbeta = reinterpret_cast<float*>(lds + LY::BETA);
    float* const sgc = reinterpret_cast<float*>(lds + LY::GC);
    float* const sdgc = reinterpret_cast<float*>(lds + LY::DGC);
    float* const sred = reinterpret_cast<float*>(lds + LY::RED);
    float* const sdbv = reinterpret_cast<float*>(lds + LY::DBV);
    float* const sgw = reinterpret_cast<float*>(lds + LY::GW);
    float* const sscl = reinterpret_cast<float*>(lds + LY::SCL);

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, qg = l >> 4, cl = l & 15;
    const int wl = w & 3, wh = w >> 2;
    const bool kact = w < DK / 16, vact = w < DV / 16;   // owns key / value column block 16w
    const int H = p.H;
    const int64_t slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int n = slot_owner(p.cu, p.N, p.seqlen, slot);
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int64_t jc = slot - (t0 / kChunk + n);
    const int64_t c0 = t0 + jc * kChunk;
    if (jc < 0 || c0 >= t1) return;   // unused slot (uniform across the workgroup)
    const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);

    const int64_t rsk = (int64_t)H * DK, rsv = (int64_t)H * DV;   // token strides
    // per-lane offsets inside a chunk fit in 32 bits (64 H max(dk, dv) < 2^31 is
    // checked on the host); only the chunk bases are 64-bit
    const int rk32 = (int)rsk, rv32 = (int)rsv;
    const float* __restrict__ nqc = p.nq_saved + (int64_t)h * p.T + c0;   // norms: head-major [H, T]
    const float* __restrict__ nkc = p.nk_saved + (int64_t)h * p.T + c0;
    const T* __restrict__ qc = reinterpret_cast<const T*>(p.q) + c0 * rsk + h * DK;
    const T* __restrict__ kc = reinterpret_cast<const T*>(p.k) + c0 * rsk + h * DK;
    const T* __restrict__ gcp = reinterpret_cast<const T*>(p.g) + c0 * rsk + h * DK;
    const T* __restrict__ vc = reinterpret_cast<const T*>(p.v) + c0 * rsv + h * DV;
    const T* __restrict__ doc = reinterpret_cast<const T*>(p.dO) + c0 * rsv + h * DV;
    const T* __restrict__ bc = reinterpret_cast<const T*>(p.b) + c0 * H + h;
    // S0 (saved by the forward) and dS1 (left by the reverse scan): fp16 scaled by
    // 2^-e per 16-column group, with 2^e in sv_scale / ds_scale
    const _Float16* __restrict__ S0 = reinterpret_cast<const _Float16*>(p.st_saved) + (slot * H + h) * (int64_t)DK * DV;
    const _Float16* __restrict__ dS1 = reinterpret_cast<const _Float16*>(p.dst_saved) + (slot * H + h) * (int64_t)DK * DV;
    const float* __restrict__ s0sc = p.sv_scale + (slot * H + h) * (DV / 16);
    const float* __restrict__ d1sc = p.ds_scale + (slot * H + h) * (DV / 16);
    // element (c, j) of the fp16 states: blocked by 16 value columns, [dv/16][dk][16]
    auto blk16 = [](int c, int j) { return ((j >> 4) * DK + c) * 16 + (j & 15); };
    // S0 / dS1 row fragments (loaded during Akk and T), kept in fp16 until used
    typedef _Float16 h8v __attribute__((ext_vector_type(8)));
    typedef _Float16 h4v __attribute__((ext_vector_type(4)));
    h8v xs0[NKV], xd0[NKV];

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int r0 = 16 * wl + 4 * qg;             // prep layout: rows r0..r0+3
    const int ck0 = wh * (DK / 2) + CPH * cl;    //   key columns ck0..ck0+CPH-1
    const int cv0 = wh * (DV / 2) + VPH * cl;    //   value columns cv0..cv0+VPH-1

    // ================= prep =================
    // The raw rows and gate cumsums are not kept across the kernel: prep_fill
    // reloads them (L2-resident) and rebuilds G from the per-wave column sums of
    // g, which the first call leaves in LDS.
    struct Prep {
        RawRow<T, CPH> q[4], k[4];
        float G[4][CPH], GC[CPH], beta[4], iq[4], ik[4], lg[4];   // lg: the beta logits
    };
    // the lane's raw rows as loaded (prep_load issues the loads, prep_finish
    // first uses them), so that a later step can have its rows in flight early
    struct PrepRaw {
        RawRow<T, CPH> q[4], k[4], g[4];
        float rb[4], nq[4], nk[4];
    };
    auto prep_load = [&](PrepRaw& R) {
        // rows past the chunk end load the last row (in bounds) and are zeroed
        // in prep_finish, once every load of the chunk is in flight
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rc = min(r0 + i, L - 1);
            R.q[i].load(qc + (rc * rk32 + ck0));
            R.k[i].load(kc + (rc * rk32 + ck0));
            R.g[i].load(gcp + (rc * rk32 + ck0));
            R.rb[i] = gload1(bc + rc * H);
            R.nq[i] = nqc[rc];     // norms saved by the forward
            R.nk[i] = nkc[rc];
        }
    };
    auto prep_finish = [&](Prep& P, PrepRaw& R, bool first) {
        RawRow<T, CPH>* rg = R.g;
        const float* rb = R.rb;
        const float* nq = R.nq;
        const float* nk = R.nk;
#pragma unroll
        for (int i = 0; i < 4; ++i) { P.q[i] = R.q[i]; P.k[i] = R.k[i]; }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = r0 + i < L;
            P.q[i].keep(ok); P.k[i].keep(ok); rg[i].keep(ok);
            // v_rcp (~1 ulp), as the forward forms beta and the reciprocal norms
            P.beta[i] = ok ? __builtin_amdgcn_rcpf(1.f + fast_exp(-rb[i])) : 0.f;
            P.lg[i] = rb[i];
            P.iq[i] = p.scale * __builtin_amdgcn_rcpf(ok ? nq[i] : 1.f);
            P.ik[i] = __builtin_amdgcn_rcpf(ok ? nk[i] : 1.f);
        }
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { a += rg[i][e] * kLog2e; P.G[i][e] = a; }
            const float tot = a;
            float s = tot, x;
            x = __shfl_up(s, 16);
            if (qg >= 1) s += x;
            x = __shfl_up(s, 32);
            if (qg >= 2) s += x;
            const float excl = s - tot;
#pragma unroll
            for (int i = 0; i < 4; ++i) P.G[i][e] += excl;
            if (first && qg == 3) sgw[wl * DK + ck0 + e] = s;
        }
        if (first) lds_barrier();
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            const int c = ck0 + e;
            float a = 0.f, tot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const float x = sgw[w2 * DK + c];
                if (w2 < wl) a += x;
                tot += x;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) P.G[i][e] += a;
            P.GC[e] = tot;
        }
    };
    // after_loads runs once the row loads are issued, before their first use:
    // more loads issued there wait only behind these
    auto prep_fill = [&](Prep& P, bool first, auto after_loads) {
        PrepRaw R;
        prep_load(R);
        after_loads();
        prep_finish(P, R, first);
    };
    // prep-layout value of qh*Gam, beta*kh*Gam, kh/Gam at (row i, col e)
    auto vQG = [&](const Prep& P, int i, int e) { return P.q[i][e] * P.iq[i] * fast_exp2(P.G[i][e]); };
    auto vKG = [&](const Prep& P, int i, int e) { return P.k[i][e] * (P.beta[i] * P.ik[i]) * fast_exp2(P.G[i][e]); };
    auto vKI = [&](const Prep& P, int i, int e) { return P.k[i][e] * P.ik[i] * fast_exp2(-P.G[i][e]); };
    // writers: row-major [r][c] tile (stride PK) or transposed [c][r] tile (stride PC)
    auto put_rm = [&](const Prep& P, T* hi, T* lo, auto val, bool split) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = (r0 + i) * PK + ck0;
            if constexpr (CPH == 4) {
                const f32x4 x = {val(P, i, 0), val(P, i, 1), val(P, i, 2), val(P, i, 3)};
                if (split) sts4_split<T, true>(hi + o, lo + o, x);
                else sts4<T>(hi + o, x);
            } else {
#pragma unroll
                for (int e = 0; e < CPH; ++e) {
                    const float x = val(P, i, e);
                    const T hv = from_f32<T>(x);
                    hi[o + e] = hv;
                    if (split) lo[o + e] = from_f32<T>(x - to_f32(hv));
                }
            }
        }
    };
    // The transposed [c][s] tiles (KG^T, KI^T, QG^T) swizzle their 8-element
    // groups by row: group g of row c sits at g ^ ((c >> 2) & 7).  A lane of
    // put_tp writes row ck0 + e, and rows four apart would otherwise fall on
    // the same banks.
    auto tsw = [](int c, int g) { return c * PC + 8 * (g ^ ((c >> 2) & 7)); };
    auto put_tp = [&](const Prep& P, T* hi, T* lo, auto val, bool split) {
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            const f32x4 x = {val(P, 0, e), val(P, 1, e), val(P, 2, e), val(P, 3, e)};
            const int o = tsw(ck0 + e, r0 >> 3) + (r0 & 7);
            if (split) sts4_split<T, true>(hi + o, lo + o, x);
            else sts4<T>(hi + o, x);
        }
    };

    // U (saved by the forward) and dU (left by the reverse scan) of this chunk for
    // value column block 16w, accumulator layout: rows 16mb+4qg+i, column 16w+cl
    h4v Uh[4], dUh[4];   // fp16 as saved, converted where first used
    f32x4 dU[4];
    RawRow<T, VPH> ddr[4], vvr[4];   // dO and v rows of this lane (prep layout), staged in LDS later
    {
    Prep P;
    // the 2 x DV/16 scales of S0 and dS1 go to LDS behind the first row loads, so
    // that no later step waits on a global round trip for them
    prep_fill(P, true, [&] {
        if (tid < 2 * (DV / 16)) sscl[tid] = tid < DV / 16 ? s0sc[tid] : d1sc[tid - DV / 16];
    });
    if (wl == 0 && qg == 0) {
#pragma unroll
        for (int e = 0; e < CPH; ++e) sgc[ck0 + e] = fast_exp2(P.GC[e]);
    }
    if (wh == 0 && cl == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sbeta[r0 + i] = P.beta[i];
    }
    put_rm(P, S(2), S(2), vKI, false);   // KI  h
    put_rm(P, S(4), S(4), vKG, false);   // KG  h
    lds_barrier();
    {
        {
            // fp16, scaled per 16-column group like S0 / dS1 (this wave's columns: group
            // w).  Loaded by every wave (a wave past dv reads group 0 and never uses it):
            // under a branch the compiler converts the halves right after the loads and
            // so waits for them there.
            const int wv = vact ? w : 0;
            const _Float16* __restrict__ ub = reinterpret_cast<const _Float16*>(p.u_saved) + (slot * H + h) * (int64_t)kChunk * DV;
            const _Float16* __restrict__ dub = reinterpret_cast<const _Float16*>(p.du_ws) + (slot * H + h) * (int64_t)kChunk * DV;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {   // fragment order (ufrag): 512 contiguous bytes per load
                const int o = ((4 * wv + mb) * 64 + l) * 4;
                Uh[mb] = *reinterpret_cast<const h4v*>(ub + o);
                dUh[mb] = *reinterpret_cast<const h4v*>(dub + o);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {   // zeroed past the chunk end when staged
            const int rc = min(r0 + i, L - 1);
            vvr[i].load(vc + (rc * rv32 + cv0));
            ddr[i].load(doc + (rc * rv32 + cv0));
        }
    }

    // S0 row fragments of key column block 16w for dQG and dW.  The loads of
    // this kernel are spread over the steps before their first use (U, dU, v,
    // dO and S0 here, dS1 two steps later): a wave stalls at issue while its
    // memory queue is full, so issuing everything at once left Akk and T
    // waiting behind it (measured 4% slower overall).
    if (kact) {
        const int nr = 16 * w + cl;
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) xs0[kk] = *reinterpret_cast<const h8v*>(S0 + blk16(nr, 32 * kk + 8 * qg));
    }
    // ================= Akk (fp32 -> slot 5) =================
    float* const Af = Sf(5);
    if (w < 4) {
        const int nb = 16 * w;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f32x4 a = zero;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int ka = (16 * mb + cl) * PK + 32 * kk + 8 * qg, kb = (nb + cl) * PK + 32 * kk + 8 * qg;
                a = mma_k32(a, lds8<T>(S(4) + ka), lds8<T>(S(2) + kb));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mb + 4 * qg + i, s = nb + cl;
                Af[r * PF + s] = s < r ? a[i] : 0.f;
            }
        }
    }
    lds_barrier();
    // ================= T = (I + Akk)^{-1} (fp32 in slot 7) =================
    float* const Tf = Sf(7);
    // the six 16 x 16 blocks above the diagonal are zero; waves 4-7 clear them
    // (384 16-byte pieces) while waves 0-3 invert the diagonal blocks, and the
    // blocks below are written by the solve (columns past 64 are never read)
    if (w >= 4) {
        for (int e = tid - 256; e < 384; e += 256) {
            const int pr = e >> 6, row = (e >> 2) & 15, q4 = e & 3;
            const int bi = pr < 3 ? 0 : (pr < 5 ? 1 : 2), bj = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
            *reinterpret_cast<f32x4*>(&Tf[(16 * bi + row) * PF + 16 * bj + 4 * q4]) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (w < 4) {
        const f32x4 na = *reinterpret_cast<const f32x4*>(&Af[(16 * w + cl) * PF + 16 * w + 4 * qg]);
        f32x4 nbv;
#pragma unroll
        for (int j = 0; j < 4; ++j) nbv[j] = Af[(16 * w + 4 * qg + j) * PF + 16 * w + cl];
        const f32x4 tw = inv_unit_lower16(na, nbv, qg, cl);
#pragma unroll
        for (int i = 0; i < 4; ++i) Tf[(16 * w + 4 * qg + i) * PF + 16 * w + cl] = tw[i];
    }
    lds_barrier();
    // dS1 row fragments of key column block 16w, for dKtil
    if (kact) {
        const int nr = 16 * w + cl;
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) xd0[kk] = *reinterpret_cast<const h8v*>(dS1 + blk16(nr, 32 * kk + 8 * qg));
    }
    // off-diagonal blocks, column j on wave j: T_ij = -T_ii sum_{k=j}^{i-1} Akk_ik T_kj
    {
        auto solve_col = [&](auto jcst) {
            constexpr int j = decltype(jcst)::value;
            f32x4 col[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) col[j][i] = Tf[(16 * j + 4 * qg + i) * PF + 16 * j + cl];
#pragma unroll
            for (int i = j + 1; i < 4; ++i) {
                f32x4 acc = zero;
#pragma unroll
                for (int k = j; k < i; ++k)
                    acc = mma_k16(acc, *reinterpret_cast<const f32x4*>(&Af[(16 * i + cl) * PF + 16 * k + 4 * qg]), col[k]);
                const f32x4 tii = *reinterpret_cast<const f32x4*>(&Tf[(16 * i + cl) * PF + 16 * i + 4 * qg]);
                col[i] = -mma_k16(zero, tii, acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) Tf[(16 * i + 4 * qg + r) * PF + 16 * j + cl] = col[i][r];
            }
        };
        if (w == 0) solve_col(std::integral_constant<int, 0>{});
        else if (w == 1) solve_col(std::integral_constant<int, 1>{});
        else if (w == 2) solve_col(std::integral_constant<int, 2>{});
    }
    lds_barrier();
    // T tile: Trm [r][s] (slot 0 first half, kept until the last products; its
    // transpose is read with the LDS transpose load), eight elements per thread;
    // KG^T [c][s] (slot 1)
    {
        static_assert(kChunk * kChunk == 8 * kWideThreads, "one 8-element row piece per thread");
        const int r = tid >> 3, c = 8 * (tid & 7);
        const f32x4 a = *reinterpret_cast<const f32x4*>(&Tf[r * PF + c]);
        const f32x4 b = *reinterpret_cast<const f32x4*>(&Tf[r * PF + c + 4]);
        *reinterpret_cast<V8T*>(S(0) + r * PC + c) = pack8<T>(a, b);
        put_tp(P, S(1), S(1), vKG, false);
    }
    }
    lds_barrier();
    // The value-side products meet in fp16 at one power-of-two scale per tensor:
    // U and S0 carry per-16-column scales sv_g (those of the saved state), dU and
    // dS1 scales ds_g; both are brought to the largest one (exact unless a value
    // underflows, and then it is negligible against that group).  v and dO come
    // in at 1/svmax and |scale|/dsmax, under the bounds the forward and the scan
    // chose those scales for.  Every product below is rescaled in fp32 after.
    float svmax = sscl[0], dsmax = sscl[DV / 16];
#pragma unroll
    for (int g = 1; g < DV / 16; ++g) {
        svmax = fmaxf(svmax, sscl[g]);
        dsmax = fmaxf(dsmax, sscl[DV / 16 + g]);
    }
    const float isv = 1.f / svmax, ids = 1.f / dsmax;      // exact: powers of two
    const float qs = fabsf(p.scale);
    const float ko = qs * ids;                              // dO -> fp16 operand
    const float FS = svmax * dsmax;                         // U/dU/S0/dS1/v products
    const float FO = qs > 0.f ? FS / qs : 0.f;              // products with dO
    // U rm (slot 4), dU rm (slot 7), dO rm (slot 6), v rm (slot 2), all fp16
    // (each lane's VPH columns: DV/32 of them, 4 at dv = 128, 2 at dv = 64)
    typedef float FV __attribute__((ext_vector_type(VPH)));
    typedef _Float16 HV __attribute__((ext_vector_type(VPH)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ddr[i].keep(r0 + i < L);
        vvr[i].keep(r0 + i < L);
        FV dvv, vvv;
#pragma unroll
        for (int e = 0; e < VPH; ++e) { dvv[e] = ddr[i][e] * ko; vvv[e] = vvr[i][e] * isv; }
        *reinterpret_cast<HV*>(Sx(6) + (r0 + i) * PV + cv0) = __builtin_convertvector(dvv, HV);
        *reinterpret_cast<HV*>(Sx(2) + (r0 + i) * PV + cv0) = __builtin_convertvector(vvv, HV);
    }
    if (vact) {
        const float us = sscl[w], dus = sscl[DV / 16 + w];
        const float ur = us * isv, dr = dus * ids;       // powers of two <= 1
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            dU[mb] = __builtin_convertvector(dUh[mb], f32x4) * dus;
            const f32x4 u2 = __builtin_convertvector(Uh[mb], f32x4) * ur;
            const f32x4 d2 = __builtin_convertvector(dUh[mb], f32x4) * dr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (16 * mb + 4 * qg + i) * PV + 16 * w + cl;
                Sx(4)[o] = (_Float16)u2[i];
                Sx(7)[o] = (_Float16)d2[i];
            }
        }
    }
    lds_barrier();

    // ================= dBV = T^T dU  ->  dv, dbeta (v part) =================
    if (vact) {
        TO* __restrict__ dvp = reinterpret_cast<TO*>(p.dv_out) + c0 * rsv + h * DV;
        float rowpart[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) rowpart[mb][i] = 0.f;
        V8T bh[2], bl[2];
        split8<T, SPLIT>(dU[0], dU[1], bh[0], bl[0]);
        split8<T, SPLIT>(dU[2], dU[3], bh[1], bl[1]);
        const int nc = 16 * w + cl;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f32x4 a = zero;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (mb >= 2 && kk == 0) continue;   // T^T rows 32.. x columns ..31: zero (T is lower)
                const V8T ah = lds_trT(S(0), PC, mb, kk, qg, cl);   // T^T
                a = mma_k32(a, ah, bh[kk]);
                a = mma_k32(a, ah, bl[kk]);
            }
            // rows past the chunk end have v = 0 in the tile: no guard on the row sums
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mb + 4 * qg + i;
                rowpart[mb][i] += (float)Sx(2)[r * PV + nc] * svmax * a[i];   // v (fp16, at 1/svmax)
                a[i] *= sbeta[r];
            }
            auto put = [&](int i) { *at32(dvp, (unsigned)((16 * mb + 4 * qg + i) * rv32 + nc)) = from_f32<TO>(a[i]); };
            if (L == kChunk) {   // uniform: every row of the chunk exists
#pragma unroll
                for (int i = 0; i < 4; ++i) put(i);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * mb + 4 * qg + i < L) put(i);
            }
        }
        // waves 0-3 write their row sums; waves 4-7 park theirs in sred (unused
        // until the chain rule) and add them after the next barrier; lane cl
        // holds the sum of rows 16(cl>>2) + 4qg + (cl&3)
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = rowpart[j >> 2][j & 3];
        (w < 4 ? sdbv : sred)[(w & 3) * 64 + 16 * (cl >> 2) + 4 * qg + (cl & 3)] = row16_scatter(v, cl);
    }
    // ================= dAqk = lower(dO U^T);  dT = (dU v^T) diag(beta) (waves 0-3) =================
    f32x4 dAqk[4], dT[4];
    if (w < 4) {
        const int nb = 16 * w;
        // dAqkT: the same product with the operands swapped, so that the accumulator
        // holds dAqk[16mb+cl][nb+4qg+i] and the row-major tile takes 4-element stores
        f32x4 dAqkT[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) { dAqk[mb] = zero; dT[mb] = zero; dAqkT[mb] = zero; }
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) {
            const int kb = (nb + cl) * PV + 32 * kk + 8 * qg;
            const f16::h8 ub = *reinterpret_cast<const f16::h8*>(Sx(4) + kb);
            const f16::h8 vb = *reinterpret_cast<const f16::h8*>(Sx(2) + kb);   // rows past the chunk end are zero
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int ka = (16 * mb + cl) * PV + 32 * kk + 8 * qg;
                const f16::h8 da = *reinterpret_cast<const f16::h8*>(Sx(6) + ka);
                dAqk[mb] = f16::mma32(dAqk[mb], da, ub);
                dAqkT[mb] = f16::mma32(dAqkT[mb], ub, da);
                dT[mb] = f16::mma32(dT[mb], *reinterpret_cast<const f16::h8*>(Sx(7) + ka), vb);
            }
        }
        // dAqk rm h/l [r][s] (slots 3 and its second half; free until the last products)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = nb + 4 * qg + i <= 16 * mb + cl ? dAqkT[mb][i] * FO : 0.f;
            const int o = (16 * mb + cl) * PC + nb + 4 * qg;
            sts4_split<T, SPLIT>(S(3) + o, Sh(3) + o, x);
        }
        const float bs = sbeta[nb + cl] * FS;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mb + 4 * qg + i;
                dAqk[mb][i] = nb + cl <= r ? dAqk[mb][i] * FO : 0.f;
                dT[mb][i] *= bs;
            }
    }
    // ================= dQG = dO S0^T;  dW = -dU S0^T;  dKt = U dS1^T (key column block 16w) =================
    f32x4 dQG[4], dW[4], dKt[4];
    if (kact) {
        const int nr = 16 * w + cl;   // key row of S0 / dS1 feeding this lane
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) { dQG[mb] = zero; dW[mb] = zero; dKt[mb] = zero; }
        float gpart = 0.f;   // this lane's share of dL/dGam_C[nr] = sum_j S0[nr][j] dS1[nr][j]
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) {
            const float ss = sscl[2 * kk + (qg >> 1)], sd = sscl[DV / 16 + 2 * kk + (qg >> 1)];
            f32x4 sa, sb, da_, db_;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sa[j] = (float)xs0[kk][j];
                sb[j] = (float)xs0[kk][j + 4];
                da_[j] = (float)xd0[kk][j];
                db_[j] = (float)xd0[kk][j + 4];
                gpart += (sa[j] * ss) * (da_[j] * sd) + (sb[j] * ss) * (db_[j] * sd);
            }
            const float sr = ss * isv, dr = sd * ids;       // powers of two <= 1
            const f16::h8 s8 = f16::cvt8(sa * sr, sb * sr), d8 = f16::cvt8(da_ * dr, db_ * dr);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int ka = (16 * mb + cl) * PV + 32 * kk + 8 * qg;
                dQG[mb] = f16::mma32(dQG[mb], *reinterpret_cast<const f16::h8*>(Sx(6) + ka), s8);
                dW[mb] = f16::mma32(dW[mb], *reinterpret_cast<const f16::h8*>(Sx(7) + ka), s8);
                dKt[mb] = f16::mma32(dKt[mb], *reinterpret_cast<const f16::h8*>(Sx(4) + ka), d8);
            }
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            dQG[mb] *= FO;
            dW[mb] *= -FS;
            dKt[mb] *= FS;
        }
        gpart += __shfl_xor(gpart, 16);
        gpart += __shfl_xor(gpart, 32);
        if (qg == 0) sdgc[nr] = gpart;
    }
    lds_barrier();
    // waves 4-7 add their dbeta (v part) row sums after waves 0-3 wrote theirs: fixed order
    if (w >= 4 && vact && cl == 0) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (w - 4) * 64 + 16 * mb + 4 * qg + i;
                sdbv[o] += sred[o];
            }
    }
    {
    Prep P;
    prep_fill(P, false, [] {});
    // dW rm (slot 2), KG rm (slot 6)
    if (kact) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) put_blk<T, false>(S(2), S(2), PK, 16 * mb, 16 * w, dW[mb], qg, cl, true);
    }
    put_rm(P, S(6), S(6), vKG, false);
    lds_barrier();
    // ================= dT += dW KG^T;  X = T^T dT -> slot 0 (2nd half) (waves 0-3) =================
    if (w < 4) {
        const int nb = 16 * w;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const V8T bk = lds8<T>(S(6) + (nb + cl) * PK + 32 * kk + 8 * qg);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                dT[mb] = mma_k32(dT[mb], lds8<T>(S(2) + (16 * mb + cl) * PK + 32 * kk + 8 * qg), bk);
        }
        V8T th[2], tl[2];
        split8<T, false>(dT[0], dT[1], th[0], tl[0]);
        split8<T, false>(dT[2], dT[3], th[1], tl[1]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f32x4 x = zero;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                if (!(mb >= 2 && kk == 0)) x = mma_k32(x, lds_trT(S(0), PC, mb, kk, qg, cl), th[kk]);   // T^T: upper
            put_blk<T, false>(Sh(0), Sh(0), PC, 16 * mb, nb, x, qg, cl, true);
        }
    }
    lds_barrier();
    // ================= dAkk = -strict(X T^T) (all waves) =================
    // column block nb on waves w and w + 4: row blocks 0-1 on waves 0-3, 2-3 on
    // waves 4-7 (an even split measured faster; the same split of Akk did not)
    f32x4 dAkk[2];
    {
        const int nb = 16 * wl;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int mb = 2 * wh + m;
            // a: dAkk[16mb+4qg+i][nb+cl]; at: operands swapped, dAkk[16mb+cl][nb+4qg+i]
            f32x4 a = zero, at = zero;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const V8T xa = lds8<T>(Sh(0) + (16 * mb + cl) * PC + 32 * kk + 8 * qg);
                const V8T tb = lds8<T>(S(0) + (nb + cl) * PC + 32 * kk + 8 * qg);
                a = mma_k32(a, xa, tb);
                at = mma_k32(at, tb, xa);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = nb + cl < 16 * mb + 4 * qg + i ? -a[i] : 0.f;
                at[i] = nb + 4 * qg + i < 16 * mb + cl ? -at[i] : 0.f;
            }
            sts4<T>(QX + (nb + cl) * PC + 16 * mb + 4 * qg, a);   // dAkk^T [s][r]
            dAkk[m] = at;
        }
    }
    lds_barrier();
    // tiles for the last products:
    //   dAkk rm [r][s] (slot 0, 2nd half), dAkk^T [s][r] (QX), dAqk rm h/l (slot 3),
    //   dAqk^T h/l (slot 7), KI^T h/l [c][s] (slots 2, 6), QG^T h/l [c][r] (slots 4, 5)
#pragma unroll
    for (int m = 0; m < 2; ++m)
        sts4<T>(Sh(0) + (16 * (2 * wh + m) + cl) * PC + 16 * wl + 4 * qg, dAkk[m]);   // dAkk rm [r][s]
    if (w < 4) {
        const int nb = 16 * w;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int o = (nb + cl) * PC + 16 * mb + 4 * qg;                // dAqk^T h/l [s][r]
            sts4_split<T, SPLIT>(S(7) + o, Sh(7) + o, dAqk[mb]);
        }
    }
    put_tp(P, S(2), S(6), vKI, true);
    put_tp(P, S(4), S(5), vQG, true);
    }
    lds_barrier();
    // ================= dKG = T^T dW + dAkk KI;  dQG += dAqk KI;  dKI = dAkk^T KG + dAqk^T QG =================
    f32x4 dKG[4], dKI[4];
    if (kact) {
        const int nb = 16 * w;
        V8T whi[2], wlo[2];
        split8<T, false>(dW[0], dW[1], whi[0], wlo[0]);
        split8<T, false>(dW[2], dW[3], whi[1], wlo[1]);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f32x4 a = zero, qq = dQG[mb], ki = zero;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int ka = (16 * mb + cl) * PC + 32 * kk + 8 * qg, kb = tsw(nb + cl, 4 * kk + qg);
                // blocks that the triangular factors make zero are skipped: T^T,
                // dAkk^T, dAqk^T vanish for rows 32.. against columns ..31 (mb >= 2,
                // kk = 0), dAkk and dAqk for rows ..31 against columns 32.. (mb <= 1,
                // kk = 1)
                if (!(mb >= 2 && kk == 0)) {
                    a = mma_k32(a, lds_trT(S(0), PC, mb, kk, qg, cl), whi[kk]);              // T^T dW
                    ki = mma_k32(ki, lds8<T>(QX + ka), lds8<T>(S(1) + kb));                  // dAkk^T KG
                    ki = mma3<true>(ki, lds8<T>(S(7) + ka), lds8<T>(Sh(7) + ka), lds8<T>(S(4) + kb),
                                    lds8<T>(S(5) + kb));                                     // dAqk^T QG
                }
                if (!(mb <= 1 && kk == 1)) {
                    const V8T kih = lds8<T>(S(2) + kb);
                    a = mma_k32(a, lds8<T>(Sh(0) + ka), kih);                                // dAkk KI
                    qq = mma3<true>(qq, lds8<T>(S(3) + ka), lds8<T>(Sh(3) + ka), kih, lds8<T>(S(6) + kb));   // dAqk KI
                }
            }
            dKG[mb] = a;
            dQG[mb] = qq;
            dKI[mb] = ki;
        }
    }
    lds_barrier();

    // ================= back to the prep layout (fp32 through LDS) =================
    // (the chain rule's rows go out now and arrive during the transposes)
    PrepRaw R3;
    prep_load(R3);
    float* const F0 = Sf(0);   // slots 0-1
    float* const F1 = Sf(2);   // slots 2-3
    float* const F2 = Sf(4);   // slots 4-5
    float* const F3 = Sf(6);   // slots 6-7
    static_assert(DK * kChunk * 4 <= 2 * LY::SLOT, "fp32 staging");
    // The staging tiles are transposed, [key column c][row r], 64 floats per
    // column: an accumulator block (rows 16mb + 4qg + i, column 16w + cl) goes
    // in as one 16-byte store per lane and the prep layout (rows r0..r0+3,
    // column ck0 + e) comes out as one 16-byte load.  The 4-row group g of
    // column c sits at g ^ f(c), f's bits being c0^c2, c0^c3, c1^c4, c0^c5, which
    // keeps both the stores (8 lanes on consecutive columns) and the loads (16
    // lanes on columns four apart) free of bank conflicts.
    auto fst = [](int c, int g) {
        const int f = ((c ^ (c >> 2)) & 1) | (((c ^ (c >> 3)) & 1) << 1) | ((((c >> 1) ^ (c >> 4)) & 1) << 2) |
                      (((c ^ (c >> 5)) & 1) << 3);
        return c * kChunk + 4 * (g ^ f);
    };
    float gQ[4][CPH], gKG[4][CPH], gKI[4][CPH], gKt[4][CPH];
    if (kact) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int o = fst(16 * w + cl, 4 * mb + qg);
            *reinterpret_cast<f32x4*>(F0 + o) = dQG[mb];
            *reinterpret_cast<f32x4*>(F1 + o) = dKG[mb];
            *reinterpret_cast<f32x4*>(F2 + o) = dKI[mb];
            *reinterpret_cast<f32x4*>(F3 + o) = dKt[mb];
        }
    }
    lds_barrier();
#pragma unroll
    for (int e = 0; e < CPH; ++e) {
        const int o = fst(ck0 + e, r0 >> 2);
        const f32x4 a = *reinterpret_cast<const f32x4*>(F0 + o), b = *reinterpret_cast<const f32x4*>(F1 + o),
                    c = *reinterpret_cast<const f32x4*>(F2 + o), d = *reinterpret_cast<const f32x4*>(F3 + o);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gQ[i][e] = a[i];
            gKG[i][e] = b[i];
            gKI[i][e] = c[i];
            gKt[i][e] = d[i];
        }
    }

    // ================= chain rule to qh, kh, beta, G =================
    Prep P;
    prep_finish(P, R3, false);
    float dqh[4][CPH], dkh[4][CPH], dG[4][CPH], dbk[4], colp[CPH];
#pragma unroll
    for (int e = 0; e < CPH; ++e) colp[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dbk[i] = 0.f;
        const float aq = P.iq[i], ai = P.ik[i];
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            const float gam = fast_exp2(P.G[i][e]), gin = fast_exp2(-P.G[i][e]), ek = sgc[ck0 + e] * gin;
            const float qh = P.q[i][e] * aq, kh = P.k[i][e] * ai;
            const float QG = qh * gam, KGv = P.beta[i] * kh * gam, KIv = kh * gin, Ktv = kh * ek;
            dqh[i][e] = gQ[i][e] * gam;
            dkh[i][e] = P.beta[i] * gam * gKG[i][e] + gKI[i][e] * gin + gKt[i][e] * ek;
            dG[i][e] = gQ[i][e] * QG + gKG[i][e] * KGv - gKI[i][e] * KIv - gKt[i][e] * Ktv;
            dbk[i] += gKG[i][e] * kh * gam;
            colp[e] += gKt[i][e] * Ktv;
        }
    }
    lds_barrier();   // F0 reads done before it holds the row sums below
    // per-lane column partials [4 row blocks][4 row groups][DK] (summed after the
    // barrier in a fixed order; no cross-lane shuffles on this path)
    float* const spart = F0 + 512;
    typedef float FC __attribute__((ext_vector_type(CPH)));   // the lane's CPH columns
    {
        FC v;
#pragma unroll
        for (int e = 0; e < CPH; ++e) v[e] = colp[e];
        *reinterpret_cast<FC*>(&spart[(wl * 4 + qg) * DK + ck0]) = v;
    }
    // per-half row sums: qh . dqh, kh . dkh, and the k part of dbeta
    float* const srow = F0;   // [2 halves][3][64]
    {
        // v[4 kind + i]: kind 0 qh . dqh, 1 kh . dkh, 2 dbeta (k part) of row r0 + i
        float v[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < CPH; ++e) { sq += P.q[i][e] * P.iq[i] * dqh[i][e]; sk += P.k[i][e] * P.ik[i] * dkh[i][e]; }
            v[i] = sq;
            v[4 + i] = sk;
            v[8 + i] = dbk[i];
            v[12 + i] = 0.f;
        }
        const float t = row16_scatter(v, cl);
        if (cl < 12) srow[(wh * 3 + (cl >> 2)) * 64 + r0 + (cl & 3)] = t;
    }
    lds_barrier();
    FC dGC = *reinterpret_cast<const FC*>(&spart[ck0]);
#pragma unroll
    for (int g = 1; g < 16; ++g) dGC += *reinterpret_cast<const FC*>(&spart[g * DK + ck0]);
    dGC += *reinterpret_cast<const FC*>(&sdgc[ck0]) * *reinterpret_cast<const FC*>(&sgc[ck0]);
    {
        // reverse cumsum of dG over the 64 rows: the lane's own four rows, then the
        // totals of every later row group (row 16 wl + 4 qg + i), from LDS
        float* const stot = F0 + 512 + 16 * DK;
        FC tot;
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 3; i >= 0; --i) { a += dG[i][e]; dG[i][e] = a; }
            tot[e] = a;
        }
        *reinterpret_cast<FC*>(&stot[(wl * 4 + qg) * DK + ck0]) = tot;
        lds_barrier();
        FC a = dGC;
        const int wlu = __builtin_amdgcn_readfirstlane(wl);   // the row block is wave-uniform
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            if (w2 < wlu) continue;
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
                const FC v = *reinterpret_cast<const FC*>(&stot[(w2 * 4 + q2) * DK + ck0]);
                if (w2 > wlu) a += v;
                else a += q2 > qg ? v : FC(0.f);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < CPH; ++e) dG[i][e] += a[e];
    }
    // ================= through the L2 norms and the sigmoid; write =================
    TO* __restrict__ dqp = reinterpret_cast<TO*>(p.dq) + c0 * rsk + h * DK;
    TO* __restrict__ dkp = reinterpret_cast<TO*>(p.dk) + c0 * rsk + h * DK;
    TO* __restrict__ dgp = reinterpret_cast<TO*>(p.dg) + c0 * rsk + h * DK;
    TO* __restrict__ dbp = reinterpret_cast<TO*>(p.db) + c0 * H + h;
    const float isc2 = p.scale != 0.f ? 1.f / (p.scale * p.scale) : 0.f;
    const bool full = L == kChunk;   // uniform
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
        if (full || r < L) {
            const float aq = P.iq[i], ai = P.ik[i];
            const float sq = srow[0 * 64 + r] + srow[3 * 64 + r];
            const float sk = srow[1 * 64 + r] + srow[4 * 64 + r];
            const float qdot = sq * isc2;   // (qh . dqh) / scale^2
            float vq[CPH], vk[CPH];
#pragma unroll
            for (int e = 0; e < CPH; ++e) {
                const float qh = P.q[i][e] * aq, kh = P.k[i][e] * ai;
                vq[e] = aq * (dqh[i][e] - qh * qdot);
                vk[e] = ai * (dkh[i][e] - kh * sk);
            }
            const int off = r * rk32 + ck0;
            store_row<TO, CPH>(dqp + off, vq);
            store_row<TO, CPH>(dkp + off, vk);
            store_row<TO, CPH>(dgp + off, dG[i]);
            if (wh == 0 && cl == 0) {
                const float db = srow[2 * 64 + r] + srow[5 * 64 + r];
                const float dbeta = db + sdbv[r] + sdbv[64 + r] + sdbv[128 + r] + sdbv[192 + r];
                // sigma'(b) from the logit itself
                dbp[r * H] = from_f32<TO>(dbeta * sigmoid_deriv(P.lg[i]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32-input variant of B2: fp32 operands in LDS gathered in any orientation and
// contracted as hi/lo bf16 (three MFMAs per step).  Used for fp32 inputs only,
// where the bf16 tiling of the kernel above does not fit the LDS.
// 8 values M[r][k..k+7] of a row-major fp32 matrix (contiguous).
__device__ __forceinline__ void g8_row(float (&x)[8], const float* M, int ld, int r, int k) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(M + (int64_t)r * ld + k);
    const f32x4 b = *reinterpret_cast<const f32x4*>(M + (int64_t)r * ld + k + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
// 8 values M[k..k+7][c] (strided).
__device__ __forceinline__ void g8_col(float (&x)[8], const float* M, int ld, int k, int c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = M[(int64_t)(k + j) * ld + c];
}

__device__ __forceinline__ f32x4 mma_split(f32x4 acc, const float (&a)[8], const float (&b)[8]) {
    bf16x8 ah, al, bh, bl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ah[j] = (bf16)a[j];
        al[j] = (bf16)(a[j] - (float)ah[j]);
        bh[j] = (bf16)b[j];
        bl[j] = (bf16)(b[j] - (float)bh[j]);
    }
    acc = mma_k32(acc, ah, bh);
    acc = mma_k32(acc, ah, bl);
    acc = mma_k32(acc, al, bh);
    return acc;
}

// acc += A[m0:m0+16, k0:k1] B[k0:k1, n0:n0+16].
// AM = 0: A stored row-major [m][k]; AM = 1: A stored transposed [k][m].
// BM = 0: B stored [k][n];           BM = 1: B stored transposed [n][k].
template <int AM, int BM>
__device__ __forceinline__ f32x4 gemm_blk(f32x4 acc, const float* A, int lda, const float* B, int ldb, int m0,
                                          int n0, int k0, int k1, int qg, int cl) {
    for (int k = k0; k < k1; k += 32) {
        float a[8], b[8];
        if constexpr (AM == 0) g8_row(a, A, lda, m0 + cl, k + 8 * qg);
        else g8_col(a, A, lda, k + 8 * qg, m0 + cl);
        if constexpr (BM == 0) g8_col(b, B, ldb, k + 8 * qg, n0 + cl);
        else g8_row(b, B, ldb, n0 + cl, k + 8 * qg);
        acc = mma_split(acc, a, b);
    }
    return acc;
}

template <int DK, int DV>
struct __attribute__((aligned(32))) ChunkSmem {
    static constexpr int LD = (DK > DV ? DK : DV) + 4;   // row stride of the 64 x d slots
    static constexpr int LQ = kChunk + 4;                // row stride of the 64 x 64 slots
    float R0[kChunk * LD];
    float R1[kChunk * LD];
    float R2[kChunk * LD];
    float Q0[kChunk * LQ];
    float Q1[kChunk * LQ];
    float Q2[kChunk * LQ];
    float beta[kChunk];
    float gc[DK];        // Gam_C
    float dgc[DK];       // dL/dGam_C  (sum over dv of S0 * dS1)
    float red[4][DK];    // cross-wave column partials
    float dbv[4][kChunk];  // per-wave row partials of sum_v v * dBV
};

template <typename T, typename TO, int DK, int DV>
__global__ __launch_bounds__(kThreads, 1) void kda_bwd_chunk_f32_kernel(BwdParams p) {
    __shared__ ChunkSmem<DK, DV> sm;
    constexpr int LD = ChunkSmem<DK, DV>::LD;
    constexpr int LQ = ChunkSmem<DK, DV>::LQ;
    constexpr int CPL = DK / 16;
    constexpr int VPL = DV / 16;
    constexpr int NBK = DK / 64;   // dk-wide output column blocks per wave
    constexpr int NBV = DV / 64;   // dv-wide output column blocks per wave

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, qg = l >> 4, cl = l & 15;
    const int H = p.H;
    const int64_t slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    const int n = slot_owner(p.cu, p.N, p.seqlen, slot);
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int64_t jc = slot - (t0 / kChunk + n);
    const int64_t c0 = t0 + jc * kChunk;
    if (jc < 0 || c0 >= t1) return;   // unused slot (uniform across the workgroup)
    const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);

    const T* __restrict__ qp = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kp = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vp = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gp = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bp = reinterpret_cast<const T*>(p.b);
    const T* __restrict__ dop = reinterpret_cast<const T*>(p.dO);
    const float* __restrict__ S0 = reinterpret_cast<const float*>(p.st_saved) + (slot * H + h) * (int64_t)DK * DV;
    const float* __restrict__ dS1 = reinterpret_cast<const float*>(p.dst_saved) + (slot * H + h) * (int64_t)DK * DV;

    // ---------------- prep (rows r_i = 16w+4qg+i, key cols CPL*cl+e) ----------------
    float qh[4][CPL], kh[4][CPL], G[4][CPL], vv[4][VPL], dov[4][VPL], beta[4], dsig[4], nq[4], nk[4];
    float GC[CPL];
    {
        float rg[4][CPL], rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * qg + i;
            if (r < L) {
                const int64_t tok = c0 + r;
                const int64_t rowk = (tok * H + h) * DK + CPL * cl;
                gload<T, CPL>(qh[i], qp + rowk);
                gload<T, CPL>(kh[i], kp + rowk);
                gload<T, CPL>(rg[i], gp + rowk);
                gload<T, VPL>(vv[i], vp + (tok * H + h) * DV + VPL * cl);
                gload<T, VPL>(dov[i], dop + (tok * H + h) * DV + VPL * cl);
                rb[i] = gload1(bp + tok * H + h);
                nq[i] = p.nq_saved[(int64_t)h * p.T + tok];     // norms saved by the forward ([H, T])
                nk[i] = p.nk_saved[(int64_t)h * p.T + tok];
            } else {
#pragma unroll
                for (int e = 0; e < CPL; ++e) { qh[i][e] = 0.f; kh[i][e] = 0.f; rg[i][e] = 0.f; }
#pragma unroll
                for (int e = 0; e < VPL; ++e) { vv[i][e] = 0.f; dov[i][e] = 0.f; }
                rb[i] = 0.f;
                nq[i] = 1.f;
                nk[i] = 1.f;
            }
            beta[i] = (r < L) ? 1.f / (1.f + fast_exp(-rb[i])) : 0.f;
            dsig[i] = (r < L) ? sigmoid_deriv(rb[i]) : 0.f;
            const float iq = p.scale / nq[i], ik = 1.f / nk[i];
#pragma unroll
            for (int e = 0; e < CPL; ++e) { qh[i][e] *= iq; kh[i][e] *= ik; }
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { a += rg[i][e]; G[i][e] = a; }
            const float tot = a;
            float s = tot, x;
            x = __shfl_up(s, 16);
            if (qg >= 1) s += x;
            x = __shfl_up(s, 32);
            if (qg >= 2) s += x;
            const float excl = s - tot;
#pragma unroll
            for (int i = 0; i < 4; ++i) G[i][e] += excl;
            if (qg == 3) sm.red[w][CPL * cl + e] = s;
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        const int c = CPL * cl + e;
        float a = 0.f, tot = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float x = sm.red[ww][c];
            if (ww < w) a += x;
            tot += x;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i][e] += a;
        GC[e] = tot;
    }
    if (w == 0 && qg == 0) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) sm.gc[CPL * cl + e] = fast_exp(GC[e]);
    }
    if (cl == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.beta[16 * w + 4 * qg + i] = beta[i];
    }
    // operand writers (prep layout -> row-major fp32 slot)
    auto put_QG = [&](float* M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < CPL; ++e) M[(16 * w + 4 * qg + i) * LD + CPL * cl + e] = qh[i][e] * fast_exp(G[i][e]);
    };
    auto put_KG = [&](float* M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < CPL; ++e)
                M[(16 * w + 4 * qg + i) * LD + CPL * cl + e] = beta[i] * kh[i][e] * fast_exp(G[i][e]);
    };
    auto put_KI = [&](float* M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < CPL; ++e) M[(16 * w + 4 * qg + i) * LD + CPL * cl + e] = kh[i][e] * fast_exp(-G[i][e]);
    };
    auto put_Kt = [&](float* M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < CPL; ++e)
                M[(16 * w + 4 * qg + i) * LD + CPL * cl + e] = kh[i][e] * fast_exp(GC[e] - G[i][e]);
    };
    auto put_BV = [&](float* M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < VPL; ++e) M[(16 * w + 4 * qg + i) * LD + VPL * cl + e] = beta[i] * vv[i][e];
    };
    auto put_dO = [&](float* M) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < VPL; ++e) M[(16 * w + 4 * qg + i) * LD + VPL * cl + e] = dov[i][e];
    };
    put_QG(sm.R0);
    put_KI(sm.R1);
    put_KG(sm.R2);
    // T slot: upper blocks must read as zero
    for (int e = tid; e < kChunk * LQ; e += kThreads) sm.Q2[e] = 0.f;
    __syncthreads();

    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // ---------------- Akk (Q0), Aqk (Q1) ----------------
    {
        const int nb = 16 * w;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            f32x4 a = gemm_blk<0, 1>(zero, sm.R2, LD, sm.R1, LD, 16 * mb, nb, 0, DK, qg, cl);
            f32x4 b = gemm_blk<0, 1>(zero, sm.R0, LD, sm.R1, LD, 16 * mb, nb, 0, DK, qg, cl);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mb + 4 * qg + i, s = nb + cl;
                a[i] = s < r ? a[i] : 0.f;
                b[i] = s <= r ? b[i] : 0.f;
            }
            st_blk(sm.Q0, LQ, 16 * mb, nb, a, qg, cl);
            st_blk(sm.Q1, LQ, 16 * mb, nb, b, qg, cl);
        }
    }
    __syncthreads();
    // ---------------- T = (I + Akk)^{-1} into Q2 (fp32, blocked) ----------------
    if (l < 16) {
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = (r == l) ? 1.f : 0.f;
#pragma unroll
            for (int c = 0; c < r; ++c) s -= sm.Q0[(16 * w + r) * LQ + 16 * w + c] * x[c];
            x[r] = s;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Q2[(16 * w + r) * LQ + 16 * w + l] = x[r];
    }
    put_BV(sm.R1);   // KI is not read again until it is rebuilt
    __syncthreads();
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        // tmp_ij = sum_{k=j}^{i-1} Akk_ik T_kj, kept in the (unused) upper block (j, i) of Q0
        for (int idx = tid; idx < (4 - d) * 256; idx += kThreads) {
            const int j = idx >> 8, i = j + d, a = (idx >> 4) & 15, b = idx & 15;
            float s = 0.f;
            for (int k = j; k < i; ++k)
#pragma unroll
                for (int t = 0; t < 16; ++t) s += sm.Q0[(16 * i + a) * LQ + 16 * k + t] * sm.Q2[(16 * k + t) * LQ + 16 * j + b];
            sm.Q0[(16 * j + a) * LQ + 16 * i + b] = s;
        }
        __syncthreads();
        for (int idx = tid; idx < (4 - d) * 256; idx += kThreads) {
            const int j = idx >> 8, i = j + d, a = (idx >> 4) & 15, b = idx & 15;
            float s = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) s += sm.Q2[(16 * i + a) * LQ + 16 * i + t] * sm.Q0[(16 * j + t) * LQ + 16 * i + b];
            sm.Q2[(16 * i + a) * LQ + 16 * j + b] = -s;
        }
        __syncthreads();
    }

    // ---------------- W = T KG, Ut = T beta v ----------------
    f32x4 Wacc[NBK][4], U[NBV][4];
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            Wacc[t][mb] = gemm_blk<0, 0>(zero, sm.Q2, LQ, sm.R2, LD, 16 * mb, 16 * (w + 4 * t), 0, kChunk, qg, cl);
#pragma unroll
    for (int t = 0; t < NBV; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            U[t][mb] = gemm_blk<0, 0>(zero, sm.Q2, LQ, sm.R1, LD, 16 * mb, 16 * (w + 4 * t), 0, kChunk, qg, cl);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.R0, LD, 16 * mb, 16 * (w + 4 * t), Wacc[t][mb], qg, cl);
    __syncthreads();
    // ---------------- U = Ut - W S0 ----------------
#pragma unroll
    for (int t = 0; t < NBV; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            U[t][mb] -= gemm_blk<0, 0>(zero, sm.R0, LD, S0, DV, 16 * mb, 16 * (w + 4 * t), 0, DK, qg, cl);
    __syncthreads();
    // R0 <- Ktil, R1 <- dO, R2 <- U
    put_Kt(sm.R0);
    put_dO(sm.R1);
#pragma unroll
    for (int t = 0; t < NBV; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.R2, LD, 16 * mb, 16 * (w + 4 * t), U[t][mb], qg, cl);
    __syncthreads();
    // ---------------- dU, dQG (S0 part), dKt, dAqk, dGam_C ----------------
    f32x4 dU[NBV][4], dQG[NBK][4], dKt[NBK][4], dAqk[4];
#pragma unroll
    for (int t = 0; t < NBV; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int nb = 16 * (w + 4 * t);
            f32x4 a = gemm_blk<1, 0>(zero, sm.Q1, LQ, sm.R1, LD, 16 * mb, nb, 0, kChunk, qg, cl);   // Aqk^T dO
            dU[t][mb] = gemm_blk<0, 0>(a, sm.R0, LD, dS1, DV, 16 * mb, nb, 0, DK, qg, cl);        // + Ktil dS1
        }
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int nb = 16 * (w + 4 * t);
            dQG[t][mb] = gemm_blk<0, 1>(zero, sm.R1, LD, S0, DV, 16 * mb, nb, 0, DV, qg, cl);    // dO S0^T
            dKt[t][mb] = gemm_blk<0, 1>(zero, sm.R2, LD, dS1, DV, 16 * mb, nb, 0, DV, qg, cl);   // U dS1^T
        }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        f32x4 a = gemm_blk<0, 1>(zero, sm.R1, LD, sm.R2, LD, 16 * mb, 16 * w, 0, DV, qg, cl);   // dO U^T
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * mb + 4 * qg + i, s = 16 * w + cl;
            a[i] = s <= r ? a[i] : 0.f;
        }
        dAqk[mb] = a;
    }
    {
        // dL/dGam_C[c] = sum_j S0[c][j] dS1[c][j]; two threads per row c when DK = 128
        constexpr int TPR = kThreads / DK;
        const int c = tid / TPR, part = tid % TPR;
        float s = 0.f;
        for (int j = part; j < DV; j += TPR) s += S0[(int64_t)c * DV + j] * dS1[(int64_t)c * DV + j];
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) s += __shfl_xor(s, m);
        if (part == 0) sm.dgc[c] = s;
    }
    __syncthreads();
    // R0 <- dU, R2 <- beta v, Q0 <- dAqk
#pragma unroll
    for (int t = 0; t < NBV; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.R0, LD, 16 * mb, 16 * (w + 4 * t), dU[t][mb], qg, cl);
    put_BV(sm.R2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st_blk(sm.Q0, LQ, 16 * mb, 16 * w, dAqk[mb], qg, cl);
    __syncthreads();
    // ---------------- dW = -dU S0^T; dBV = T^T dU (-> dv, dbeta part); dT = dU (beta v)^T ----------------
    f32x4 dW[NBK][4], dT[4];
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
            dW[t][mb] = -gemm_blk<0, 1>(zero, sm.R0, LD, S0, DV, 16 * mb, 16 * (w + 4 * t), 0, DV, qg, cl);
    {
        TO* __restrict__ dvp = reinterpret_cast<TO*>(p.dv_out);
        float rowpart[4][4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) rowpart[mb][i] = 0.f;
#pragma unroll
        for (int t = 0; t < NBV; ++t)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int nb = 16 * (w + 4 * t);
                const f32x4 dbv = gemm_blk<1, 0>(zero, sm.Q2, LQ, sm.R0, LD, 16 * mb, nb, 0, kChunk, qg, cl);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * mb + 4 * qg + i;
                    if (r < L) {
                        const int64_t off = ((c0 + r) * H + h) * DV + nb + cl;
                        dvp[off] = from_f32<TO>(sm.beta[r] * dbv[i]);
                        rowpart[mb][i] += to_f32(vp[off]) * dbv[i];
                    }
                }
            }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float s = rowpart[mb][i];
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) s += __shfl_xor(s, m);
                if (cl == 0) sm.dbv[w][16 * mb + 4 * qg + i] = s;
            }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) dT[mb] = gemm_blk<0, 1>(zero, sm.R0, LD, sm.R2, LD, 16 * mb, 16 * w, 0, DV, qg, cl);
    __syncthreads();
    // R1 <- dW, R2 <- KG
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.R1, LD, 16 * mb, 16 * (w + 4 * t), dW[t][mb], qg, cl);
    put_KG(sm.R2);
    __syncthreads();
    // dT += dW KG^T  -> Q1
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) dT[mb] = gemm_blk<0, 1>(dT[mb], sm.R1, LD, sm.R2, LD, 16 * mb, 16 * w, 0, DK, qg, cl);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) st_blk(sm.Q1, LQ, 16 * mb, 16 * w, dT[mb], qg, cl);
    __syncthreads();
    // X = T^T dT -> R0 (as a 64 x 64 block with stride LQ)
    {
        f32x4 X[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) X[mb] = gemm_blk<1, 0>(zero, sm.Q2, LQ, sm.Q1, LQ, 16 * mb, 16 * w, 0, kChunk, qg, cl);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.R0, LQ, 16 * mb, 16 * w, X[mb], qg, cl);
    }
    __syncthreads();
    // dAkk = -strict(X T^T) -> Q1
    {
        f32x4 D[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            D[mb] = gemm_blk<0, 1>(zero, sm.R0, LQ, sm.Q2, LQ, 16 * mb, 16 * w, 0, kChunk, qg, cl);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * mb + 4 * qg + i, s = 16 * w + cl;
                D[mb][i] = s < r ? -D[mb][i] : 0.f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.Q1, LQ, 16 * mb, 16 * w, D[mb], qg, cl);
    }
    put_KI(sm.R0);
    __syncthreads();
    // ---------------- dKG = T^T dW + dAkk KI;  dQG += dAqk KI ----------------
    f32x4 dKG[NBK][4], dKI[NBK][4];
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int nb = 16 * (w + 4 * t);
            f32x4 a = gemm_blk<1, 0>(zero, sm.Q2, LQ, sm.R1, LD, 16 * mb, nb, 0, kChunk, qg, cl);
            dKG[t][mb] = gemm_blk<0, 0>(a, sm.Q1, LQ, sm.R0, LD, 16 * mb, nb, 0, kChunk, qg, cl);
            dQG[t][mb] = gemm_blk<0, 0>(dQG[t][mb], sm.Q0, LQ, sm.R0, LD, 16 * mb, nb, 0, kChunk, qg, cl);
        }
    __syncthreads();
    put_QG(sm.R1);   // dW is no longer needed
    __syncthreads();
    // ---------------- dKI = dAkk^T KG + dAqk^T QG ----------------
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int nb = 16 * (w + 4 * t);
            f32x4 a = gemm_blk<1, 0>(zero, sm.Q1, LQ, sm.R2, LD, 16 * mb, nb, 0, kChunk, qg, cl);
            dKI[t][mb] = gemm_blk<1, 0>(a, sm.Q0, LQ, sm.R1, LD, 16 * mb, nb, 0, kChunk, qg, cl);
        }
    __syncthreads();
    // ---------------- back to the prep layout ----------------
    float gQ[4][CPL], gKG[4][CPL], gKI[4][CPL], gKt[4][CPL];
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int nb = 16 * (w + 4 * t);
            st_blk(sm.R0, LD, 16 * mb, nb, dQG[t][mb], qg, cl);
            st_blk(sm.R1, LD, 16 * mb, nb, dKG[t][mb], qg, cl);
            st_blk(sm.R2, LD, 16 * mb, nb, dKI[t][mb], qg, cl);
        }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int o = (16 * w + 4 * qg + i) * LD + CPL * cl + e;
            gQ[i][e] = sm.R0[o];
            gKG[i][e] = sm.R1[o];
            gKI[i][e] = sm.R2[o];
        }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NBK; ++t)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) st_blk(sm.R0, LD, 16 * mb, 16 * (w + 4 * t), dKt[t][mb], qg, cl);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < CPL; ++e) gKt[i][e] = sm.R0[(16 * w + 4 * qg + i) * LD + CPL * cl + e];

    // ---------------- chain rule to qh, kh, beta, G ----------------
    float dqh[4][CPL], dkh[4][CPL], dG[4][CPL], dbk[4], colp[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) colp[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dbk[i] = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const float gam = fast_exp(G[i][e]), gin = fast_exp(-G[i][e]), ek = fast_exp(GC[e] - G[i][e]);
            const float QG = qh[i][e] * gam, KGv = beta[i] * kh[i][e] * gam, KIv = kh[i][e] * gin, Ktv = kh[i][e] * ek;
            dqh[i][e] = gQ[i][e] * gam;
            dkh[i][e] = beta[i] * gam * gKG[i][e] + gKI[i][e] * gin + gKt[i][e] * ek;
            dG[i][e] = gQ[i][e] * QG + gKG[i][e] * KGv - gKI[i][e] * KIv - gKt[i][e] * Ktv;
            dbk[i] += gKG[i][e] * kh[i][e] * gam;
            colp[e] += gKt[i][e] * Ktv;
        }
    }
    // column sums over the chunk of dKt * Ktil -> dL/dG_C
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        float s = colp[e];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (qg == 0) sm.red[w][CPL * cl + e] = s;
    }
    __syncthreads();
    float dGC[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        const int c = CPL * cl + e;
        dGC[e] = sm.red[0][c] + sm.red[1][c] + sm.red[2][c] + sm.red[3][c] + sm.dgc[c] * sm.gc[c];
    }
    __syncthreads();
    // dg = reverse cumulative sum of dG over the chunk, with dL/dG_C entering at the last row
    {
        float suf[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 3; i >= 0; --i) { a += dG[i][e]; dG[i][e] = a; }
            const float tot = a;
            float s = tot, x;
            x = __shfl_down(s, 16);
            if (qg <= 2) s += x;
            x = __shfl_down(s, 32);
            if (qg <= 1) s += x;
            suf[e] = s - tot;   // rows of later lane groups in this wave
            if (qg == 0) sm.red[w][CPL * cl + e] = s;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int c = CPL * cl + e;
            float a = suf[e] + dGC[e];
#pragma unroll
            for (int ww = 0; ww < 4; ++ww)
                if (ww > w) a += sm.red[ww][c];
#pragma unroll
            for (int i = 0; i < 4; ++i) dG[i][e] += a;
        }
    }
    // ---------------- through the L2 norms and the sigmoid; write ----------------
    TO* __restrict__ dqp = reinterpret_cast<TO*>(p.dq);
    TO* __restrict__ dkp = reinterpret_cast<TO*>(p.dk);
    TO* __restrict__ dgp = reinterpret_cast<TO*>(p.dg);
    TO* __restrict__ dbp = reinterpret_cast<TO*>(p.db);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * qg + i;
        float aq = 0.f, ak = 0.f, db = dbk[i];
#pragma unroll
        for (int e = 0; e < CPL; ++e) { aq += qh[i][e] * dqh[i][e]; ak += kh[i][e] * dkh[i][e]; }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) { aq += __shfl_xor(aq, m); ak += __shfl_xor(ak, m); db += __shfl_xor(db, m); }
        if (r < L) {
            const int64_t tok = c0 + r;
            const float sc = p.scale;
            // qh = scale * qbar: dL/dq = (scale * dqh - qbar (qbar . scale * dqh)) / nq
            const float iq = sc / nq[i], ik = 1.f / nk[i];
            const float qdot = sc != 0.f ? aq / (sc * sc) : 0.f;   // (qh . dqh) / scale^2
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int64_t off = (tok * H + h) * DK + CPL * cl + e;
                dqp[off] = from_f32<TO>(iq * (dqh[i][e] - qh[i][e] * qdot));
                dkp[off] = from_f32<TO>(ik * (dkh[i][e] - kh[i][e] * ak));
                dgp[off] = from_f32<TO>(dG[i][e]);
            }
            if (cl == 0) {
                const float dbeta = db + sm.dbv[0][r] + sm.dbv[1][r] + sm.dbv[2][r] + sm.dbv[3][r];
                dbp[tok * H + h] = from_f32<TO>(dbeta * dsig[i]);
            }
        }
    }
}

// ============================================================================
template <typename T, int DK>
static hipError_t launch_scan(const BwdParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if constexpr (std::is_same<T, bf16>::value)
        return launch_scan16(p, DK, s);   // fp16 matrix-core operands (kda_scan16.hip)
    else
        hipLaunchKernelGGL((kda_bwd_scan_kernel<T, DK>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename T, typename TO, int DK>
static hipError_t launch_chunk(const BwdParams& p, hipStream_t s) {
    const int64_t blocks = num_slots(p.T, p.N) * p.H;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if constexpr (std::is_same<T, float>::value) {
        if (p.dv == 128)
            hipLaunchKernelGGL((kda_bwd_chunk_f32_kernel<T, TO, DK, 128>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((kda_bwd_chunk_f32_kernel<T, TO, DK, 64>), grid, block, 0, s, p);
    } else {
        if (p.dv == 128)
            hipLaunchKernelGGL((kda_bwd_grads_kernel<TO, DK, 128>), grid, dim3(kWideThreads), 0, s, p);
        else
            hipLaunchKernelGGL((kda_bwd_grads_kernel<TO, DK, 64>), grid, dim3(kWideThreads), 0, s, p);
    }
    return hipGetLastError();
}

template <typename T, typename TO, int DK>
static hipError_t launch_bwd_t(const BwdParams& p, int stages, hipStream_t s) {
    if (stages & kBwdScan) {
        const hipError_t e = launch_scan<T, DK>(p, s);
        if (e != hipSuccess) return e;
    }
    if (stages & kBwdGrads) {
        const hipError_t e = launch_chunk<T, TO, DK>(p, s);
        if (e != hipSuccess) return e;
        // chunks past the factorised range are recomputed pair by pair (kda_exact.hip)
        return launch_bwd_exact(p, std::is_same<T, bf16>::value ? 1 : 0, std::is_same<TO, bf16>::value ? 1 : 0, DK,
                                true, s);
    }
    return hipSuccess;
}

hipError_t launch_bwd(const BwdParams& p, int in_dtype, int out_dtype, int dk, int stages, hipStream_t s) {
    if (in_dtype == 1) {
        if (dk == 128)
            return out_dtype == 1 ? launch_bwd_t<bf16, bf16, 128>(p, stages, s)
                                  : launch_bwd_t<bf16, float, 128>(p, stages, s);
        return out_dtype == 1 ? launch_bwd_t<bf16, bf16, 64>(p, stages, s) : launch_bwd_t<bf16, float, 64>(p, stages, s);
    }
    if (dk == 128) {
        // fp32 inputs at dk = 128: token-by-token reverse scan, pair-exact chunk gradients
        if (stages & kBwdScan) {
            const hipError_t e = launch_bwd_scan_token(p, in_dtype, dk, s);
            if (e != hipSuccess) return e;
        }
        if (stages & kBwdGrads) return launch_bwd_exact(p, in_dtype, out_dtype, dk, false, s);
        return hipSuccess;
    }
    return out_dtype == 1 ? launch_bwd_t<float, bf16, 64>(p, stages, s) : launch_bwd_t<float, float, 64>(p, stages, s);
}

}  // namespace kda
