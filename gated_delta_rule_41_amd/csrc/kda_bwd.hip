// kda_bwd.hip -- chunked KDA backward for gfx950.
//
// The pages ask the backward to reuse what the forward saved (normalisation
// statistics and states) and to join state-gradient propagation with the Q/K
// gradients ("TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and
// training practice", section "KDA pre/post-processing fusion").  Here:
//
//  B1  kda_bwd_scan_kernel: reverse state-gradient scan.  One persistent
//      workgroup per (sequence, head, 64-column value slice) walks the chunks
//      backwards with dL/dS (dk x 64, fp32) resident in MFMA accumulators:
//          dU  = Aqk^T dO + Ktil dS1
//          dS0 = Diag(Gam_C) dS1 + (qh Gam)^T dO - W^T dU
//      and writes dS1 (dL/dS at the end of every chunk) for B2.
//  B2  kda_bwd_chunk_kernel: chunk-parallel gradients.  One workgroup per
//      (chunk, head) recomputes the chunk's intra matrices, reads the saved
//      entering state S0 and dS1, and forms dq, dk, dv, dg, dbeta.
//
// Chunk equations (G the in-chunk cumulative log-decay, Gam = exp(G)):
//   QG = qh Gam, KG = beta kh Gam, KI = kh / Gam, Ktil = kh Gam_C / Gam
//   Akk = strict(KG KI^T), Aqk = lower(QG KI^T), T = (I + Akk)^{-1}
//   W = T KG, U = T beta v - W S0, O = QG S0 + Aqk U,
//   S1 = Diag(Gam_C) S0 + Ktil^T U
// and their reverse-mode derivatives (dAkk = -strict(T^T dT T^T), ...).
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

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
// Every matrix lives in LDS in fp32; an MFMA operand fragment (8 values along
// the contraction index) is gathered in whichever orientation the product
// needs, split into bf16 hi + lo, and contracted with three k32 MFMAs
// (hi.hi + hi.lo + lo.hi), which keeps about 16 mantissa bits per operand.

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

__device__ __forceinline__ void st_blk(float* M, int ld, int m0, int n0, f32x4 x, int qg, int cl) {
#pragma unroll
    for (int i = 0; i < 4; ++i) M[(m0 + 4 * qg + i) * ld + n0 + cl] = x[i];
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

// Find the sequence that owns state slot `slot` (slot = floor(cu[n]/64) + n + j).
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

template <typename T, typename TO, int DK, int DV>
__global__ __launch_bounds__(kThreads, 1) void kda_bwd_chunk_kernel(BwdParams p) {
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
    float qh[4][CPL], kh[4][CPL], G[4][CPL], vv[4][VPL], dov[4][VPL], beta[4], nq[4], nk[4];
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
                nq[i] = p.nq_saved[tok * H + h];     // norms saved by the forward
                nk[i] = p.nk_saved[tok * H + h];
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
                dbp[tok * H + h] = from_f32<TO>(dbeta * beta[i] * (1.f - beta[i]));
            }
        }
    }
}

// ============================================================================
template <typename T, int DK>
static hipError_t launch_scan(const BwdParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices)), block(kThreads);
    hipLaunchKernelGGL((kda_bwd_scan_kernel<T, DK>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <typename T, typename TO, int DK>
static hipError_t launch_chunk(const BwdParams& p, hipStream_t s) {
    const int64_t blocks = num_slots(p.T, p.N) * p.H;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (p.dv == 128)
        hipLaunchKernelGGL((kda_bwd_chunk_kernel<T, TO, DK, 128>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((kda_bwd_chunk_kernel<T, TO, DK, 64>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <typename T, typename TO, int DK>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t s) {
    hipError_t e = launch_scan<T, DK>(p, s);
    if (e != hipSuccess) return e;
    return launch_chunk<T, TO, DK>(p, s);
}

hipError_t launch_bwd(const BwdParams& p, int in_dtype, int out_dtype, int dk, hipStream_t s) {
    if (in_dtype == 1) {
        if (dk == 128)
            return out_dtype == 1 ? launch_bwd_t<bf16, bf16, 128>(p, s) : launch_bwd_t<bf16, float, 128>(p, s);
        return out_dtype == 1 ? launch_bwd_t<bf16, bf16, 64>(p, s) : launch_bwd_t<bf16, float, 64>(p, s);
    }
    return out_dtype == 1 ? launch_bwd_t<float, bf16, 64>(p, s) : launch_bwd_t<float, float, 64>(p, s);
}

}  // namespace kda
