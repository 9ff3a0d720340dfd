// kda_fwd.hip -- fused chunked KDA forward for fp32 inputs on gfx950 (fp32
// matrix-core operands; bf16 inputs use kda_fwd16.hip).
//
// One persistent workgroup per (sequence, head, 64-wide slice of the value
// dimension) walks the sequence chunk by chunk (64 tokens).  The dk x 64 fp32
// state slice never leaves the MFMA accumulators; each chunk does, on chip:
//
//   prep   qh, kh = L2-normalised q, k; beta = sigmoid(b); G = inclusive
//          in-chunk cumulative sum of g (per key channel); Gam = exp(G)
//   intra  Akk = strict_lower(beta kh Gam (kh/Gam)^T), Aqk = lower(qh Gam (kh/Gam)^T)
//          [W | Ut] = (I + Akk)^{-1} [beta kh Gam | beta v]   (blocked solve)
//   inter  U = Ut - W S ; O = (qh Gam) S + Aqk U ;
//          S <- Diag(Gam_C) S + (kh Gam_C/Gam)^T U
//
// which is the gated delta rule unrolled over the chunk: the pages organise
// KDA as intra-chunk processing plus inter-chunk state passing with the Q/K
// normalisation, beta transform and gating fused into the forward
// ("TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
// practice", section "KDA pre/post-processing fusion"), and fuse the stages
// into one kernel to avoid intermediate HBM round trips ("Ascend implements
// LoRA training of Kimi K3.1 Pro", section "KDA: big fused forward and
// backward").  Only the inputs are read and only o (plus, for training, the
// per-chunk entering states and the q/k norms) are written.
//
// Work split inside the workgroup (4 waves):
//   prep   wave w owns chunk rows 16w..16w+15; lane (qg, cl) holds rows
//          16w+4qg+i (i=0..3) and key columns [CPL*cl, CPL*cl+CPL).
//   intra  20 lower-triangular 16x16 blocks of Akk and Aqk, 5 per wave;
//          wave w inverts diagonal block w of I+Akk by forward substitution;
//          the blocked solve gives wave w the columns it owns.
//   inter  wave w owns value columns 16w..16w+15 of the slice: its state
//          columns, U columns and O columns stay in its registers.
#include <cstddef>
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"
#include "kda_token.h"

namespace kda {

template <typename T, int DK>
struct __attribute__((aligned(32))) FwdSmem {
    // bf16 operands carry a second "lo" tile (x - bf16(x)) wherever the
    // rounding of a single bf16 operand is visible in the output (see SPLIT).
    static constexpr bool SPLIT = std::is_same<T, bf16>::value;
    static constexpr int PK = DK + 8;        // row stride of [64][DK] tiles
    static constexpr int PC = kChunk + 8;    // row stride of [*][64] tiles
    static constexpr int RK = kChunk * PK;
    static constexpr int RT = DK * PC;
    static constexpr int RG = RK > RT ? RK : RT;
    T qg[RK];                 // qh*Gam                       [r][perm32(c)]
    T qgl[SPLIT ? RK : 16];   //   lo part
    T kg[RK];                 // beta*kh*Gam                  [r][perm32(c)]
    T ki[RK];                 // kh/Gam; after intra: -W      [r][perm32(c)]
    T kil[SPLIT ? RG : 16];   // kh/Gam lo; after intra: Ktil^T lo
    T kt[RT];                 // Ktil^T = (kh*Gam_C/Gam)^T    [c][perm32(r)]
    T aqk[kChunk * PC];       // lower(Aqk)                   [r][perm32(s)]
    T aqkl[SPLIT ? kChunk * PC : 16];
    T akk[kChunk * PC];       // strict_lower(Akk)            [r][s]
    T vt[kSlice * PC];        // v transposed (input values)  [c][r]
    float beta[kChunk];
    float adiag[4][16][20];   // diagonal blocks of Akk (fp32)
    float tdiag[4][16][20];   // (I + Akk_bb)^{-1}
    float gc[DK];             // Gam_C
    float red[4][DK];         // per-wave column sums of g
};

// Row stride (floats) of a state wave's 64 x 16 O patch staged for the stores
// (rows 16-byte aligned).  Two patches fit in the Akk tile and two in the
// diagonal-block arrays.
constexpr int kOStride = 16;
static_assert(2 * kChunk * kOStride * 4 <= kChunk * (kChunk + 8) * 2, "O patches exceed the Akk tile");
static_assert(2 * kChunk * kOStride * 4 <= 2 * 4 * 16 * 20 * 4, "O patches exceed the diagonal-block arrays");

template <typename T, typename TO, int DK, bool SAVE>
__global__ __launch_bounds__(kThreads, 1) void kda_fwd_kernel(FwdParams p) {
    __shared__ FwdSmem<T, DK> sm;
    typedef FwdSmem<T, DK> SM;
    constexpr bool SPLIT = SM::SPLIT;
    constexpr int PK = SM::PK;
    constexpr int PC = SM::PC;
    constexpr int CPL = DK / 16;    // key columns per lane (prep layout)
    constexpr int VPL = kSlice / 16;
    constexpr int NKB = DK / 32;    // k32 steps over dk
    constexpr int NMB = DK / 16;    // 16-row blocks of the state
    constexpr int NWB = DK / 64;    // W column blocks per wave in the solve
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
    const int vcol = dv0 + 16 * w + cl;   // value column owned by this lane in the inter phase

    const T* __restrict__ qp = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kp = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vp = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gp = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bp = reinterpret_cast<const T*>(p.b);
    TO* __restrict__ op = reinterpret_cast<TO*>(p.o);

    // ---- state slice in accumulator layout: S[mb][i] = S[16mb+4qg+i][vcol]
    const int64_t sbase = ((int64_t)n * H + h) * DK * dv;
    f32x4 S[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[mb][i] = p.s0 ? p.s0[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + vcol] : 0.f;

    // ---- raw chunk registers (prefetched one chunk ahead, kept in input format)
    RawRow<T, CPL> rq[4], rk[4], rg[4];
    RawRow<T, VPL> rv[4];
    RawScalar<T> rb[4];
    const int64_t rs_k = (int64_t)H * DK, rs_v = (int64_t)H * dv;   // token strides
    auto load_chunk = [&](int64_t c0) {
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);
        const int r0 = 16 * w + 4 * qg;
        const T* qc = qp + (c0 + r0) * rs_k + h * DK + CPL * cl;
        const T* kc = kp + (c0 + r0) * rs_k + h * DK + CPL * cl;
        const T* gc = gp + (c0 + r0) * rs_k + h * DK + CPL * cl;
        const T* vc = vp + (c0 + r0) * rs_v + h * dv + dv0 + VPL * cl;
        const T* bc = bp + (c0 + r0) * H + h;
        if (r0 + 4 <= L) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rq[i].load(qc + i * rs_k);
                rk[i].load(kc + i * rs_k);
                rg[i].load(gc + i * rs_k);
                rv[i].load(vc + i * rs_v);
                rb[i].load(bc + i * H);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (r0 + i < L) {
                    rq[i].load(qc + i * rs_k);
                    rk[i].load(kc + i * rs_k);
                    rg[i].load(gc + i * rs_k);
                    rv[i].load(vc + i * rs_v);
                    rb[i].load(bc + i * H);
                } else {
                    rq[i].zero(); rk[i].zero(); rg[i].zero(); rv[i].zero();
                    rb[i].zero();
                }
            }
        }
    };
    if (t0 < t1) load_chunk(t0);
    // The k32 steps of Aqk U read the upper 16x16 blocks (0,1) and (2,3) of the
    // Aqk tiles, which no chunk writes: clear them once.  (The first barrier
    // inside the chunk loop orders this before any read.)
    for (int e = tid; e < kChunk * PC; e += kThreads) {
        sm.aqk[e] = from_f32<T>(0.f);
        if constexpr (SPLIT) sm.aqkl[e] = from_f32<T>(0.f);
    }

    int64_t slot = t0 / kChunk + n;
    for (int64_t c0 = t0; c0 < t1; c0 += kChunk, ++slot) {
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);

        // ================= prep (registers) =================
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
            beta[i] = (r < L) ? 1.f / (1.f + fast_exp(-rb[i].f())) : 0.f;
        }
        // inclusive cumulative sum of g over the chunk rows, in log2 units
        float G[4][CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            float a = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { a += rg[i][e] * kLog2e; G[i][e] = a; }
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
            for (int e = 0; e < CPL; ++e) sm.gc[CPL * cl + e] = fast_exp2(GC[e]);
        }
        if (cl == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.beta[16 * w + 4 * qg + i] = beta[i];
        }
        if (SAVE && slice == 0 && cl == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * qg + i;
                if (r < L) {
                    p.nq_saved[(int64_t)h * p.T + c0 + r] = nq[i];   // head-major [H, T]
                    p.nk_saved[(int64_t)h * p.T + c0 + r] = nk[i];
                }
            }
        }
        {
            // decay past the factorised range: the recurrence token by token
            // (every wave holds every channel's sum, so the branch is uniform)
            bool tok = false;
#pragma unroll
            for (int e = 0; e < CPL; ++e) tok |= !(GC[e] >= kTokenBelow * kLog2e);
            if (__builtin_amdgcn_ballot_w64(tok) != 0) {
                if (c0 + kChunk < t1) load_chunk(c0 + kChunk);
                if (SAVE) {
                    float* st = reinterpret_cast<float*>(p.st_saved) + (slot * H + h) * (int64_t)DK * dv;
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) st[(int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = S[mb][i];
                }
                const TokSrc<T> src = {qp, kp, gp, bp, vp, H, h, dv, vcol, qg, p.eps, p.scale};
                token_fwd<T, TO, DK>(S, src, c0, L, op, nullptr, nullptr, false);
                __syncthreads();
                continue;
            }
        }
        // operand tiles: qh Gam, beta kh Gam, kh / Gam
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * qg + i;
            const float aq = p.scale / nq[i], ai = 1.f / nk[i], ak = beta[i] * ai;
#pragma unroll
            for (int e4 = 0; e4 < CPL; e4 += 4) {
                f32x4 vq, vk, vi;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = e4 + j;
                    const float gam = fast_exp2(G[i][e]);
                    const float gin = fast_exp2(-G[i][e]);
                    vq[j] = (rq[i][e] * aq) * gam;
                    vk[j] = (rk[i][e] * ak) * gam;
                    vi[j] = (rk[i][e] * ai) * gin;
                }
                const int pc = perm32(CPL * cl + e4);
                sts4_split<T, SPLIT>(&sm.qg[r * PK + pc], &sm.qgl[SPLIT ? r * PK + pc : 0], vq);
                sts4<T>(&sm.kg[r * PK + pc], vk);
                sts4_split<T, SPLIT>(&sm.ki[r * PK + pc], &sm.kil[SPLIT ? r * PK + pc : 0], vi);
            }
        }
#pragma unroll
        for (int e = 0; e < VPL; ++e) {
            f32x4 x = {rv[0][e], rv[1][e], rv[2][e], rv[3][e]};
            sts4<T>(&sm.vt[(VPL * cl + e) * PC + 16 * w + 4 * qg], x);   // exact: v is an input value
        }
        // the raw registers are free: fetch the next chunk while this one computes
        if (c0 + kChunk < t1) load_chunk(c0 + kChunk);
        __syncthreads();

        // ================= intra: Akk, Aqk =================
        {
#pragma unroll 1
            for (int st = 0; st < 5; ++st) {
                const int it = w + 4 * st;          // 0..9: Akk blocks, 10..19: Aqk blocks
                const bool isqk = it >= 10;
                const int pi = isqk ? it - 10 : it;  // lower-triangle block index
                const int ib = pi >= 6 ? 3 : (pi >= 3 ? 2 : (pi >= 1 ? 1 : 0));
                const int jb = pi - (ib * (ib + 1)) / 2;
                const int ra = (16 * ib + cl) * PK + 8 * qg, rbk = (16 * jb + cl) * PK + 8 * qg;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (isqk) {
#pragma unroll
                    for (int kk = 0; kk < NKB; ++kk) {
                        const V8T ah = lds8<T>(sm.qg + ra + 32 * kk), bh = lds8<T>(sm.ki + rbk + 32 * kk);
                        if constexpr (SPLIT)
                            acc = mma3<true>(acc, ah, lds8<T>(sm.qgl + ra + 32 * kk), bh, lds8<T>(sm.kil + rbk + 32 * kk));
                        else
                            acc = mma_k32(acc, ah, bh);
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < NKB; ++kk)
                        acc = mma_k32(acc, lds8<T>(sm.kg + ra + 32 * kk), lds8<T>(sm.ki + rbk + 32 * kk));
                }
                const int s = 16 * jb + cl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * ib + 4 * qg + i;
                    if (isqk) {
                        const float val = s <= r ? acc[i] : 0.f;
                        const T hi = from_f32<T>(val);
                        sm.aqk[r * PC + perm32(s)] = hi;
                        if constexpr (SPLIT) sm.aqkl[r * PC + perm32(s)] = from_f32<T>(val - to_f32(hi));
                    } else {
                        const float val = s < r ? acc[i] : 0.f;
                        sm.akk[r * PC + s] = from_f32<T>(val);
                        if (ib == jb) sm.adiag[ib][4 * qg + i][cl] = val;
                    }
                }
            }
        }
        // Ktil = kh Gam_C / Gam = (kh/Gam) * Gam_C, from the hi+lo tiles (read
        // before the barrier: the lo tile is overwritten right after it)
        float ktv[CPL][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * w + 4 * qg + i;
#pragma unroll
            for (int e4 = 0; e4 < CPL; e4 += 4) {
                const int pc = perm32(CPL * cl + e4);
                f32x4 x = lds4f<T>(&sm.ki[r * PK + pc]);
                if constexpr (SPLIT) x += lds4f<T>(&sm.kil[r * PK + pc]);
                const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[CPL * cl + e4]);
#pragma unroll
                for (int j = 0; j < 4; ++j) ktv[e4 + j][i] = x[j] * gcv[j];
            }
        }
        __syncthreads();

        // ======== (I + Akk_ww)^{-1} for diagonal block w ========
        {
            const f32x4 na = *reinterpret_cast<const f32x4*>(&sm.adiag[w][cl][4 * qg]);
            f32x4 nb;
#pragma unroll
            for (int j = 0; j < 4; ++j) nb[j] = sm.adiag[w][4 * qg + j][cl];
            const f32x4 tw = inv_unit_lower16(na, nb, qg, cl);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.tdiag[w][4 * qg + i][cl] = tw[i];
        }
        // Ktil^T tiles: the lo part goes where kh/Gam lo lived (read only by intra)
        {
            const int pr = perm32(16 * w + 4 * qg);
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                f32x4 x = {ktv[e][0], ktv[e][1], ktv[e][2], ktv[e][3]};
                sts4_split<T, SPLIT>(&sm.kt[(CPL * cl + e) * PC + pr], &sm.kil[SPLIT ? (CPL * cl + e) * PC + pr : 0], x);
            }
        }
        __syncthreads();

        // ======== blocked solve [W | Ut] = (I + Akk)^{-1} [beta kh Gam | beta v] ========
        // X_i = T_ii (B_i - sum_{j<i} Akk_ij X_j), per 16-column block owned by this wave.
        f32x4 U[4];
        {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            V4T tii[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) tii[i] = pack4<T>(*reinterpret_cast<const f32x4*>(&sm.tdiag[i][cl][4 * qg]));
#pragma unroll
            for (int cb = 0; cb <= NWB; ++cb) {
                const bool isw = cb < NWB;
                const int nb = 16 * (w + 4 * cb);    // W: key column block; Ut: value block
                f32x4 X[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f32x4 acc;
                    if (isw) {
                        const int pc = perm32(nb + cl);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[j] = to_f32(sm.kg[(16 * i + 4 * qg + j) * PK + pc]);
                    } else {
                        const f32x4 vv = lds4f<T>(&sm.vt[(16 * w + cl) * PC + 16 * i + 4 * qg]);
                        const f32x4 bb = *reinterpret_cast<const f32x4*>(&sm.beta[16 * i + 4 * qg]);
                        acc = vv * bb;   // beta v, exact in fp32
                    }
#pragma unroll
                    for (int jp = 0; jp < i; ++jp)
                        acc = mma_k16(acc, neg4(lds4<T>(&sm.akk[(16 * i + cl) * PC + 16 * jp + 4 * qg])),
                                      pack4<T>(X[jp]));
                    const V4T ah = pack4<T>(acc);
                    X[i] = mma_k16(zero, tii[i], ah);
                    if constexpr (SPLIT) {
                        if (!isw) X[i] = mma_k16(X[i], tii[i], pack4<T>(acc - unpack4(ah)));
                    }
                }
                if (isw) {
                    const int pc = perm32(nb + cl);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 4; ++j) sm.ki[(16 * i + 4 * qg + j) * PK + pc] = from_f32<T>(-X[i][j]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) U[i] = X[i];
                }
            }
        }
        __syncthreads();

        // ================= inter-chunk: U, O, S =================
        V8T sfh[NKB], sfl[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) split8<T, SPLIT>(S[2 * kk], S[2 * kk + 1], sfh[kk], sfl[kk]);
        if (SAVE) {
            // entering state of this chunk, fp32 (the backward's state-coupled
            // gradient terms need more than bf16 precision)
            float* st = reinterpret_cast<float*>(p.st_saved) + (slot * H + h) * (int64_t)DK * dv;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[(int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = S[mb][i];
        }
        // U = Ut - W S   (the tile holds -W)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk)
                U[i] = mma_k32(U[i], lds8<T>(sm.ki + (16 * i + cl) * PK + 32 * kk + 8 * qg), sfh[kk]);
        V8T ufh[2], ufl[2];
        split8<T, SPLIT>(U[0], U[1], ufh[0], ufl[0]);
        split8<T, SPLIT>(U[2], U[3], ufh[1], ufl[1]);
        // O = (qh Gam) S + Aqk U
#pragma unroll 2
        for (int i = 0; i < 4; ++i) {
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
            const int ro = (16 * i + cl) * PK + 8 * qg, ra = (16 * i + cl) * PC + 8 * qg;
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk)
                O = mma3<SPLIT>(O, lds8<T>(sm.qg + ro + 32 * kk), lds8<T>(sm.qgl + (SPLIT ? ro + 32 * kk : 0)),
                                sfh[kk], sfl[kk]);
#pragma unroll
            for (int kk = 0; kk <= (i >> 1); ++kk)
                O = mma3<SPLIT>(O, lds8<T>(sm.aqk + ra + 32 * kk), lds8<T>(sm.aqkl + (SPLIT ? ra + 32 * kk : 0)),
                                ufh[kk], ufl[kk]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * i + 4 * qg + j;
                if (r < L) op[((c0 + r) * H + h) * dv + vcol] = from_f32<TO>(O[j]);
            }
        }
        // S <- Diag(Gam_C) S + (kh Gam_C / Gam)^T U
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[16 * mb + 4 * qg]);
            S[mb] *= gcv;
            const int rt = (16 * mb + cl) * PC + 8 * qg;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                S[mb] = mma3<SPLIT>(S[mb], lds8<T>(sm.kt + rt + 32 * kk), lds8<T>(sm.kil + (SPLIT ? rt + 32 * kk : 0)),
                                    ufh[kk], ufl[kk]);
        }
        __syncthreads();
    }

    if (p.sfinal) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) p.sfinal[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = S[mb][i];
    }
}

template <typename T, typename TO, int DK>
static hipError_t launch_fwd_t(const FwdParams& p, bool save, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if (save)
        hipLaunchKernelGGL((kda_fwd_kernel<T, TO, DK, true>), grid, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((kda_fwd_kernel<T, TO, DK, false>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd_maps(const FwdParams& p, int dk, hipStream_t s) { return launch_fwd16_maps(p, dk, s); }

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int out_dtype, int dk, bool save,
                      hipStream_t s) {
    if (in_dtype == 1) return launch_fwd16(p, out_dtype, dk, save, s);
    // fp32 inputs: fp32 MFMA at dk = 64; at dk = 128 (whose fp32 tiles exceed
    // LDS) the recurrence token by token (kda_exact.hip)
    if (dk == 128) return launch_fwd_token(p, in_dtype, out_dtype, dk, save, s);
    return out_dtype == 1 ? launch_fwd_t<float, bf16, 64>(p, save, s)
                          : launch_fwd_t<float, float, 64>(p, save, s);
}

}  // namespace kda
