// kda_fwd.hip -- fused chunked KDA forward for gfx950.
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
                    p.nq_saved[(c0 + r) * H + h] = nq[i];
                    p.nk_saved[(c0 + r) * H + h] = nk[i];
                }
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

// ============================================================================
// bf16 inputs: 8 waves in two groups of four.
//
// The state-coupled work of chunk n (U, O, the state update) runs on the four
// "state" waves, which own the value columns as in the kernel above.  The
// per-element preparation of chunk n+1 (norms, sigmoid, gate cumsum, exp2, the
// hi/lo operand values) is split by key columns: the four "prep" waves take the
// first half and the state waves the second, so the state waves' VALU work
// fills their MFMA and LDS latency; each group also issues the loads of chunk
// n+2 for its half.  The two halves' partial row norms meet in LDS.  The
// intra-chunk products, the diagonal inverses and the blocked solve are shared.
//
// MAP = true is the first level of the two-level forward for long sequences:
// each "sequence" is a segment, and the workgroup computes a slice of the
// segment's affine map S_out = M S_in + B.  The state is [M | B] (dk x
// (dk + dv)): slices [0, dk/64) start from the identity with zero values and
// give M, the others start from zero with the real values and give B.  Nothing
// but that state is written.
// ============================================================================
template <typename TO, int DK, bool SAVE, bool MAP>
__global__ __launch_bounds__(kWideThreads, 1) void kda_fwd_bf16_kernel(FwdParams p) {
    typedef bf16 T;
    __shared__ FwdSmem<T, DK> sm;
    __shared__ float snrm[2][2][kChunk];   // [half][q, k][row]: partial sums of squares
    typedef FwdSmem<T, DK> SM;
    constexpr int PK = SM::PK;
    constexpr int PC = SM::PC;
    constexpr int CPH = DK / 32;    // key columns per lane: half a row per group (prep layout)
    constexpr int VPL = kSlice / 16;
    constexpr int NKB = DK / 32;    // k32 steps over dk
    constexpr int NMB = DK / 16;    // 16-row blocks of the state
    typedef bf16x8 V8T;
    typedef bf16x4 V4T;
    typedef __bf16 VH __attribute__((ext_vector_type(CPH)));   // one lane's half-row of bf16 values

    const int tid = threadIdx.x, w = tid >> 6;
    // Lane coordinates.  refresh() hides the lane index from the optimiser at
    // the top of every step, so the addresses and masks derived from it are
    // recomputed per step instead of being held in registers across the loop.
    int l = tid & 63, qg = l >> 4, cl = l & 15;
    const bool is_state = w < 4;      // wave-uniform
    const int ww = w & 3;             // index inside the group
    const int hf = is_state ? 1 : 0;  // key-column half this wave prepares
    int chain, slice;
    map_block(blockIdx.x, p.N * p.H, p.nslices, chain, slice);
    const int n = chain / p.H, h = chain % p.H;
    int64_t t0, t1;
    seq_bounds(p.cu, n, p.seqlen, p.T, t0, t1);
    const int dv = p.dv, H = p.H;
    const bool mslice = MAP && slice < p.map_slices;           // this slice carries M
    const int dv0 = MAP ? (mslice ? 0 : (slice - p.map_slices) * kSlice) : slice * kSlice;
    const int ld = MAP ? DK + dv : dv;                         // row stride of the state arrays
    const int sc0 = MAP ? slice * kSlice : dv0;                // first state column of the slice
    int vcol = dv0 + 16 * ww + cl;   // value column of a state-wave lane
    int scol = sc0 + 16 * ww + cl;   // its state column

    const T* __restrict__ qp = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kp = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vp = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gp = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bp = reinterpret_cast<const T*>(p.b);
    TO* __restrict__ op = reinterpret_cast<TO*>(p.o);
    const int64_t rs_k = (int64_t)H * DK, rs_v = (int64_t)H * dv;   // token strides

    // ---------------- prep layout: rows 16ww+4qg+i, key columns ck0..ck0+CPH-1
    int r0 = 16 * ww + 4 * qg;
    int ck0 = hf * (DK / 2) + CPH * cl;
    int pc0 = perm32(ck0);                  // their (contiguous) tile position
    auto refresh = [&]() {
        asm volatile("" : "+v"(l));
        qg = l >> 4;
        cl = l & 15;
        vcol = dv0 + 16 * ww + cl;
        scol = sc0 + 16 * ww + cl;
        r0 = 16 * ww + 4 * qg;
        ck0 = hf * (DK / 2) + CPH * cl;
        pc0 = perm32(ck0);
    };
    RawRow<T, CPH> rq[4], rk[4], rg[4];     // raw rows of the chunk being prepared
    RawRow<T, VPL> rv[4];                   // (prep waves) its v slice
    RawScalar<T> rb[4];
    float nq[4], nk[4], beta[4];
    int Lp = 0;                             // valid rows of the chunk being prepared
    VH xkil[4];                             // kh/Gam lo of the next chunk to run
    float xgc[CPH];                         // Gam_C of the next chunk to run

    // The rows of a chunk load in three parts (0: q and beta, 1: k, 2: g and the
    // v slice), issued in different steps: a wave stalls at issue while its
    // memory queue is full, so one burst of every load left the end of the
    // chunk waiting behind it.  load_chunk issues all three.
    auto load_part = [&](int64_t c0, int part) {
        // the maps (no queries, no outputs) measured faster with one burst
        if constexpr (MAP) {
            if (part != 0) return;
        }
        const bool p0 = MAP || part == 0, p1 = MAP || part == 1, p2 = MAP || part == 2;
        const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);
        // uniform chunk bases (scalar registers) + 32-bit per-lane offsets
        const T* qc = qp + c0 * rs_k + h * DK;
        const T* kc = kp + c0 * rs_k + h * DK;
        const T* gc = gp + c0 * rs_k + h * DK;
        const T* vc = vp + c0 * rs_v + h * dv + dv0;
        const T* bc = bp + c0 * H + h;
        const int sk = (int)rs_k, sv = (int)rs_v;
        // Rows past the chunk end load the last row (in bounds) and are zeroed
        // where they are first used (prep_a): no branch around the loads, and
        // 32-bit unsigned offsets from the uniform bases.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rc = min(r0 + i, L - 1);
            const unsigned okr = (unsigned)(rc * sk + ck0);
            if (p0) {
                if (MAP) rq[i].zero();   // the maps need no queries
                else rq[i].load(at32(qc, okr));
                rb[i].load(at32(bc, (unsigned)(rc * H)));
            }
            if (p1) rk[i].load(at32(kc, okr));
            if (p2) {
                rg[i].load(at32(gc, okr));
                if (!is_state) {
                    if (mslice) rv[i].zero();
                    else rv[i].load(at32(vc, (unsigned)(rc * sv + VPL * cl)));
                }
            }
        }
        if (p0) Lp = L;
    };
    auto load_chunk = [&](int64_t c0) { load_part(c0, 0); load_part(c0, 1); load_part(c0, 2); };
    // In-wave inclusive prefix of the gates over the wave's 16 rows, for key
    // column ck0+e: one k16 MFMA of the lower-triangular ones matrix with the raw
    // bf16 gates, which already sit in B-fragment layout (lane (qg, cl) holds
    // rows 4qg..4qg+3 of the column).  Exact products, fp32 sums; the result
    // comes back in the same rows.
    auto gate_prefix = [&](int e) {
        V4T ltri;
#pragma unroll
        for (int j = 0; j < 4; ++j) ltri[j] = from_f32<T>(4 * qg + j <= cl ? 1.f : 0.f);
        const V4T b = __builtin_bit_cast(V4T, u16x4{rg[0].x[e], rg[1].x[e], rg[2].x[e], rg[3].x[e]});
        return mma_k16(f32x4{0.f, 0.f, 0.f, 0.f}, ltri, b);
    };
    // first half of the prep: this half's sums of squares, sigmoid, the wave's
    // gate column sums
    auto prep_a = [&]() {
        if (Lp < kChunk) {   // uniform: the last chunk of a document zeroes its rows past the end
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = r0 + i < Lp;
                rq[i].keep(ok); rk[i].keep(ok); rg[i].keep(ok);
                if (!is_state) rv[i].keep(ok);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < CPH; ++e) { sq += rq[i][e] * rq[i][e]; sk += rk[i][e] * rk[i][e]; }
            sq = row16_sum(sq);
            sk = row16_sum(sk);
            if (cl == 0) { snrm[hf][0][r0 + i] = sq; snrm[hf][1][r0 + i] = sk; }
            beta[i] = (r0 + i < Lp) ? __builtin_amdgcn_rcpf(1.f + fast_exp(-rb[i].f())) : 0.f;
        }
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            const f32x4 g4 = gate_prefix(e);
            if (qg == 3) sm.red[ww][ck0 + e] = g4[3];   // row 15: the wave's column sum
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) { rq[i].fence(); rk[i].fence(); rg[i].fence(); }
    };
    // second half (after both groups' partial sums are in LDS): norms, G and the
    // operand values.  kh/Gam lo and Gam_C stay in registers until the chunk's
    // first step (the state waves still read those tiles while this runs); every
    // other tile is written now.
    auto prep_b = [&](int64_t c0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // reciprocal norms (v_rsq, ~1 ulp); halves summed in a fixed order
            nq[i] = __builtin_amdgcn_rsqf(snrm[0][0][r0 + i] + snrm[1][0][r0 + i] + p.eps);
            nk[i] = __builtin_amdgcn_rsqf(snrm[0][1][r0 + i] + snrm[1][1][r0 + i] + p.eps);
        }
        f32x4 G[CPH];   // G[e][i]: gate cumsum (log2 units) at row r0+i, column ck0+e
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            const int c = ck0 + e;
            float a = 0.f, tot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const float x = sm.red[w2][c];
                if (w2 < ww) a += x;
                tot += x;
            }
            xgc[e] = fast_exp2(tot * kLog2e);
            const f32x4 g4 = gate_prefix(e);
#pragma unroll
            for (int i = 0; i < 4; ++i) G[e][i] = (g4[i] + a) * kLog2e;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + i;
            const float aq = p.scale * nq[i], ai = nk[i], ak = beta[i] * ai;
            float vq[CPH], vk[CPH], vi[CPH];
#pragma unroll
            for (int e = 0; e < CPH; ++e) {
                const float gam = fast_exp2(G[e][i]);
                const float gin = fast_exp2(-G[e][i]);
                vq[e] = (rq[i][e] * aq) * gam;
                vk[e] = (rk[i][e] * ak) * gam;
                vi[e] = (rk[i][e] * ai) * gin;
            }
            VH qh, ql, kg, kih;
            split_n<CPH>(vq, qh, ql);
            split_n<CPH>(vi, kih, xkil[i]);
#pragma unroll
            for (int e = 0; e < CPH; ++e) kg[e] = from_f32<T>(vk[e]);
            if (!MAP) {
                *reinterpret_cast<VH*>(&sm.qg[r * PK + pc0]) = qh;
                *reinterpret_cast<VH*>(&sm.qgl[r * PK + pc0]) = ql;
            }
            *reinterpret_cast<VH*>(&sm.kg[r * PK + pc0]) = kg;
            *reinterpret_cast<VH*>(&sm.ki[r * PK + pc0]) = kih;
        }
        if (!is_state) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + i;
                if (cl == 0) sm.beta[r] = beta[i];
                if (SAVE && slice == 0 && cl == 0 && r < Lp) {
                    const int64_t nb = c0 * H + h;   // uniform base; the row offset r*H fits in 32 bits
                    p.nq_saved[nb + r * H] = __builtin_amdgcn_rcpf(nq[i]);
                    p.nk_saved[nb + r * H] = __builtin_amdgcn_rcpf(nk[i]);
                }
            }
            static_assert(VPL == 4, "v slice: four columns per lane");
#pragma unroll
            for (int e = 0; e < VPL; ++e)   // v is an input value: its bits move as they are
                *reinterpret_cast<V4T*>(&sm.vt[kt_off(VPL * cl + e, r0)]) = col4(rv[0].x, rv[1].x, rv[2].x, rv[3].x, e);
        }
    };
    // step 1 (both groups): the tiles held in registers
    auto store_held = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<VH*>(&sm.kil[(r0 + i) * PK + pc0]) = xkil[i];
        if (ww == 0 && qg == 0) {
#pragma unroll
            for (int e = 0; e < CPH; ++e) sm.gc[ck0 + e] = xgc[e];
        }
    };
    // step 3 (both groups): Ktil^T = (kh Gam_C / Gam)^T from the kh/Gam hi+lo values
    // of this half; its lo tile goes where kh/Gam lo lived (read only by step 2)
    auto store_ktil = [&]() {
        const int pr = perm32(r0);
        f32x4 kv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const VH hv = *reinterpret_cast<const VH*>(&sm.ki[(r0 + i) * PK + pc0]);
#pragma unroll
            for (int e = 0; e < CPH; ++e) kv[i][e] = to_f32(hv[e]) + to_f32(xkil[i][e]);
        }
#pragma unroll
        for (int e = 0; e < CPH; ++e) {
            const int c = ck0 + e;
            f32x4 x = {kv[0][e] * xgc[e], kv[1][e] * xgc[e], kv[2][e] * xgc[e], kv[3][e] * xgc[e]};
            sts4_split<T, true>(&sm.kt[kt_off(c, pr)], &sm.kil[kt_off(c, pr)], x);
        }
    };

    // The k32 steps of Aqk U read the upper 16x16 blocks (0,1) and (2,3) of the
    // Aqk tiles, which no chunk writes: clear them once.  (The first barrier
    // inside the chunk loop orders this before any read.)
    for (int e = tid; e < kChunk * PC; e += kWideThreads) {
        sm.aqk[e] = from_f32<T>(0.f);
        sm.aqkl[e] = from_f32<T>(0.f);
    }

    // step 2, shared by both groups: Akk and Aqk, one lower-triangle block pair per item
    auto intra_products = [&]() {
#pragma unroll 1
        for (int it = w; it < 10; it += 8) {
            const int ib = it >= 6 ? 3 : (it >= 3 ? 2 : (it >= 1 ? 1 : 0));
            const int jb = it - (ib * (ib + 1)) / 2;
            const int ra = (16 * ib + cl) * PK + 8 * qg, rbk = (16 * jb + cl) * PK + 8 * qg;
            f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk) {
                const V8T bh = lds8<T>(sm.ki + rbk + 32 * kk);
                akk = mma_k32(akk, lds8<T>(sm.kg + ra + 32 * kk), bh);
                if (!MAP)
                    aqk = mma3<true>(aqk, lds8<T>(sm.qg + ra + 32 * kk), lds8<T>(sm.qgl + ra + 32 * kk), bh,
                                     lds8<T>(sm.kil + rbk + 32 * kk));
            }
            const int s = 16 * jb + cl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * ib + 4 * qg + i;
                if (!MAP) {
                    const float vq = s <= r ? aqk[i] : 0.f;
                    const T hi = from_f32<T>(vq);
                    sm.aqk[kt_off(r, perm32(s))] = hi;
                    sm.aqkl[kt_off(r, perm32(s))] = from_f32<T>(vq - to_f32(hi));
                }
                const float vk = s < r ? akk[i] : 0.f;
                sm.akk[r * PC + s] = from_f32<T>(vk);
                if (ib == jb) sm.adiag[ib][4 * qg + i][cl] = vk;
            }
        }
    };
    // diagonal inverses of I + Akk as bf16 k16 A fragments
    auto load_tii = [&](V4T (&tii)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) tii[i] = pack4<T>(*reinterpret_cast<const f32x4*>(&sm.tdiag[i][cl][4 * qg]));
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // W = (I + Akk)^{-1} beta kh Gam for key column block cb, stored negated over the kh/Gam hi tile
    auto solve_w = [&](int cb, const V4T (&tii)[4]) {
        const int pc = perm32(16 * cb + cl);
        f32x4 X[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = to_f32(sm.kg[(16 * i + 4 * qg + j) * PK + pc]);
#pragma unroll
            for (int jp = 0; jp < i; ++jp)
                acc = mma_k16(acc, neg4(lds4<T>(&sm.akk[(16 * i + cl) * PC + 16 * jp + 4 * qg])), pack4<T>(X[jp]));
            X[i] = mma_k16(zero, tii[i], pack4<T>(acc));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.ki[(16 * i + 4 * qg + j) * PK + pc] = from_f32<T>(-X[i][j]);
    };

    // A state wave writes a 64 x 16 fp32 accumulator block (rows 16i+4qg+j,
    // column cl of its 16 columns) to rows 0..nrows-1 of a row-major array
    // (row stride ld elements; dst = row 0, the wave's first column) through
    // its own patch of LDS that no step uses when this runs (the Akk tile, the
    // diagonal-block arrays), so that each lane stores 4 contiguous columns:
    // four 16-byte stores per lane instead of sixteen 4-byte ones.  Only the
    // wave touches its patch, and a wave's LDS operations complete in order.
    // (Used for o; the fp32 saves for the backward measured no faster this way.)
    static_assert(offsetof(SM, tdiag) == offsetof(SM, adiag) + sizeof(sm.adiag) && offsetof(SM, akk) % 16 == 0 &&
                      offsetof(SM, adiag) % 16 == 0,
                  "the store patches need adiag/tdiag adjacent and 16-byte aligned tiles");
    auto patch_out = [&](auto* dst, int64_t ld, const f32x4 (&blk)[4], int nrows) {
        char* const patch = ww < 2 ? reinterpret_cast<char*>(sm.akk) : reinterpret_cast<char*>(sm.adiag);
        float* ot = reinterpret_cast<float*>(patch) + (ww & 1) * kChunk * kOStride;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) ot[(16 * i + 4 * qg + j) * kOStride + cl] = blk[i][j];
        const int cg = l & 3, rr = l >> 2;
        typedef typename std::remove_pointer<decltype(dst)>::type E;
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int r = 16 * pass + rr;
            const f32x4 x = *reinterpret_cast<const f32x4*>(&ot[r * kOStride + 4 * cg]);
            if (r < nrows) sts4<E>(dst + (r * (int)ld + 4 * cg), x);   // r * ld < 2^31 (checked on the host)
        }
    };

    // Prologue: both groups prepare the first chunk.  Then the two groups run
    // separate loops with the same barrier sequence: six barriers per chunk.
    if (t0 < t1) {
        load_chunk(t0);
        prep_a();
        lds_barrier();
        prep_b(t0);
        if (t0 + kChunk < t1) load_part(t0 + kChunk, 0);   // parts 1 and 2 in steps 1 and 2
    }
    if (is_state) {
        // ---------------------------------------------------------------- state waves
        const int64_t sbase = ((int64_t)n * H + h) * DK * ld;
        f32x4 S[NMB];
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * mb + 4 * qg + i;
                if (MAP)
                    S[mb][i] = (mslice && row == scol) ? 1.f : 0.f;
                else
                    S[mb][i] = p.s0 ? p.s0[sbase + (int64_t)row * dv + vcol] : 0.f;
            }
        int64_t slot = t0 / kChunk + n;
        for (int64_t c0 = t0; c0 < t1; c0 += kChunk, ++slot) {
            const int L = (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk);
            const bool more = c0 + kChunk < t1;
            // The entering state of this chunk (fp32) is saved a quarter per step
            // over steps 1-4 (S changes only in 5b): a wave stalls at issue while
            // its memory queue is full, so the stores go out beside the work.
            auto save_state = [&](int part) {
                if (SAVE) {
                    float* st = reinterpret_cast<float*>(p.st_saved) + (slot * H + h) * (int64_t)DK * dv;
                    constexpr int PER = NMB / 4;
#pragma unroll
                    for (int mb = part * PER; mb < (part + 1) * PER; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) *at32(st, (16 * mb + 4 * qg + i) * dv + vcol) = S[mb][i];
                }
            };
            refresh();
            // 1: held tiles
            if (more) load_part(c0 + kChunk, 1);
            store_held();
            save_state(0);
            lds_barrier();
            // 2
            refresh();
            if (more) load_part(c0 + kChunk, 2);
            save_state(1);
            intra_products();
            lds_barrier();
            // 3: (I + Akk_bb)^{-1}, block b = this wave; Ktil^T of this half
            refresh();
            save_state(2);
            {
                const f32x4 na = *reinterpret_cast<const f32x4*>(&sm.adiag[ww][cl][4 * qg]);
                f32x4 nb;
#pragma unroll
                for (int j = 0; j < 4; ++j) nb[j] = sm.adiag[ww][4 * qg + j][cl];
                const f32x4 tw = inv_unit_lower16_x3(na, nb, qg, cl);
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.tdiag[ww][4 * qg + i][cl] = tw[i];
            }
            store_ktil();
            lds_barrier();
            // 4: Ut = (I + Akk)^{-1} diag(beta) v for this wave's 16 value columns
            //    (and, at dk = 128, W for key column block ww + 4)
            refresh();
            save_state(3);
            f32x4 Ut[4];
            {
                V4T tii[4];
                load_tii(tii);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 vv = lds4f<T>(&sm.vt[kt_off(16 * ww + cl, 16 * i + 4 * qg)]);
                    const f32x4 bb = *reinterpret_cast<const f32x4*>(&sm.beta[16 * i + 4 * qg]);
                    f32x4 acc = vv * bb;   // beta v, exact in fp32
#pragma unroll
                    for (int jp = 0; jp < i; ++jp)
                        acc = mma_k16(acc, neg4(lds4<T>(&sm.akk[(16 * i + cl) * PC + 16 * jp + 4 * qg])), pack4<T>(Ut[jp]));
                    const V4T ah = pack4<T>(acc);
                    Ut[i] = mma_k16(zero, tii[i], ah);
                    Ut[i] = mma_k16(Ut[i], tii[i], pack4<T>(acc - unpack4(ah)));
                }
                if constexpr (DK == 128) solve_w(ww + 4, tii);
            }
            lds_barrier();
            // 5a: U = Ut - W S  (the tile holds -W) ;  O = (qh Gam) S ; next chunk's partial sums
            refresh();
            f32x4 O[4];
            V8T ufh[2], ufl[2];
            {
                V8T sfh[NKB], sfl[NKB];
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) split8<T, true>(S[2 * kk], S[2 * kk + 1], sfh[kk], sfl[kk]);
                // k-step outer: the twelve fragments of a step are read together
                // and feed four independent accumulator chains, so the LDS
                // latency is paid once per step rather than before every MFMA
#pragma unroll
                for (int i = 0; i < 4; ++i) O[i] = zero;
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) {
                    V8T aw[4], ah[4], al[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int ro = (16 * i + cl) * PK + 8 * qg + 32 * kk;
                        aw[i] = lds8<T>(sm.ki + ro);
                        ah[i] = lds8<T>(sm.qg + ro);
                        al[i] = lds8<T>(sm.qgl + ro);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        Ut[i] = mma_k32(Ut[i], aw[i], sfh[kk]);
                        O[i] = mma3<true>(O[i], ah[i], al[i], sfh[kk], sfl[kk]);
                    }
                }
            }
            if (SAVE) {
                // U of this chunk (fp32), for the chunk-parallel gradients, stored
                // column-major ([dv][64]): a lane's four rows are 16 contiguous bytes
                float* ub = p.u_saved + (slot * H + h) * (int64_t)kChunk * dv;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<f32x4*>(at32(ub, vcol * kChunk + 16 * i + 4 * qg)) = Ut[i];
            }
            split8<T, true>(Ut[0], Ut[1], ufh[0], ufl[0]);
            split8<T, true>(Ut[2], Ut[3], ufh[1], ufl[1]);
            if (more) prep_a();
            lds_barrier();
            refresh();
            // 5b: O += Aqk U ;  S <- Diag(Gam_C) S + Ktil^T U ; next chunk's operand values
            const KtFrag kf(qg, cl);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int kk = 0; kk <= (i >> 1); ++kk)
                    O[i] = mma3<true>(O[i], lds8<T>(sm.aqk + kf.at(i, kk)), lds8<T>(sm.aqkl + kf.at(i, kk)), ufh[kk],
                                      ufl[kk]);
            }
            if (!MAP) patch_out(op + (c0 * H + h) * dv + dv0 + 16 * ww, rs_v, O, L);
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb) {
                const f32x4 gcv = *reinterpret_cast<const f32x4*>(&sm.gc[16 * mb + 4 * qg]);
                S[mb] *= gcv;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int rt = kf.at(mb, kk);
                    S[mb] = mma3<true>(S[mb], lds8<T>(sm.kt + rt), lds8<T>(sm.kil + rt), ufh[kk], ufl[kk]);
                }
            }
            if (more) {
                prep_b(c0 + kChunk);
                if (c0 + 2 * kChunk < t1) load_part(c0 + 2 * kChunk, 0);
            }
            lds_barrier();
        }
        const int nd = p.sf_dst ? p.sf_dst[n] : n;   // the row of sfinal this sequence ends
        if (p.sfinal && nd >= 0) {
            const int64_t fbase = ((int64_t)nd * H + h) * DK * ld;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) p.sfinal[fbase + (int64_t)(16 * mb + 4 * qg + i) * ld + scol] = S[mb][i];
        }
    } else {
        // ---------------------------------------------------------------- prep waves
        for (int64_t c0 = t0; c0 < t1; c0 += kChunk) {
            const bool more = c0 + kChunk < t1;
            refresh();
            if (more) load_part(c0 + kChunk, 1);
            store_held();
            lds_barrier();
            refresh();
            if (more) load_part(c0 + kChunk, 2);
            intra_products();
            lds_barrier();
            refresh();
            store_ktil();
            lds_barrier();
            refresh();
            // 4: W for key column block ww (and, at dk = 64, that is all of W)
            {
                V4T tii[4];
                load_tii(tii);
                solve_w(ww, tii);
            }
            lds_barrier();
            refresh();
            if (more) prep_a();
            lds_barrier();
            refresh();
            if (more) {
                prep_b(c0 + kChunk);
                if (c0 + 2 * kChunk < t1) load_part(c0 + 2 * kChunk, 0);
            }
            lds_barrier();
        }
    }
}

template <typename T, typename TO, int DK>
static hipError_t launch_fwd_t(const FwdParams& p, bool save, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if constexpr (std::is_same<T, bf16>::value) {
        if (save)
            hipLaunchKernelGGL((kda_fwd_bf16_kernel<TO, DK, true, false>), grid, dim3(kWideThreads), 0, s, p);
        else
            hipLaunchKernelGGL((kda_fwd_bf16_kernel<TO, DK, false, false>), grid, dim3(kWideThreads), 0, s, p);
    } else {
        if (save)
            hipLaunchKernelGGL((kda_fwd_kernel<T, TO, DK, true>), grid, dim3(kThreads), 0, s, p);
        else
            hipLaunchKernelGGL((kda_fwd_kernel<T, TO, DK, false>), grid, dim3(kThreads), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_fwd_maps(const FwdParams& p, int dk, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if (dk == 128)
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<float, 128, false, true>), grid, dim3(kWideThreads), 0, s, p);
    else
        hipLaunchKernelGGL((kda_fwd_bf16_kernel<float, 64, false, true>), grid, dim3(kWideThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int out_dtype, int dk, bool save,
                      hipStream_t s) {
    if (in_dtype == 1) {
        if (dk == 128)
            return out_dtype == 1 ? launch_fwd_t<bf16, bf16, 128>(p, save, s)
                                  : launch_fwd_t<bf16, float, 128>(p, save, s);
        return out_dtype == 1 ? launch_fwd_t<bf16, bf16, 64>(p, save, s)
                              : launch_fwd_t<bf16, float, 64>(p, save, s);
    }
    // fp32 inputs: fp32 MFMA; dk = 64 only (the fp32 tiles of dk = 128 exceed LDS)
    return out_dtype == 1 ? launch_fwd_t<float, bf16, 64>(p, save, s)
                          : launch_fwd_t<float, float, 64>(p, save, s);
}

}  // namespace kda
