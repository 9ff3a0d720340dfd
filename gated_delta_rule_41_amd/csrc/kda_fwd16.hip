// kda_fwd16.hip -- fused chunked KDA forward for bf16 inputs on gfx950, with
// fp16 matrix-core operands.
//
// One persistent workgroup per (sequence, head, 64-wide slice of the value
// dimension) walks the sequence chunk by chunk (64 tokens), as the pages
// organise KDA: intra-chunk work plus inter-chunk state passing, with the Q/K
// normalisation, the beta transform and the gating fused into the forward
// ("TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
// practice", section "KDA pre/post-processing fusion"), and the stages fused
// into one kernel so that only the inputs are read and only o (and, when
// training, the per-chunk states) are written ("Ascend implements LoRA
// training of Kimi K3.1 Pro", section "KDA: big fused forward and backward").
//
// Per chunk (rows r, s = 0..63; G = inclusive in-chunk cumsum of g, log2 units):
//
//   prep    qh, kh = L2-normalised q, k;  beta = sigmoid(b);  G
//   intra   Akk = strict_lower(beta kh kh^T o 2^(G_r - G_s))
//           Aqk = lower(qh kh^T o 2^(G_r - G_s))
//           Td  = the four diagonal 16x16 blocks of (I + Akk)^{-1}
//   state   X = beta v - (beta kh 2^G) S
//           U = (I + Akk)^{-1} X           (blocked forward substitution)
//           O = (qh 2^G) S + Aqk U
//           S <- Diag(2^G_C) S + (kh 2^(G_C - G))^T U
//
// which is the gated delta rule unrolled over the chunk (U holds the per-token
// delta-rule updates beta (v - p) of the token recurrence).
//
// Wave roles.  Waves 0-3 ("state waves") own 16 value columns each: their
// dk x 16 fp32 state slice lives in MFMA accumulators for the whole sequence,
// and they run the state part of chunk n.  Waves 4-7 ("prep waves") prepare
// chunk n+1 meanwhile: prep wave p owns chunk rows 16p..16p+15.  The two
// groups meet at three LDS barriers per chunk; operands the state waves read
// late in a chunk are double-buffered, those read in its first phase are
// rewritten after the first barrier.
//
// Numerics.  Every matrix-core operand is a single fp16 rounding (11-bit
// significand) with fp32 accumulation.  fp16 has the range of neither the
// gate factors nor arbitrary values, so:
//  * gate factors are referenced to 16-row block boundaries: the off-diagonal
//    blocks of Akk/Aqk pair a row factor 2^(G_r - G_ref) <= 1 with a column
//    factor 2^(G_ref - G_s) <= 1 (ref between s and r); the diagonal blocks
//    pair 2^(G_r - G_b) <= 1 with 2^(G_b - G_s) <= 2^14 (G_b: block start),
//    which needs every channel's decay over each 16-row block to stay within
//    2^-14.  A chunk that breaks that bound is run token by token in fp32 by
//    the state waves (exact, no factorisation), so every gate is supported;
//  * the value side (state, v, X, U) is scaled per state wave and chunk by a
//    power of two that keeps its largest entry in [2^2, 2^8).
// A numpy emulation of every rounding point of this scheme gives
// max |o - o_ref| ~ 0.8% of rms(o) on the bf16 workloads.
#include <cstddef>
#include <type_traits>
#include <utility>

#include "kda_device.h"
#include "kda_f16.h"
#include "kda_internal.h"

namespace kda {
namespace f16 {

template <int DK>
struct __attribute__((aligned(16))) Smem {
    static constexpr int PK = DK + 8;      // row stride of [64][DK] tiles (halfs)
    static constexpr int PC = kChunk + 8;  // row stride of [64][64] tiles
    static constexpr int PV = kChunk + 8;  // row stride of the transposed v tile
    static constexpr int TDS = 20;         // row stride of a 16x16 diagonal inverse
    static constexpr int PKT = DK + 16;    // row stride of the row-major Ktil tile (rows 8 banks apart)
    // single-buffered: read by the state waves in the first phase of a chunk,
    // rewritten by the prep waves in the second
    h16 qg[kChunk * PK];          // qh 2^G                       [r][perm32(c)]
    h16 nbkg[kChunk * PK];        // -beta kh 2^G                 [r][perm32(c)]
    struct Buf {
        unsigned short vt[kSlice * PV];   // v (bf16 bits) transposed  [j][r]
        float beta[kChunk];
        h16 kt[kChunk * PKT];     // kh 2^(G_C - G), row-major    [r][c] (read transposed)
        h16 aqk[kChunk * PC];     // lower(Aqk)                   [r][perm32(s)]
        h16 nakk[kChunk * PC];    // -Akk, off-diagonal blocks    [r][s]
        h16 td[4][16 * TDS];      // (I + Akk_bb)^{-1}            [b][r][s]
        float gamc[DK];           // 2^G_C
        int flag[4];              // per prep wave: the chunk breaks the fp16 gate bound
    } buf[2];
    float etot[4][DK];            // 2^(block decay) per 16-row block
    h16 etoth[4][DK];             //   the same in fp16
    h16 kcol[3][16 * PK];         // blocks 0-2: kh 2^(G_b - G) (column operands), fragment order
    h8 ninv[4][64];               // per block, per lane: the A and B fragments of its strictly
                                  // lower diagonal block N (the state waves invert I + N)
};

template <typename TO, int DK, bool SAVE, bool MAP>
__global__ __launch_bounds__(kWideThreads, 1) void kda_fwd16_kernel(FwdParams p) {
    typedef bf16 T;
    typedef Smem<DK> SM;
    __shared__ SM sm;
    constexpr int PK = SM::PK, PC = SM::PC, PV = SM::PV, TDS = SM::TDS, PKT = SM::PKT;
    constexpr int CPL = DK / 4;     // key channels per prep lane (row layout)
    constexpr int CPG = DK / 16;    // key channels per prep lane (gate column layout)
    constexpr int NKB = DK / 32;    // k32 steps over dk
    constexpr int NMB = DK / 16;    // 16-row blocks of the state

    const int tid = threadIdx.x, w = tid >> 6;
    // Lane coordinates.  refresh() hides the lane index from the optimiser at
    // the top of every phase, so the addresses and masks derived from it are
    // recomputed there instead of being held in registers across the loop.
    int l = tid & 63, qg = l >> 4, cl = l & 15;
    auto refresh = [&]() {
        asm volatile("" : "+v"(l));
        qg = l >> 4;
        cl = l & 15;
    };
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
    const int nch = (int)((t1 - t0 + kChunk - 1) / kChunk);
    const int64_t slot0 = t0 / kChunk + n;

    const T* __restrict__ qp = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kp = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ vp = reinterpret_cast<const T*>(p.v);
    const T* __restrict__ gp = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bp = reinterpret_cast<const T*>(p.b);
    const int64_t rs_k = (int64_t)H * DK, rs_v = (int64_t)H * dv;   // token strides

    // The upper 16x16 blocks (0,1) and (2,3) of the Aqk tiles are read by the
    // k32 steps of Aqk U and never written: clear every tile once.
    for (int e = tid; e < kChunk * PC; e += kWideThreads) {
        sm.buf[0].aqk[e] = (h16)0.f;
        sm.buf[1].aqk[e] = (h16)0.f;
    }
    lds_barrier();

    // Schedule.  Iteration `it` has two phases separated by barriers.  The state
    // waves finish chunk it-1 (O += Aqk U, the state update) and start chunk it
    // (X, the state term of O) in phase A, and solve for U of chunk it in phase
    // B.  The prep waves prepare chunk it+1: in phase A everything that needs no
    // other wave's data, in phase B the rest.  Buffer b = chunk & 1; a prep
    // wave writes the tiles of chunk it+1 that the state waves read in phase A
    // (kt, aqk, gamc of chunk it-1, the same buffer) only in phase B.
    if (w < 4) {
        // ============================================================ state waves
        const int vl = 16 * w + cl;        // column inside the slice
        const int vcol = dv0 + vl;         // value column
        const int scol = sc0 + vl;         // state column
        TO* __restrict__ op = reinterpret_cast<TO*>(p.o);
        f32x4 S[NMB];
        const int64_t sbase = ((int64_t)n * H + h) * DK * dv;
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
        // S holds the state times 2^-e
        int e = 0;
        float sc = 1.f, usc = 1.f;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 X[4], O[4];
        h8 uf[2];
        bool pend = false;   // chunk it-1 ran the matrix path and waits for its second half

        for (int it = -1; it <= nch; ++it) {
            // --------------------------------------------------------- phase A
            refresh();
            if (pend) {
                // finish chunk it-1: O += Aqk U, store O; S <- Diag(2^G_C) S + Ktil^T U
                const int ip = it - 1;
                const typename SM::Buf& B = sm.buf[ip & 1];
                const int64_t cp = t0 + (int64_t)ip * kChunk;
                const int Lp = (int)((t1 - cp) < kChunk ? (t1 - cp) : kChunk);
                if (!MAP) {
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
                        for (int kk = 0; kk <= (ib >> 1); ++kk)
                            O[ib] = mma32(O[ib], *reinterpret_cast<const h8*>(&B.aqk[(16 * ib + cl) * PC + 32 * kk + 8 * qg]),
                                          uf[kk]);
                    }
                    // uniform row base + 32-bit lane offset (4qg rows + column)
                    TO* ob = op + (cp * H + h) * dv;
                    const float ousc = usc * p.scale;
                    const unsigned lane_off = (unsigned)(qg * 4 * (int)rs_v + dv0 + 16 * w + cl);
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = 16 * ib + 4 * qg + i;
                            if (r < Lp) *at32(ob + (int64_t)(16 * ib + i) * rs_v, lane_off) = from_f32<TO>(O[ib][i] * ousc);
                        }
                }
                // Ktil^T fragments by transpose reads of the row-major tile: lane
                // (qg, cl) gets channel 16mb + cl of rows 32kk + 16h + 4qg .. + 3,
                // positions 8qg + 4h + j (the perm32 order of uf)
                const h16* kb = &B.kt[(4 * qg + (cl >> 2)) * PKT + 4 * (cl & 3)];
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const f32x4 gcv = *reinterpret_cast<const f32x4*>(&B.gamc[16 * mb + 4 * qg]);
                    S[mb] *= gcv;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const h4 lo = lds_tr4(kb + (32 * kk) * PKT + 16 * mb);
                        const h4 hi = lds_tr4(kb + (32 * kk + 16) * PKT + 16 * mb);
                        S[mb] = mma32(S[mb], __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), uf[kk]);
                    }
                }
                pend = false;
            }
            const bool act = it >= 0 && it < nch;
            const int bi = it & 1;
            const int64_t c0 = t0 + (int64_t)it * kChunk;
            const int L = act ? (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk) : 0;
            const int64_t slot = slot0 + it;
            bool safe = false;
            if (act) {
                const typename SM::Buf& B = sm.buf[bi];
                safe = __builtin_amdgcn_readfirstlane(B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3]) == 0;
                // v of this lane's rows and the chunk's beta
                f32x4 vv[4];
                float mv = 0.f;
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    const u16x4 raw = *reinterpret_cast<const u16x4*>(&B.vt[vl * PV + 16 * ib + 4 * qg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        vv[ib][i] = __uint_as_float(((unsigned)raw[i]) << 16);
                        mv = fmaxf(mv, fabsf(vv[ib][i]));
                    }
                }
                // Power-of-two scale of the value side: S holds the state times
                // 2^-e with e chosen from the entering state and this chunk's v
                // alone (not from the history), so that a sequence split into
                // calls at a chunk boundary computes the same bits.  Afterwards
                // |S| < 2^6 and |beta v 2^-e| < 2^6, which keeps X and U inside
                // the fp16 range.
                {
                    float ms = 0.f;
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(S[mb][i]));
                    // the largest |state| (true scale, exact) or |v|
                    const float m = wave_max(fmaxf(ms * usc, mv));
                    if (m > 0.f && m < __builtin_inff()) {
                        int Et;
                        frexpf(m, &Et);   // m in [2^(Et-1), 2^Et)
                        const int en = min(max(Et - 6, -100), 100);
                        const int d = en - e;
                        if (d != 0) {
                            e = en;
#pragma unroll
                            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                                for (int i = 0; i < 4; ++i) S[mb][i] = ldexpf(S[mb][i], -d);
                            sc = ldexpf(1.f, -e);
                            usc = ldexpf(1.f, e);
                        }
                    }
                }
                if (SAVE) {
                    // entering state of this chunk: the scaled state in fp16 (|S| < 2^6
                    // here) and 2^e of this wave's 16 columns.  Saved blocked by 16
                    // value columns ([dv/16][dk][16]), so this wave's dk x 16 block is
                    // contiguous; each 16x16 block is turned into rows of four by the
                    // matrix core, so that one store writes 512 contiguous bytes
                    h16* st = reinterpret_cast<h16*>(p.st_saved) + (slot * H + h) * (int64_t)DK * dv +
                              ((dv0 >> 4) + w) * DK * 16;
                    const unsigned lane_off = (unsigned)(cl * 16 + 4 * qg);
                    const h4 eye4 = block_eye4(qg, cl);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
                        *reinterpret_cast<h4*>(at32(st + 256 * mb, lane_off)) = block_rows4(S[mb], eye4);
                    if (l == 0) p.sv_scale[(slot * H + h) * (dv / 16) + (dv0 >> 4) + w] = usc;
                }
                if (safe) {
                    h8 sf[NKB];
#pragma unroll
                    for (int kk = 0; kk < NKB; ++kk) sf[kk] = cvt8(S[2 * kk], S[2 * kk + 1]);
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        const f32x4 bb = *reinterpret_cast<const f32x4*>(&B.beta[16 * ib + 4 * qg]);
                        X[ib] = vv[ib] * (bb * sc);
                        O[ib] = zero;
                    }
#pragma unroll
                    for (int kk = 0; kk < NKB; ++kk) {
                        h8 an[4], aq[4];
#pragma unroll
                        for (int ib = 0; ib < 4; ++ib) {
                            const int ro = (16 * ib + cl) * PK + 32 * kk + 8 * qg;
                            an[ib] = *reinterpret_cast<const h8*>(&sm.nbkg[ro]);
                            if (!MAP) aq[ib] = *reinterpret_cast<const h8*>(&sm.qg[ro]);
                        }
#pragma unroll
                        for (int ib = 0; ib < 4; ++ib) {
                            X[ib] = mma32(X[ib], an[ib], sf[kk]);
                            if (!MAP) O[ib] = mma32(O[ib], aq[ib], sf[kk]);
                        }
                        asm volatile("" ::: "memory");
                    }
                } else {
                    // ---- token-by-token recurrence in fp32 for a chunk whose gate
                    // decay exceeds the fp16 factor range (exact: no factorisation)
                    const float l2e = kLog2e;
#pragma unroll 1
                    for (int t = 0; t < L; ++t) {
                        const int64_t tok = c0 + t;
                        const T* qr = qp + (tok * H + h) * DK + 4 * qg;
                        const T* kr = kp + (tok * H + h) * DK + 4 * qg;
                        const T* gr = gp + (tok * H + h) * DK + 4 * qg;
                        // the lane's channels 16mb+4qg+i, kept as bf16 bits
                        u16x4 qb[NMB], kb[NMB];
                        float skk = 0.f, sqq = 0.f;
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb) {
                            kb[mb] = *reinterpret_cast<const u16x4*>(kr + 16 * mb);
                            qb[mb] = MAP ? u16x4{0, 0, 0, 0} : *reinterpret_cast<const u16x4*>(qr + 16 * mb);
                            const u16x4 gb = *reinterpret_cast<const u16x4*>(gr + 16 * mb);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float kx = __uint_as_float(((unsigned)kb[mb][i]) << 16);
                                const float qx = __uint_as_float(((unsigned)qb[mb][i]) << 16);
                                skk += kx * kx;
                                sqq += qx * qx;
                                S[mb][i] *= fast_exp2(__uint_as_float(((unsigned)gb[i]) << 16) * l2e);
                            }
                        }
                        const float rk = 1.f / sqrtf(qsum(skk) + p.eps);
                        float pp = 0.f;
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) pp += S[mb][i] * __uint_as_float(((unsigned)kb[mb][i]) << 16);
                        const float pk = qsum(pp) * rk;
                        const float vtk = __uint_as_float(((unsigned)B.vt[vl * PV + t]) << 16) * sc;
                        const float u = B.beta[t] * (vtk - pk);
                        const float uk = u * rk;
                        float oo = 0.f;
#pragma unroll
                        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                S[mb][i] += __uint_as_float(((unsigned)kb[mb][i]) << 16) * uk;
                                oo += S[mb][i] * __uint_as_float(((unsigned)qb[mb][i]) << 16);
                            }
                        // (cross-lane sums on every lane, before the store branch)
                        const float o = MAP ? 0.f : qsum(oo) * (p.scale / sqrtf(qsum(sqq) + p.eps)) * usc;
                        if (qg == 0) {
                            if (!MAP) op[(tok * H + h) * dv + vcol] = from_f32<TO>(o);
                            if (SAVE) reinterpret_cast<h16*>(p.u_saved)[(slot * H + h) * (int64_t)kChunk * dv + ufrag(t, vcol)] = (h16)u;
                        }
                    }
                }
            }
            lds_barrier();
            // --------------------------------------------------------- phase B
            refresh();
            if (act && safe) {
                const typename SM::Buf& B = sm.buf[bi];
                // U = (I + Akk)^{-1} X by blocked forward substitution
                f32x4 U[4];
                h4 ub[4];
#pragma unroll
                for (int ib = 0; ib < 4; ++ib) {
                    f32x4 acc = X[ib];
#pragma unroll
                    for (int jb = 0; jb < ib; ++jb)
                        acc = mma16(acc, *reinterpret_cast<const h4*>(&B.nakk[(16 * ib + cl) * PC + 16 * jb + 4 * qg]),
                                    ub[jb]);
                    U[ib] = mma16(zero, *reinterpret_cast<const h4*>(&B.td[ib][cl * TDS + 4 * qg]), cvt4(acc));
                    ub[ib] = cvt4(U[ib]);
                }
                uf[0] = __builtin_shufflevector(ub[0], ub[1], 0, 1, 2, 3, 4, 5, 6, 7);
                uf[1] = __builtin_shufflevector(ub[2], ub[3], 0, 1, 2, 3, 4, 5, 6, 7);
                if (SAVE) {
                    // U of this chunk in fp16, scaled like the saved state, in MFMA
                    // fragment order (ufrag): each store is 512 contiguous bytes
                    h16* ubase = reinterpret_cast<h16*>(p.u_saved) + (slot * H + h) * (int64_t)kChunk * dv +
                                 ((dv0 >> 4) + w) * 1024;
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) *reinterpret_cast<h4*>(at32(ubase, 256 * ib + 4 * l)) = ub[ib];
                }
                pend = true;
            }
            if (it + 1 < nch) {
                // (I + N)^{-1} of row block w of chunk it+1, N from the prep wave of that
                // block: (I - N)(I + N^2)(I + N^4)(I + N^8), every product one fp16 k16
                // product; X and X^T carried as accumulator pairs (the accumulator of X
                // is the B operand of X and the A operand of X^T); T^T comes out in the
                // accumulator layout
                const h8 nn = sm.ninv[w][l];
                const h4 na = __builtin_shufflevector(nn, nn, 0, 1, 2, 3);   // A operand of N
                const h4 nb = __builtin_shufflevector(nn, nn, 4, 5, 6, 7);   // B operand of N
                f32x4 eyev;
#pragma unroll
                for (int i = 0; i < 4; ++i) eyev[i] = (4 * qg + i == cl) ? 1.f : 0.f;
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                const f32x4 p2 = mma16(z, na, nb);
                const f32x4 p2t = mma16(z, nb, na);
                const h4 p2h = cvt4(p2), p2th = cvt4(p2t);
                const f32x4 p4 = mma16(z, p2th, p2h);
                const f32x4 p4t = mma16(z, p2h, p2th);
                const h4 p4h = cvt4(p4), p4th = cvt4(p4t);
                const f32x4 p8 = mma16(z, p4th, p4h);
                const f32x4 y = mma16(eyev + p4 + p8, p4th, cvt4(p8));
                const f32x4 zz = mma16(y, p2th, cvt4(y));
                const f32x4 tt = mma16(z, cvt4(zz), cvt4(eyev - __builtin_convertvector(na, f32x4)));   // (I-N)^T
                *reinterpret_cast<h4*>(&sm.buf[(it + 1) & 1].td[w][cl * TDS + 4 * qg]) = cvt4(tt);
            }
            lds_barrier();
        }
        const int nd = p.sf_dst ? p.sf_dst[n] : n;   // the row of sfinal this sequence ends
        if (p.sfinal && nd >= 0) {
            const int64_t fbase = ((int64_t)nd * H + h) * DK * ld;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.sfinal[fbase + (int64_t)(16 * mb + 4 * qg + i) * ld + scol] = S[mb][i] * usc;
        }
    } else {
        // ============================================================ prep waves
        // The wave's 16-row block is a compile-time constant of its code path.
        auto prep = [&](auto pwc) {
        constexpr int pw = decltype(pwc)::value;
        int rr = 16 * pw + cl;             // row layout: row of this lane, channels CPL*qg ..
        RawRow<T, CPL> rq, rk;
        RawRow<T, CPG> rg[4];              // gate rows 16pw+4qg+j, channels CPG*cl ..
        RawRow<T, 4> rv[4];                // v rows 16pw+4qg+j, slice columns 4cl ..
        RawScalar<T> rb;
        // next-chunk rows go out in two groups, each as soon as its registers
        // are free: gates, beta and v after the gate prefix, q and k after the
        // diagonal-block products
        auto chunk_len = [&](int64_t c0) { return (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk); };
        auto load_gbv = [&](int64_t c0) {
            const int L = chunk_len(c0);
            const T* gc = gp + c0 * rs_k + h * DK;
            const T* vc = vp + c0 * rs_v + h * dv + dv0;
            const T* bc = bp + c0 * H + h;
            const int sk = (int)rs_k, sv = (int)rs_v;
            // rows past the chunk end load the last row (in bounds) and are
            // zeroed where first used
            rb.load(at32(bc, row_off(min(rr, L - 1), H, 0)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rj = min(16 * pw + 4 * qg + j, L - 1);
                rg[j].load(at32(gc, row_off(rj, sk, CPG * cl)));
                if (mslice) rv[j].zero();
                else rv[j].load(at32(vc, row_off(rj, sv, 4 * cl)));
            }
        };
        auto load_qk = [&](int64_t c0) {
            const int L = chunk_len(c0);
            const T* qc = qp + c0 * rs_k + h * DK;
            const T* kc = kp + c0 * rs_k + h * DK;
            const int sk = (int)rs_k;
            const int r = min(rr, L - 1);
            if (MAP) rq.zero();
            else rq.load(at32(qc, row_off(r, sk, CPL * qg)));
            rk.load(at32(kc, row_off(r, sk, CPL * qg)));
        };
        if (nch > 0) {
            load_gbv(t0);
            load_qk(t0);
        }

        for (int it = -1; it <= nch; ++it) {
            const int m = it + 1;              // chunk prepared in this iteration
            const bool act = m < nch;
            typename SM::Buf& B = sm.buf[m & 1];
            const int64_t cm = t0 + (int64_t)m * kChunk;
            // --------------------------------------------------------- phase A
            // Everything that needs no other wave's data: norms, sigmoid, the
            // block-local gate prefix and its decays, the row and column operands
            // referenced at the block start, the diagonal blocks of Akk and Aqk
            // and the inverses of the diagonal blocks of I + Akk.  The raw rows
            // are used up by the end of it, so the next chunk's loads go out here.
            refresh();
            rr = 16 * pw + cl;
            h8 Rq[NKB], Rk[NKB], Cd[NKB];
            f32x4 d3 = {0.f, 0.f, 0.f, 0.f};
            if (act) {
                const int Lm = __builtin_amdgcn_readfirstlane(chunk_len(cm));
                const bool more = m + 1 < nch;
                if (Lm < kChunk) {
                    // the last chunk of a document: rows past its end are zero
                    const bool rok = rr < Lm;
                    rq.keep(rok);
                    rk.keep(rok);
                    rb.x = rok ? rb.x : (unsigned short)0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool ok = 16 * pw + 4 * qg + j < Lm;
                        rg[j].keep(ok);
                        rv[j].keep(ok);
                    }
                }
                // v transposed (bf16 bits) for the state waves
#pragma unroll
                for (int ee = 0; ee < 4; ++ee) {
                    const u16x4 x = {rv[0].x[ee], rv[1].x[ee], rv[2].x[ee], rv[3].x[ee]};
                    *reinterpret_cast<u16x4*>(&B.vt[(4 * cl + ee) * PV + 16 * pw + 4 * qg]) = x;
                }
                // 1/||q||, 1/||k|| and the sigmoid by the hardware reciprocal
                // (square root), ~1 ulp: the operands they scale are rounded to
                // fp16 (11 bits)
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    sq += rq[c] * rq[c];
                    sk += rk[c] * rk[c];
                }
                const float ssq = qsum(sq) + p.eps;
                const float ssk = qsum(sk) + p.eps;
                // (the query scale is applied to O, which is linear in qh)
                const float rqs = __builtin_amdgcn_rsqf(ssq), rkk = __builtin_amdgcn_rsqf(ssk);
                const float beta = (rr < Lm) ? __builtin_amdgcn_rcpf(1.f + fast_exp(-rb.f())) : 0.f;
                if (qg == 0) B.beta[rr] = beta;
                // block-local inclusive prefix of g over the wave's 16 rows, as one
                // k16 product per column group (exact bf16 products, fp32 sums); it
                // returns lane (qg, cl) row 16pw+cl, channels CPG*(4qg+i)+e
                bf16x4 ltri;
#pragma unroll
                for (int j = 0; j < 4; ++j) ltri[j] = (bf16)((4 * qg + j <= cl) ? 1.f : 0.f);
                float Gl[CPL];
#pragma unroll
                for (int ee = 0; ee < CPG; ++ee) {
                    const u16x4 a = {rg[0].x[ee], rg[1].x[ee], rg[2].x[ee], rg[3].x[ee]};
                    const f32x4 d = mma_k16(f32x4{0.f, 0.f, 0.f, 0.f}, __builtin_bit_cast(bf16x4, a), ltri);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Gl[CPG * i + ee] = d[i] * kLog2e;
                }
                // The fp16 factors need every row's block-local log2 decay in
                // [-14, 0] (g <= 0 makes the prefix non-increasing, so its minimum
                // is the block total); anything else is run token by token.
                float gmin = 0.f, gmax = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    gmin = fminf(gmin, Gl[c]);
                    gmax = fmaxf(gmax, Gl[c]);
                }
                const bool bad = !(gmin >= kUnsafe) || !(gmax <= 0.f);
                const bool anybad = __builtin_amdgcn_ballot_w64(bad) != 0;
                if (l == 0) B.flag[pw] = anybad ? 1 : 0;
                // gates, beta and v are used up
                asm volatile("" ::: "memory");
                if (more) load_gbv(cm + kChunk);
                // operands referenced at the block start: rows x 2^Gl (<= 1),
                // columns kh 2^-Gl (<= 2^14), and the diagonal-block products
                f32x4 d1 = {0.f, 0.f, 0.f, 0.f}, d2 = d1;
                const float rkb = rkk * beta;
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) {
                    float rh[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int c = 8 * kk + j;
                        const float rho = fast_exp2(Gl[c]), iota = fast_exp2(-Gl[c]);
                        rh[j] = rho;
                        Rq[kk][j] = (h16)(rq[c] * (rqs * rho));
                        Rk[kk][j] = (h16)(rk[c] * (rkb * rho));
                        Cd[kk][j] = (h16)(rk[c] * (rkk * iota));
                    }
                    d1 = mma32(d1, Cd[kk], Rk[kk]);              // Akk^T: [4qg+i][cl] = Akk[cl][4qg+i]
                    d2 = mma32(d2, Rk[kk], Cd[kk]);              // Akk:   [4qg+i][cl] = Akk[4qg+i][cl]
                    if (!MAP) d3 = mma32(d3, Cd[kk], Rq[kk]);    // Aqk^T
                    // later blocks read this block's column operands
                    if constexpr (pw < 3)
                        *reinterpret_cast<h8*>(&sm.kcol[pw][cl * PK + CPL * qg + 8 * kk]) = Cd[kk];
                    // the block's last row holds 2^(block total) per channel (fp32 and
                    // fp16), which phase B reads for the other blocks' decays
                    if (cl == 15) {
                        float* et = &sm.etot[pw][CPL * qg + 8 * kk];
                        *reinterpret_cast<f32x4*>(et) = f32x4{rh[0], rh[1], rh[2], rh[3]};
                        *reinterpret_cast<f32x4*>(et + 4) = f32x4{rh[4], rh[5], rh[6], rh[7]};
                        h8 eh;
#pragma unroll
                        for (int j = 0; j < 8; ++j) eh[j] = (h16)rh[j];
                        *reinterpret_cast<h8*>(&sm.etoth[pw][CPL * qg + 8 * kk]) = eh;
                    }
                }
                // q and k are used up
                asm volatile("" ::: "memory");
                if (more) load_qk(cm + kChunk);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sI = 4 * qg + i;
                    d1[i] = sI < cl ? d1[i] : 0.f;    // N^T, accumulator layout
                    d2[i] = cl < sI ? d2[i] : 0.f;    // N
                    d3[i] = sI <= cl ? d3[i] : 0.f;
                }
                // the diagonal block N as the A and B fragments of the inverse, which
                // state wave pw forms in phase B (it has the time there)
                sm.ninv[pw][l] = __builtin_shufflevector(cvt4(d1), cvt4(d2), 0, 1, 2, 3, 4, 5, 6, 7);
                if (SAVE && slice == 0 && qg == 0 && rr < Lm) {
                    // head-major [H, T]: the block's 16 rows are 64 contiguous bytes
                    p.nq_saved[(int64_t)h * p.T + cm + rr] = sqrtf(ssq);
                    p.nk_saved[(int64_t)h * p.T + cm + rr] = sqrtf(ssk);
                }
            }
            lds_barrier();
            // --------------------------------------------------------- phase B
            // From the other waves' block decays: the chunk-start referenced
            // tiles (qh 2^G, -beta kh 2^G), Ktil^T, and the off-diagonal blocks of
            // Akk and Aqk; then this chunk's Aqk diagonal block and 2^G_C.
            refresh();
            rr = 16 * pw + cl;
            if (act) {
                h16* dq = &sm.qg[rr * PK];
                h16* dk = &sm.nbkg[rr * PK];
                // off-diagonal blocks (pw, jb): A = block jb's column operand times
                // 2^(G at the start of this block - G at the start of block jb) <= 1,
                // B = this wave's rows; the products come out transposed, so a lane
                // holds row 16pw+cl, columns 16jb+4qg..+3
                f32x4 aoff[3][2];
#pragma unroll
                for (int jb = 0; jb < 3; ++jb) aoff[jb][0] = aoff[jb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                h8 aqs[2], aks[2];   // (dk = 128) fragments 0 and 1, written beside 2 and 3
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) {
                    // the four blocks' decays of these 8 channels, in fp16 (each is
                    // >= 2^-14 on this path); in every product below a factor that
                    // may underflow is the last one, so what it makes tiny is tiny
                    h8 E[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) E[b] = *reinterpret_cast<const h8*>(&sm.etoth[b][CPL * qg + 8 * kk]);
                    h8 eoff = (h8)(h16)1.f, eaft = (h8)(h16)1.f;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        if (b < pw) eoff = eoff * E[b];
                        if (b > pw) eaft = eaft * E[b];
                    }
                    const h8 aq = Rq[kk] * eoff;                 // qh 2^G
                    const h8 ak = Rk[kk] * (-eoff);              // -beta kh 2^G
                    const h8 kt8 = (Cd[kk] * E[pw]) * eaft;      // kh 2^(G_C - G)
                    // qh 2^G, -beta kh 2^G (contraction index permuted: position
                    // 8q'+4hh+j of a 32-block holds channel 16hh+4q'+j)
                    if constexpr (DK == 128) {
                        if (kk < 2) {
                            aqs[kk] = aq;
                            aks[kk] = ak;
                        } else {
                            // 16-byte groups 8(kk-2) and 8(kk-2)+8 of the lane's 32-block:
                            // channels {4u..4u+3} of fragment kk-2 beside {16+4u..} of kk
#pragma unroll
                            for (int u2 = 0; u2 < 2; ++u2) {
                                const int pos = 32 * qg + 8 * (2 * (kk - 2) + u2);
                                h8 a, b;
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    a[j] = aqs[kk - 2][4 * u2 + j];
                                    a[j + 4] = aq[4 * u2 + j];
                                    b[j] = aks[kk - 2][4 * u2 + j];
                                    b[j + 4] = ak[4 * u2 + j];
                                }
                                if (!MAP) *reinterpret_cast<h8*>(dq + pos) = a;
                                *reinterpret_cast<h8*>(dk + pos) = b;
                            }
                        }
                    } else {
                        // 16 channels: half hh = qg & 1 of the 32-block qg >> 1
#pragma unroll
                        for (int u2 = 0; u2 < 2; ++u2) {
                            const int pos = 32 * (qg >> 1) + 4 * (qg & 1) + 8 * (2 * kk + u2);
                            h4 a, b;
#pragma unroll
                            for (int j = 0; j < 4; ++j) { a[j] = aq[4 * u2 + j]; b[j] = ak[4 * u2 + j]; }
                            if (!MAP) *reinterpret_cast<h4*>(dq + pos) = a;
                            *reinterpret_cast<h4*>(dk + pos) = b;
                        }
                    }
                    // Ktil, row-major (the state waves read it transposed)
                    *reinterpret_cast<h8*>(&B.kt[rr * PKT + CPL * qg + 8 * kk]) = kt8;
                    // off-diagonal products of this fragment
                    h8 f = (h8)(h16)1.f;   // running factor from block pw-1 down
#pragma unroll
                    for (int jb = pw - 1; jb >= 0; --jb) {
                        const h8 kc = *reinterpret_cast<const h8*>(&sm.kcol[jb][cl * PK + CPL * qg + 8 * kk]);
                        const h8 a = (kc * E[jb]) * f;
                        aoff[jb][0] = mma32(aoff[jb][0], a, Rk[kk]);
                        if (!MAP) aoff[jb][1] = mma32(aoff[jb][1], a, Rq[kk]);
                        f = f * E[jb];
                    }
                    asm volatile("" ::: "memory");
                }
                if constexpr (pw == 0) {
                    // 2^G_C in fp32 (it scales the fp32 state): two channels per lane
                    if (2 * l < DK) {
                        float2 gc = *reinterpret_cast<const float2*>(&sm.etot[0][2 * l]);
#pragma unroll
                        for (int b = 1; b < 4; ++b) {
                            const float2 x = *reinterpret_cast<const float2*>(&sm.etot[b][2 * l]);
                            gc.x *= x.x;
                            gc.y *= x.y;
                        }
                        *reinterpret_cast<float2*>(&B.gamc[2 * l]) = gc;
                    }
                }
#pragma unroll
                for (int jb = 0; jb < pw; ++jb) {
                    *reinterpret_cast<h4*>(&B.nakk[rr * PC + 16 * jb + 4 * qg]) = cvt4(-aoff[jb][0]);
                    if (!MAP) *reinterpret_cast<h4*>(&B.aqk[rr * PC + perm32(16 * jb + 4 * qg)]) = cvt4(aoff[jb][1]);
                }
                if (!MAP) *reinterpret_cast<h4*>(&B.aqk[rr * PC + perm32(16 * pw + 4 * qg)]) = cvt4(d3);
            }
            lds_barrier();
        }
        };
        switch (__builtin_amdgcn_readfirstlane(w)) {
            case 4: prep(std::integral_constant<int, 0>{}); break;
            case 5: prep(std::integral_constant<int, 1>{}); break;
            case 6: prep(std::integral_constant<int, 2>{}); break;
            default: prep(std::integral_constant<int, 3>{}); break;
        }
    }
}

template <typename TO, int DK>
static hipError_t launch_t(const FwdParams& p, bool save, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if (save)
        hipLaunchKernelGGL((kda_fwd16_kernel<TO, DK, true, false>), grid, dim3(kWideThreads), 0, s, p);
    else
        hipLaunchKernelGGL((kda_fwd16_kernel<TO, DK, false, false>), grid, dim3(kWideThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace f16

hipError_t launch_fwd16(const FwdParams& p, int out_dtype, int dk, bool save, hipStream_t s) {
    if (dk == 128)
        return out_dtype == 1 ? f16::launch_t<bf16, 128>(p, save, s) : f16::launch_t<float, 128>(p, save, s);
    return out_dtype == 1 ? f16::launch_t<bf16, 64>(p, save, s) : f16::launch_t<float, 64>(p, save, s);
}

hipError_t launch_fwd16_maps(const FwdParams& p, int dk, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if (dk == 128)
        hipLaunchKernelGGL((f16::kda_fwd16_kernel<float, 128, false, true>), grid, dim3(kWideThreads), 0, s, p);
    else
        hipLaunchKernelGGL((f16::kda_fwd16_kernel<float, 64, false, true>), grid, dim3(kWideThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
