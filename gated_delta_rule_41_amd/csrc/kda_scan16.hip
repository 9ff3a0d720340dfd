// kda_scan16.hip -- reverse state-gradient scan for bf16 inputs on gfx950, with
// fp16 matrix-core operands.
//
// The backward joins state-gradient propagation with the Q/K gradients and
// reuses what the forward saved ("TorchTitan Ascend open source: Kimi K3.1 Pro
// adaptation and training practice", section "KDA pre/post-processing
// fusion").  This kernel is the propagation: one persistent workgroup per
// (sequence, head, 64-wide value slice) walks the chunks backwards with
// dL/dS (dk x 64, fp32) resident in MFMA accumulators.  Per chunk (rows r, s;
// G the in-chunk cumsum of g in log2 units; Akk, Aqk as in the forward):
//
//   dU  = Aqk^T dO + Ktil dS1                 Ktil = kh 2^(G_C - G)
//   Y   = (I + Akk)^{-T} dU                   blocked back substitution
//   dS0 = Diag(2^G_C) dS1 + (qh 2^G)^T dO - (beta kh 2^G)^T Y
//
// with dS1 = dL/dS after the chunk and dS0 before it.  It writes dS1 and dU of
// every chunk for the chunk-parallel gradients (the W = T beta kh 2^G of the
// chunk form is never formed: dS0 takes its product with dU through Y).
//
// Layout and numerics follow the fp16 forward (kda_fwd16.hip): waves 0-3 own
// 16 value columns of dL/dS each; waves 4-7 prepare the chunk the state waves
// take next (16 rows each); gate factors are referenced to 16-row block
// boundaries, so a chunk in which some channel decays by more than 2^-14
// within a 16-row block is stepped token by token in fp32 (kda_token.h) and
// flagged for the pair-exact gradient kernel; dL/dS and dO are scaled per
// state wave and chunk by a power of two that keeps their largest entry in
// [2^2, 2^8).
#include <cstddef>
#include <type_traits>
#include <utility>

#include "kda_device.h"
#include "kda_f16.h"
#include "kda_internal.h"
#include "kda_token.h"

namespace kda {
namespace f16 {

template <int DK>
struct __attribute__((aligned(16))) ScanSmem16 {
    static constexpr int PK = DK + 8;      // row stride of [64][DK] tiles (halfs)
    static constexpr int PC = kChunk + 8;  // row stride of [64][64] tiles
    static constexpr int PV = kChunk + 8;  // row stride of the transposed dO tile
    static constexpr int TDS = 20;         // row stride of a 16x16 diagonal block
    static constexpr int PKT = DK + 16;    // row stride of the row-major qh 2^G / beta kh 2^G tiles
    // single-buffered: read by the state waves in the first phase of a chunk,
    // rewritten by the prep waves in the second
    h16 ktr[kChunk * PK];         // kh 2^(G_C - G)               [r][perm32(c)]
    h16 aqt[kChunk * PC];         // Aqk^T                        [s][perm32(r)]  (blocks r < s stay 0)
    struct Buf {
        unsigned short dot[kSlice * PV];  // dO (bf16 bits) transposed     [j][perm32(r)]
        h16 qgt[kChunk * PKT];    // qh 2^G, row-major            [r][c] (read transposed)
        h16 nkgt[kChunk * PKT];   // -beta kh 2^G, row-major      [r][c] (read transposed)
        h16 nakt[kChunk * PC];    // -Akk^T, off-diagonal blocks  [s][r]
        h16 tdt[4][16 * TDS];     // ((I + Akk_bb)^{-1})^T        [b][s][r]
        float gamc[DK];           // 2^G_C
        int flag[4];              // per prep wave: the chunk breaks the fp16 gate bound
    } buf[2];
    float etot[4][DK];            // 2^(block decay) per 16-row block
    h16 etoth[4][DK];             //   the same in fp16
    h16 kcol[3][16 * PK];         // blocks 0-2: kh 2^(G_b - G) (column operands)
};

template <int DK>
__global__ __launch_bounds__(kWideThreads, 1) void kda_bwd_scan16_kernel(BwdParams p) {
    typedef bf16 T;
    typedef ScanSmem16<DK> SM;
    __shared__ SM sm;
    constexpr int PK = SM::PK, PC = SM::PC, PV = SM::PV, TDS = SM::TDS, PKT = SM::PKT;
    constexpr int CPL = DK / 4;     // key channels per prep lane (row layout)
    constexpr int CPG = DK / 16;    // key channels per prep lane (gate column layout)
    constexpr int NKB = DK / 32;    // k32 steps over dk
    constexpr int NMB = DK / 16;    // 16-row blocks of the state

    const int tid = threadIdx.x, w = tid >> 6;
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
    const int dv0 = slice * kSlice;
    const int nch = (int)((t1 - t0 + kChunk - 1) / kChunk);
    const int64_t slot0 = t0 / kChunk + n;

    const T* __restrict__ qp = reinterpret_cast<const T*>(p.q);
    const T* __restrict__ kp = reinterpret_cast<const T*>(p.k);
    const T* __restrict__ gp = reinterpret_cast<const T*>(p.g);
    const T* __restrict__ bp = reinterpret_cast<const T*>(p.b);
    const T* __restrict__ dop = reinterpret_cast<const T*>(p.dO);
    const int64_t rs_k = (int64_t)H * DK, rs_v = (int64_t)H * dv;   // token strides

    // Aqk^T blocks with r-block < s-block are read by the k32 steps of dU and
    // never written: clear the tile once.
    for (int e = tid; e < kChunk * PC; e += kWideThreads) sm.aqt[e] = (h16)0.f;
    lds_barrier();

    // Schedule.  Iteration `it` takes chunk nch-1-it (processing order runs
    // backwards in time).  The state waves finish the previous one (its dS0) and
    // start this one (dS1 out, dU) in phase A and solve for Y in phase B; the
    // prep waves prepare the next one.  Buffer b = it & 1; the prep waves write
    // the tiles the state waves read in phase A of a later iteration (qgt,
    // nkgt, gamc) and the single-buffered ones (ktr, aqt) only in their phase B.
    if (w < 4) {
        // ============================================================ state waves
        const int vl = 16 * w + cl;        // column inside the slice
        const int vcol = dv0 + vl;         // value column
        h16* __restrict__ dst = reinterpret_cast<h16*>(p.dst_saved);
        f32x4 dS[NMB];
        const int64_t sbase = ((int64_t)n * H + h) * DK * dv;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dS[mb][i] = p.dS_final ? p.dS_final[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + vcol] : 0.f;
        // dS holds dL/dS times 2^-e
        int e = 0;
        float sc = 1.f, usc = 1.f;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 dU[4];
        h8 dof[2], yf[2];
        bool pend = false;   // the previous chunk ran the matrix path and waits for its dS0

        for (int it = -1; it <= nch; ++it) {
            // --------------------------------------------------------- phase A
            refresh();
            if (pend) {
                // dS0 = Diag(2^G_C) dS1 + (qh 2^G)^T dO - (beta kh 2^G)^T Y
                const typename SM::Buf& B = sm.buf[(it - 1) & 1];
                // transposed fragments by LDS transpose reads of the row-major tiles:
                // lane (qg, cl) gets channel 16mb + cl of rows 32kk + 16h + 4qg .. + 3
                const int fo = (4 * qg + (cl >> 2)) * PKT + 4 * (cl & 3);
#pragma unroll
                for (int mb = 0; mb < NMB; ++mb) {
                    const f32x4 gcv = *reinterpret_cast<const f32x4*>(&B.gamc[16 * mb + 4 * qg]);
                    dS[mb] *= gcv;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const int o0 = fo + (32 * kk) * PKT + 16 * mb, o1 = o0 + 16 * PKT;
                        const h8 aq = __builtin_shufflevector(lds_tr4(&B.qgt[o0]), lds_tr4(&B.qgt[o1]), 0, 1, 2, 3, 4, 5, 6, 7);
                        const h8 ak = __builtin_shufflevector(lds_tr4(&B.nkgt[o0]), lds_tr4(&B.nkgt[o1]), 0, 1, 2, 3, 4, 5, 6, 7);
                        dS[mb] = mma32(dS[mb], aq, dof[kk]);
                        dS[mb] = mma32(dS[mb], ak, yf[kk]);
                    }
                }
                pend = false;
            }
            const bool act = it >= 0 && it < nch;
            const int jc = nch - 1 - it;
            const int bi = it & 1;
            const int64_t c0 = t0 + (int64_t)jc * kChunk;
            const int L = act ? (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk) : 0;
            const int64_t slot = slot0 + jc;
            bool safe = false;
            if (act) {
                const typename SM::Buf& B = sm.buf[bi];
                safe = __builtin_amdgcn_readfirstlane(B.flag[0] | B.flag[1] | B.flag[2] | B.flag[3]) == 0;
                // chunks stepped token by token have no dU: the pair-exact kernel redoes them
                if (slice == 0 && tid == 0) p.chunk_flags[slot * H + h] = safe ? 0 : 1;
                // dO of this lane's B fragments (positions 32kk + 8qg .. + 7 of its column)
                u16x8 draw[2];
                float md = 0.f;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    draw[kk] = *reinterpret_cast<const u16x8*>(&B.dot[vl * PV + 32 * kk + 8 * qg]);
#pragma unroll
                    for (int j = 0; j < 8; ++j) md = fmaxf(md, fabsf(__uint_as_float(((unsigned)draw[kk][j]) << 16)));
                }
                md *= fabsf(p.scale);   // dO enters only through qh, so it carries the query scale
                // power-of-two scale from the entering dL/dS and this chunk's dO
                // alone (not the history), as in the forward
                {
                    float ms = 0.f;
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) ms = fmaxf(ms, fabsf(dS[mb][i]));
                    const float m = wave_max(fmaxf(ms * usc, md));
                    if (m > 0.f && m < __builtin_inff()) {
                        int Et;
                        frexpf(m, &Et);
                        const int en = min(max(Et - 6, -100), 100);
                        const int d = en - e;
                        if (d != 0) {
                            e = en;
#pragma unroll
                            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                                for (int i = 0; i < 4; ++i) dS[mb][i] = ldexpf(dS[mb][i], -d);
                            sc = ldexpf(1.f, -e);
                            usc = ldexpf(1.f, e);
                        }
                    }
                }
                {
                    // dL/dS at the end of this chunk: the scaled values in fp16 and
                    // 2^e of this wave's 16 columns, blocked by 16 value columns
                    // ([dv/16][dk][16]) as the forward saves its states
                    // (each 16x16 block turned into rows of four by the matrix core:
                    // one store writes 512 contiguous bytes)
                    h16* out = dst + (slot * H + h) * (int64_t)DK * dv + ((dv0 >> 4) + w) * DK * 16;
                    const unsigned lane_off = (unsigned)(cl * 16 + 4 * qg);
                    const h4 eye4 = block_eye4(qg, cl);
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb)
                        *reinterpret_cast<h4*>(at32(out + 256 * mb, lane_off)) = block_rows4(dS[mb], eye4);
                    if (l == 0) p.ds_scale[(slot * H + h) * (dv / 16) + (dv0 >> 4) + w] = usc;
                }
                if (safe) {
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            dof[kk][j] = (h16)(__uint_as_float(((unsigned)draw[kk][j]) << 16) * (sc * p.scale));
                    h8 sf[NKB];
#pragma unroll
                    for (int kk = 0; kk < NKB; ++kk) sf[kk] = cvt8(dS[2 * kk], dS[2 * kk + 1]);
                    // dU = Aqk^T dO + Ktil dS1
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb) {
                        dU[sb] = zero;
#pragma unroll
                        for (int kk = sb >> 1; kk < 2; ++kk)
                            dU[sb] = mma32(dU[sb], *reinterpret_cast<const h8*>(&sm.aqt[(16 * sb + cl) * PC + 32 * kk + 8 * qg]),
                                           dof[kk]);
                    }
#pragma unroll
                    for (int kk = 0; kk < NKB; ++kk) {
                        h8 a[4];
#pragma unroll
                        for (int sb = 0; sb < 4; ++sb)
                            a[sb] = *reinterpret_cast<const h8*>(&sm.ktr[(16 * sb + cl) * PK + 32 * kk + 8 * qg]);
#pragma unroll
                        for (int sb = 0; sb < 4; ++sb) dU[sb] = mma32(dU[sb], a[sb], sf[kk]);
                        asm volatile("" ::: "memory");
                    }
                } else {
                    // ---- the transposed recurrence token by token in fp32, for a
                    // chunk whose gate decay exceeds the fp16 factor range
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) dS[mb] *= usc;
                    e = 0;
                    sc = usc = 1.f;
                    const TokSrc<T> src = {qp, kp, gp, bp, dop, H, h, dv, vcol, qg, p.eps, p.scale};
                    token_bwd<T, DK>(dS, src, c0, L);
                }
            }
            lds_barrier();
            // --------------------------------------------------------- phase B
            refresh();
            if (act && safe) {
                const typename SM::Buf& B = sm.buf[bi];
                // Y = (I + Akk)^{-T} dU, from the last block up
                h4 yb[4];
#pragma unroll
                for (int sb = 3; sb >= 0; --sb) {
                    f32x4 acc = dU[sb];
#pragma unroll
                    for (int jb = sb + 1; jb < 4; ++jb)
                        acc = mma16(acc, *reinterpret_cast<const h4*>(&B.nakt[(16 * sb + cl) * PC + 16 * jb + 4 * qg]),
                                    yb[jb]);
                    yb[sb] = cvt4(mma16(zero, *reinterpret_cast<const h4*>(&B.tdt[sb][cl * TDS + 4 * qg]), cvt4(acc)));
                }
                yf[0] = __builtin_shufflevector(yb[0], yb[1], 0, 1, 2, 3, 4, 5, 6, 7);
                yf[1] = __builtin_shufflevector(yb[2], yb[3], 0, 1, 2, 3, 4, 5, 6, 7);
                // dU of this chunk in fp16 (scaled like dS1), in MFMA fragment order
                // as the forward's U (ufrag): each store is 512 contiguous bytes
                h16* ub = reinterpret_cast<h16*>(p.du_ws) + (slot * H + h) * (int64_t)kChunk * dv + ((dv0 >> 4) + w) * 1024;
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) *reinterpret_cast<h4*>(at32(ub, 256 * sb + 4 * l)) = cvt4(dU[sb]);
                pend = true;
            }
            lds_barrier();
        }
        if (p.dS0) {
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.dS0[sbase + (int64_t)(16 * mb + 4 * qg + i) * dv + vcol] = dS[mb][i] * usc;
        }
    } else {
        // ============================================================ prep waves
        auto prep = [&](auto pwc) {
        constexpr int pw = decltype(pwc)::value;
        int rr = 16 * pw + cl;             // row layout: row of this lane, channels CPL*qg ..
        RawRow<T, CPL> rq, rk;
        RawRow<T, CPG> rg[4];              // gate rows 16pw+4qg+j, channels CPG*cl ..
        RawRow<T, 4> rd[4];                // dO rows 16pw+4qg+j, slice columns 4cl ..
        RawScalar<T> rb;
        auto chunk_len = [&](int64_t c0) { return (int)((t1 - c0) < kChunk ? (t1 - c0) : kChunk); };
        auto load_gbd = [&](int64_t c0) {
            const int L = chunk_len(c0);
            const T* gc = gp + c0 * rs_k + h * DK;
            const T* dc = dop + c0 * rs_v + h * dv + dv0;
            const T* bc = bp + c0 * H + h;
            const int sk = (int)rs_k, sv = (int)rs_v;
            // rows past the chunk end load the last row (in bounds) and are
            // zeroed where first used
            rb.load(at32(bc, row_off(min(rr, L - 1), H, 0)));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rj = min(16 * pw + 4 * qg + j, L - 1);
                rg[j].load(at32(gc, row_off(rj, sk, CPG * cl)));
                rd[j].load(at32(dc, row_off(rj, sv, 4 * cl)));
            }
        };
        auto load_qk = [&](int64_t c0) {
            const int L = chunk_len(c0);
            const T* qc = qp + c0 * rs_k + h * DK;
            const T* kc = kp + c0 * rs_k + h * DK;
            const int sk = (int)rs_k;
            const int r = min(rr, L - 1);
            rq.load(at32(qc, row_off(r, sk, CPL * qg)));
            rk.load(at32(kc, row_off(r, sk, CPL * qg)));
        };
        if (nch > 0) {
            const int64_t cl0 = t0 + (int64_t)(nch - 1) * kChunk;
            load_gbd(cl0);
            load_qk(cl0);
        }

        for (int it = -1; it <= nch; ++it) {
            const int m = it + 1;              // processing index prepared in this iteration
            const bool act = m < nch;
            typename SM::Buf& B = sm.buf[m & 1];
            const int64_t cm = t0 + (int64_t)(nch - 1 - m) * kChunk;
            // --------------------------------------------------------- phase A
            refresh();
            rr = 16 * pw + cl;
            h8 Rq[NKB], Rk[NKB], Cd[NKB];
            f32x4 d3 = {0.f, 0.f, 0.f, 0.f};   // the diagonal block of Aqk, written in phase B
            if (act) {
                const int Lm = __builtin_amdgcn_readfirstlane(chunk_len(cm));
                const bool more = m + 1 < nch;
                if (Lm < kChunk) {
                    const bool rok = rr < Lm;
                    rq.keep(rok);
                    rk.keep(rok);
                    rb.x = rok ? rb.x : (unsigned short)0;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool ok = 16 * pw + 4 * qg + j < Lm;
                        rg[j].keep(ok);
                        rd[j].keep(ok);
                    }
                }
                // dO transposed (bf16 bits) for the state waves; four consecutive
                // rows stay consecutive under perm32
#pragma unroll
                for (int ee = 0; ee < 4; ++ee) {
                    const u16x4 x = {rd[0].x[ee], rd[1].x[ee], rd[2].x[ee], rd[3].x[ee]};
                    *reinterpret_cast<u16x4*>(&B.dot[(4 * cl + ee) * PV + perm32(16 * pw + 4 * qg)]) = x;
                }
                float sq = 0.f, sk = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    sq += rq[c] * rq[c];
                    sk += rk[c] * rk[c];
                }
                const float nq = sqrtf(qsum(sq) + p.eps);
                const float nk = sqrtf(qsum(sk) + p.eps);
                // (the query scale is applied to dO, which qh only ever multiplies)
                const float rqs = 1.f / nq, rkk = 1.f / nk;
                const float beta = (rr < Lm) ? 1.f / (1.f + fast_exp(-rb.f())) : 0.f;
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
                float gmin = 0.f, gmax = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    gmin = fminf(gmin, Gl[c]);
                    gmax = fmaxf(gmax, Gl[c]);
                }
                const bool bad = !(gmin >= kUnsafe) || !(gmax <= 0.f);
                const bool anybad = __builtin_amdgcn_ballot_w64(bad) != 0;
                if (l == 0) B.flag[pw] = anybad ? 1 : 0;
                if (cl == 15) {
#pragma unroll
                    for (int c = 0; c < CPL; c += 4)
                        *reinterpret_cast<f32x4*>(&sm.etot[pw][CPL * qg + c]) =
                            f32x4{Gl[c], Gl[c + 1], Gl[c + 2], Gl[c + 3]};
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                __builtin_amdgcn_wave_barrier();
                {
                    float2* e2 = reinterpret_cast<float2*>(&sm.etot[pw][(2 * l) & (DK - 1)]);
                    float2 x = *e2;
                    x.x = fast_exp2(x.x);
                    x.y = fast_exp2(x.y);
                    __builtin_amdgcn_wave_barrier();
                    if (2 * l < DK) {
                        *e2 = x;
                        *reinterpret_cast<hx2*>(&sm.etoth[pw][2 * l]) = __builtin_convertvector(f2{x.x, x.y}, hx2);
                    }
                }
                asm volatile("" ::: "memory");
                if (more) load_gbd(cm - kChunk);
                // operands referenced at the block start: rows x 2^Gl (<= 1),
                // columns kh 2^-Gl (<= 2^14), and the diagonal-block products
                f32x4 d1 = {0.f, 0.f, 0.f, 0.f}, d2 = d1;
                const float rkb = rkk * beta;
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int c = 8 * kk + j;
                        const float rho = fast_exp2(Gl[c]), iota = fast_exp2(-Gl[c]);
                        Rq[kk][j] = (h16)(rq[c] * (rqs * rho));
                        Rk[kk][j] = (h16)(rk[c] * (rkb * rho));
                        Cd[kk][j] = (h16)(rk[c] * (rkk * iota));
                    }
                    d1 = mma32(d1, Cd[kk], Rk[kk]);   // Akk^T: [4qg+i][cl] = Akk[cl][4qg+i]
                    d2 = mma32(d2, Rk[kk], Cd[kk]);   // Akk:   [4qg+i][cl] = Akk[4qg+i][cl]
                    d3 = mma32(d3, Rq[kk], Cd[kk]);   // Aqk:   [4qg+i][cl] = Aqk[4qg+i][cl]
                    if constexpr (pw < 3)
                        *reinterpret_cast<h8*>(&sm.kcol[pw][cl * PK + CPL * qg + 8 * kk]) = Cd[kk];
                }
                asm volatile("" ::: "memory");
                if (more) load_qk(cm - kChunk);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int sI = 4 * qg + i;
                    d1[i] = sI < cl ? d1[i] : 0.f;    // N^T, accumulator layout
                    d2[i] = cl < sI ? d2[i] : 0.f;    // N
                    d3[i] = sI >= cl ? d3[i] : 0.f;   // lower(Aqk): row 4qg+i >= column cl
                }
                // diagonal block inverse as in the forward; tt = T^T in accumulator
                // layout, i.e. lane (qg, cl) holds T[cl][4qg+i], stored transposed
                {
                    f32x4 eyev;
#pragma unroll
                    for (int i = 0; i < 4; ++i) eyev[i] = (4 * qg + i == cl) ? 1.f : 0.f;
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const h4 na = cvt4(d1), nb = cvt4(d2);
                    const f32x4 p2 = mma16(z, na, nb);
                    const f32x4 p2t = mma16(z, nb, na);
                    const h4 p2h = cvt4(p2), p2th = cvt4(p2t);
                    const f32x4 p4 = mma16(z, p2th, p2h);
                    const f32x4 p4t = mma16(z, p2h, p2th);
                    const h4 p4h = cvt4(p4), p4th = cvt4(p4t);
                    const f32x4 p8 = mma16(z, p4th, p4h);
                    const f32x4 y = mma16(eyev + p4 + p8, p4th, cvt4(p8));
                    const f32x4 zz = mma16(y, p2th, cvt4(y));
                    const f32x4 tt = mma16(z, cvt4(zz), cvt4(eyev - d1));
                    const h4 th = cvt4(tt);
#pragma unroll
                    for (int i = 0; i < 4; ++i) B.tdt[pw][(4 * qg + i) * TDS + cl] = th[i];
                }
            }
            lds_barrier();
            // --------------------------------------------------------- phase B
            refresh();
            rr = 16 * pw + cl;
            if (act) {
                h16* dkt = &sm.ktr[rr * PK];
                // off-diagonal blocks (pw, jb): rows of this wave (A) against block
                // jb's column operand times 2^(G at the start of this block - G at
                // the start of block jb) (B), so that a lane holds rows
                // 16pw+4qg..+3 of column 16jb+cl -- the transposed tiles' order
                f32x4 aoff[3][2];
#pragma unroll
                for (int jb = 0; jb < 3; ++jb) aoff[jb][0] = aoff[jb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                h8 kts[2];   // (dk = 128) fragments 0 and 1, written beside 2 and 3
#pragma unroll
                for (int kk = 0; kk < NKB; ++kk) {
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
                    // Ktil rows (contraction index permuted as in the forward's row tiles)
                    if constexpr (DK == 128) {
                        if (kk < 2) {
                            kts[kk] = kt8;
                        } else {
#pragma unroll
                            for (int u2 = 0; u2 < 2; ++u2) {
                                const int pos = 32 * qg + 8 * (2 * (kk - 2) + u2);
                                h8 a;
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    a[j] = kts[kk - 2][4 * u2 + j];
                                    a[j + 4] = kt8[4 * u2 + j];
                                }
                                *reinterpret_cast<h8*>(dkt + pos) = a;
                            }
                        }
                    } else {
#pragma unroll
                        for (int u2 = 0; u2 < 2; ++u2) {
                            const int pos = 32 * (qg >> 1) + 4 * (qg & 1) + 8 * (2 * kk + u2);
                            h4 a;
#pragma unroll
                            for (int j = 0; j < 4; ++j) a[j] = kt8[4 * u2 + j];
                            *reinterpret_cast<h4*>(dkt + pos) = a;
                        }
                    }
                    // qh 2^G and -beta kh 2^G row-major (the state waves read them transposed)
                    *reinterpret_cast<h8*>(&B.qgt[rr * PKT + CPL * qg + 8 * kk]) = aq;
                    *reinterpret_cast<h8*>(&B.nkgt[rr * PKT + CPL * qg + 8 * kk]) = ak;
                    h8 f = (h8)(h16)1.f;
#pragma unroll
                    for (int jb = pw - 1; jb >= 0; --jb) {
                        const h8 kc = *reinterpret_cast<const h8*>(&sm.kcol[jb][cl * PK + CPL * qg + 8 * kk]);
                        const h8 a = (kc * E[jb]) * f;
                        aoff[jb][0] = mma32(aoff[jb][0], Rk[kk], a);
                        aoff[jb][1] = mma32(aoff[jb][1], Rq[kk], a);
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
                    // row s = 16jb + cl of the transposed tiles, rows r = 16pw + 4qg ..
                    *reinterpret_cast<h4*>(&B.nakt[(16 * jb + cl) * PC + 16 * pw + 4 * qg]) = cvt4(-aoff[jb][0]);
                    *reinterpret_cast<h4*>(&sm.aqt[(16 * jb + cl) * PC + perm32(16 * pw + 4 * qg)]) = cvt4(aoff[jb][1]);
                }
                // the diagonal block of Aqk^T: row s = 16pw + cl, positions of r = 16pw + 4qg ..
                *reinterpret_cast<h4*>(&sm.aqt[(16 * pw + cl) * PC + perm32(16 * pw + 4 * qg)]) = cvt4(d3);
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

}  // namespace f16

hipError_t launch_scan16(const BwdParams& p, int dk, hipStream_t s) {
    const dim3 grid((unsigned)(p.N * p.H * p.nslices));
    if (dk == 128)
        hipLaunchKernelGGL((f16::kda_bwd_scan16_kernel<128>), grid, dim3(kWideThreads), 0, s, p);
    else
        hipLaunchKernelGGL((f16::kda_bwd_scan16_kernel<64>), grid, dim3(kWideThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
