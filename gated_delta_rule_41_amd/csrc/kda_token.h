// kda_token.h -- the gated delta rule token by token in fp32, on a state slice
// held in the accumulator layout of the chunked kernels.
//
// The chunked kernels factor the decay between two tokens r >= s of a chunk as
// exp(G_r) * exp(-G_s), both referenced to the chunk start (G the in-chunk
// cumulative sum of g).  Once a channel decays by more than about e^-87 inside
// one chunk, exp(-G_s) overflows fp32.  The recurrence itself needs no such
// factorisation, so chunks past a threshold are run without it: the forward
// and the reverse state-gradient scan step such a chunk one token at a time
// (this file), and the chunk gradients evaluate every decay between two tokens
// as exp(G_r - G_s) directly (kda_exact.hip).  The recurrence is the one of
// "TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
// practice" (section "Kimi K3.1 Pro model structure"), a per-channel decay in
// (0, 1] for every key channel.
//
// Layout: lane (qg, cl) of a wave holds rows 16 mb + 4 qg + i (mb < DK/16,
// i < 4) of one state column; a sum over all DK rows is the sum over the
// lane's own rows and then over the four lane groups qg (lanes l, l^16, l^32,
// l^48), which every lane of the four receives bitwise equal.
#pragma once
#include "kda_device.h"

namespace kda {

// Thresholds on a chunk's smallest per-channel decay sum, sum_chunk g (natural
// log).  Sequential kernels step a chunk token by token below kTokenBelow; the
// chunk-gradient fallback recomputes every chunk below kExactBelow.  Since
// kTokenBelow < kExactBelow, every chunk the reverse scan stepped token by
// token (for which it wrote no dU) is recomputed by the fallback, whatever the
// rounding of the two kernels' sums, and the factorised kernels only keep
// chunks above kTokenBelow, whose factors stay below e^70 ~ 2.5e30.
constexpr float kExactBelow = -60.f;
constexpr float kTokenBelow = -70.f;

__device__ __forceinline__ float qg_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// One token's inputs at the lane's rows (channels 16 mb + 4 qg .. + 3) and the
// scalar at its column (v in the forward, dO in the reverse scan).
template <typename T, int NMB>
struct TokRow {
    RawRow<T, 4> q[NMB], k[NMB], g[NMB];
    RawScalar<T> b, x;
    __device__ __forceinline__ void load(const T* qr, const T* kr, const T* gr, const T* br, const T* xr) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
            q[mb].load(qr + 16 * mb);
            k[mb].load(kr + 16 * mb);
            g[mb].load(gr + 16 * mb);
        }
        b.load(br);
        x.load(xr);
    }
};

// Where one document's inputs are: token-major [T, H, *] arrays, head h.
template <typename T>
struct TokSrc {
    const T* q;
    const T* k;
    const T* g;
    const T* b;
    const T* x;   // v (forward) or dO (reverse scan), [T, H, dv]
    int H, h, dv, col, qg;
    float eps, scale;
    template <int NMB>
    __device__ __forceinline__ void load(TokRow<T, NMB>& r, int64_t tok) const {
        const int64_t base = (tok * H + h) * (int64_t)(16 * NMB) + 4 * qg;
        r.load(q + base, k + base, g + base, b + tok * H + h, x + (tok * H + h) * (int64_t)dv + col);
    }
};

// Tokens c0 .. c0 + L - 1 of the forward recurrence on the state slice S:
//   S <- Diag(exp g_t) S;  u = beta_t (v_t - S^T kh_t);  S <- S + kh_t u^T;  o_t = S^T qh_t
// with kh = k / sqrt(|k|^2 + eps), qh = scale q / sqrt(|q|^2 + eps),
// beta = sigmoid(b).  o_t of the lane's column is stored by lane group 0 when
// op is set; when nq_out is set, `wnorm` lanes store the two norms.
template <typename T, typename TO, int DK>
__device__ void token_fwd(f32x4 (&S)[DK / 16], const TokSrc<T>& src, int64_t c0, int L, TO* op, float* nq_out,
                          float* nk_out, bool wnorm) {
    constexpr int NMB = DK / 16;
    TokRow<T, NMB> cur, nxt;
    if (L > 0) src.load(cur, c0);
#pragma unroll 1
    for (int t = 0; t < L; ++t) {
        const int64_t tok = c0 + t;
        if (t + 1 < L) src.load(nxt, tok + 1);
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sq += cur.q[mb][i] * cur.q[mb][i];
                sk += cur.k[mb][i] * cur.k[mb][i];
                S[mb][i] *= fast_exp(cur.g[mb][i]);
            }
        const float nk = sqrtf(qg_sum(sk) + src.eps), nq = sqrtf(qg_sum(sq) + src.eps);
        const float rk = 1.f / nk;
        float pp = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) pp += S[mb][i] * cur.k[mb][i];
        const float beta = 1.f / (1.f + fast_exp(-cur.b.f()));
        const float u = beta * (cur.x.f() - qg_sum(pp) * rk);
        const float uk = u * rk;
        float oo = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S[mb][i] += cur.k[mb][i] * uk;
                oo += S[mb][i] * cur.q[mb][i];
            }
        const float o = qg_sum(oo) * (src.scale / nq);
        if (op && src.qg == 0) op[(tok * src.H + src.h) * (int64_t)src.dv + src.col] = from_f32<TO>(o);
        if (nq_out && wnorm) {
            nq_out[tok] = nq;   // this head's row of the head-major norms
            nk_out[tok] = nk;
        }
        cur = nxt;
    }
}

// dL/dS through tokens c0 + L - 1 down to c0 (R enters as dL/dS after the
// last of them and leaves as dL/dS before the first):
//   R <- R + qh_t dO_t^T;  w = R^T kh_t;  R <- Diag(exp g_t) (R - beta_t kh_t w^T)
// the transpose of the forward step, which needs no state.
template <typename T, int DK>
__device__ void token_bwd(f32x4 (&R)[DK / 16], const TokSrc<T>& src, int64_t c0, int L) {
    constexpr int NMB = DK / 16;
    TokRow<T, NMB> cur, nxt;
    if (L > 0) src.load(cur, c0 + L - 1);
#pragma unroll 1
    for (int t = L - 1; t >= 0; --t) {
        if (t > 0) src.load(nxt, c0 + t - 1);
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sq += cur.q[mb][i] * cur.q[mb][i];
                sk += cur.k[mb][i] * cur.k[mb][i];
            }
        const float nk = sqrtf(qg_sum(sk) + src.eps), nq = sqrtf(qg_sum(sq) + src.eps);
        const float dq = cur.x.f() * (src.scale / nq);
        float ww = 0.f;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                R[mb][i] += cur.q[mb][i] * dq;
                ww += R[mb][i] * cur.k[mb][i];
            }
        const float beta = 1.f / (1.f + fast_exp(-cur.b.f()));
        const float c = beta * qg_sum(ww) / (nk * nk);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) R[mb][i] = fast_exp(cur.g[mb][i]) * (R[mb][i] - cur.k[mb][i] * c);
        cur = nxt;
    }
}

}  // namespace kda
