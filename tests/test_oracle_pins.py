"""Pins for the fp64 oracle against what mathematics fixes independently of it.

Each test below would fail on a plausible mistake in the oracle: a dropped or
mis-signed term, a transposed operand, a wrong index, decay applied after the
write instead of before, output read before the update, a missing chain rule
through the norm or the sigmoid.

The pages print no formula, example or number for KDA, so there is no golden
value from them; every pin is a mathematical one:
  * brute-force unrolled products of explicit dk x dk transition matrices;
  * closed forms for beta = 0 (pure decay) and alpha = 1 (ungated delta rule);
  * exact recall identities of the delta rule with beta = 1;
  * prep against numpy/scipy library routines;
  * chunk-size invariance of the chunked form against the recurrence;
  * central finite differences for every gradient, the adjoint identity and
    the scale invariance of the L2 normalisation.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import chunked

EPS = 1e-6


def _rand_case(rng, T, H, dk, dv, gate_mean=-2.0):
    q = rng.normal(size=(T, H, dk))
    k = rng.normal(size=(T, H, dk))
    v = rng.normal(size=(T, H, dv))
    b = rng.normal(size=(T, H))
    g = -np.logaddexp(0.0, rng.normal(gate_mean, 1.0, size=(T, H, dk)))
    return q, k, v, g, b


def _prep(q, k, g, b, eps=EPS):
    qh = q / np.sqrt(np.linalg.norm(q, axis=-1, keepdims=True) ** 2 + eps)
    kh = k / np.sqrt(np.linalg.norm(k, axis=-1, keepdims=True) ** 2 + eps)
    return qh, kh, np.exp(g), expit(b)


# ------------------------------------------------------------ forward pins
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_unrolled_products(seed):
    """S_t = (M_t...M_1) S_0 + sum_s (M_t...M_{s+1}) beta_s kh_s v_s^T with
    M_t = (I - beta_t kh_t kh_t^T) Diag(alpha_t), o_t = S_t^T qh_t."""
    rng = np.random.default_rng(seed)
    T, H, dk, dv = 8, 2, 5, 3
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv, gate_mean=0.0)
    s0 = rng.normal(size=(1, H, dk, dv))
    o, sf = oracle.fwd(q, k, v, g, b, initial_state=s0, eps=EPS)
    qh, kh, al, be = _prep(q, k, g, b)
    for h in range(H):
        M = [(np.eye(dk) - be[t, h] * np.outer(kh[t, h], kh[t, h])) @ np.diag(al[t, h]) for t in range(T)]
        for t in range(T):
            P = np.eye(dk)                                  # P = M_t ... M_0
            for s in range(t + 1):
                P = M[s] @ P
            St = P @ s0[0, h]
            for s in range(t + 1):
                Q = np.eye(dk)
                for r in range(s + 1, t + 1):
                    Q = M[r] @ Q
                St = St + Q @ (be[s, h] * np.outer(kh[s, h], v[s, h]))
            np.testing.assert_allclose(o[t, h], St.T @ qh[t, h], rtol=1e-12, atol=1e-13)
            if t == T - 1:
                np.testing.assert_allclose(sf[0, h], St, rtol=1e-12, atol=1e-13)


def test_beta_zero_is_pure_decay():
    """beta = 0: S_t = Diag(prod_{s<=t} alpha_s) S_0, o_t = S_t^T qh_t."""
    rng = np.random.default_rng(3)
    T, H, dk, dv = 40, 2, 6, 4
    qh = rng.normal(size=(T, H, dk))
    kh = rng.normal(size=(T, H, dk))
    v = rng.normal(size=(T, H, dv))
    alpha = rng.uniform(0.5, 1.0, size=(T, H, dk))
    beta = np.zeros((T, H))
    s0 = rng.normal(size=(1, H, dk, dv))
    o, sf = oracle.fwd_core(qh, kh, v, alpha, beta, initial_state=s0)
    cp = np.cumprod(alpha, axis=0)                      # [T, H, dk]
    St = cp[:, :, :, None] * s0[0][None]                 # [T, H, dk, dv]
    np.testing.assert_allclose(o, np.einsum("thkv,thk->thv", St, qh), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sf[0], St[-1], rtol=1e-12, atol=1e-14)


def test_alpha_one_is_ungated_delta_rule():
    """alpha = 1: the Widrow-Hoff / LMS delta rule S <- S + beta k (v - S^T k)^T."""
    rng = np.random.default_rng(4)
    T, H, dk, dv = 30, 1, 7, 5
    kh = rng.normal(size=(T, H, dk))
    qh = rng.normal(size=(T, H, dk))
    v = rng.normal(size=(T, H, dv))
    beta = rng.uniform(0, 1, size=(T, H))
    o, sf = oracle.fwd_core(qh, kh, v, np.ones((T, H, dk)), beta)
    S = np.zeros((dk, dv))
    for t in range(T):
        err = v[t, 0] - S.T @ kh[t, 0]
        S = S + beta[t, 0] * np.outer(kh[t, 0], err)
        np.testing.assert_allclose(o[t, 0], S.T @ qh[t, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sf[0, 0], S, rtol=1e-12, atol=1e-13)


def test_beta_one_writes_exactly():
    """beta = 1 with a unit key: right after the write S_t^T kh_t = v_t,
    whatever the gate, because (I - kh kh^T) annihilates kh."""
    rng = np.random.default_rng(5)
    T, H, dk, dv = 25, 2, 8, 6
    kh = rng.normal(size=(T, H, dk))
    kh /= np.linalg.norm(kh, axis=-1, keepdims=True)
    v = rng.normal(size=(T, H, dv))
    alpha = rng.uniform(0.2, 1.0, size=(T, H, dk))
    s0 = rng.normal(size=(1, H, dk, dv))
    # query with the key itself: o_t = S_t^T kh_t must equal v_t
    o, _ = oracle.fwd_core(kh, kh, v, alpha, np.ones((T, H)), initial_state=s0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_exact_recall():
    """beta = 1, alpha = 1, orthonormal keys, S_0 = 0: S = sum_i k_i v_i^T, so
    every stored value is recalled exactly by its key."""
    rng = np.random.default_rng(6)
    dk, dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.normal(size=(dk, dk)))
    kh = Qm.T[:, None, :]                               # T = dk orthonormal keys
    v = rng.normal(size=(T, 1, dv))
    _, sf = oracle.fwd_core(kh, kh, v, np.ones((T, 1, dk)), np.ones((T, 1)))
    np.testing.assert_allclose(sf[0, 0], sum(np.outer(kh[i, 0], v[i, 0]) for i in range(T)), atol=1e-13)
    np.testing.assert_allclose(sf[0, 0].T @ kh[:, 0, :].T, v[:, 0, :].T, atol=1e-13)


def test_prep_matches_library_routines():
    """Raw-input forward == prepared forward fed with numpy's L2 norm,
    scipy's expit (sigmoid) and numpy's exp."""
    rng = np.random.default_rng(7)
    T, H, dk, dv = 50, 3, 16, 8
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    o1, s1 = oracle.fwd(q, k, v, g, b, eps=EPS)
    qh, kh, al, be = _prep(q, k, g, b)
    o2, s2 = oracle.fwd_core(qh, kh, v, al, be)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-14)


def test_causality():
    """Changing tokens after t leaves o_<=t unchanged (bitwise)."""
    rng = np.random.default_rng(8)
    T, H, dk, dv = 64, 2, 8, 8
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    o1, _ = oracle.fwd(q, k, v, g, b)
    for x in (q, k, v, g):
        x[40:] = rng.normal(size=x[40:].shape)
    b[40:] = 3.0
    o2, _ = oracle.fwd(q, k, v, g, b)
    assert np.array_equal(o1[:40], o2[:40])
    assert not np.allclose(o1[40:], o2[40:])


def test_varlen_equals_separate_calls_and_state_carry():
    rng = np.random.default_rng(9)
    H, dk, dv = 2, 8, 6
    lens = [17, 1, 64, 30]
    T = sum(lens)
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    s0 = rng.normal(size=(len(lens), H, dk, dv))
    o, sf = oracle.fwd(q, k, v, g, b, cu_seqlens=cu, initial_state=s0)
    for n in range(len(lens)):
        a, z = cu[n], cu[n + 1]
        on, sn = oracle.fwd(q[a:z], k[a:z], v[a:z], g[a:z], b[a:z], initial_state=s0[n:n + 1])
        np.testing.assert_array_equal(o[a:z], on)
        np.testing.assert_array_equal(sf[n], sn[0])
    # two calls chained through the state equal one call
    a = 23
    o1, s1 = oracle.fwd(q[:a], k[:a], v[:a], g[:a], b[:a])
    o2, s2 = oracle.fwd(q[a:], k[a:], v[a:], g[a:], b[a:], initial_state=s1)
    o_all, s_all = oracle.fwd(q, k, v, g, b)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o_all, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, s_all, rtol=1e-13, atol=1e-14)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(10)
    T, H, dk, dv = 100, 3, 16, 32
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    o1, s1 = oracle.fwd(q, k, v, g, b, threads=1)
    o8, s8 = oracle.fwd(q, k, v, g, b, threads=8)
    assert np.array_equal(o1, o8) and np.array_equal(s1, s8)


# --------------------------------------------------------- chunked algebra
@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64, 128])
def test_chunk_size_invariance(C):
    rng = np.random.default_rng(11)
    H, dk, dv = 2, 8, 6
    lens = [150, 1, 63, 66]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    s0 = 0.1 * rng.normal(size=(len(lens), H, dk, dv))
    o_ref, s_ref = oracle.fwd(q, k, v, g, b, cu_seqlens=cu, initial_state=s0)
    o_c, s_c = chunked.fwd(q, k, v, g, b, cu_seqlens=cu, initial_state=s0, chunk=C)
    scale = np.abs(o_ref).max()
    assert np.abs(o_c - o_ref).max() <= 1e-11 * scale
    assert np.abs(s_c - s_ref).max() <= 1e-11 * np.abs(s_ref).max()


def test_chunk_T_is_inverse():
    rng = np.random.default_rng(12)
    q, k, v, g, b = _rand_case(rng, 64, 1, 16, 8)
    _, _, kept = chunked.fwd(q, k, v, g, b, chunk=64, keep_stages=True)
    st = kept[0][3]
    Akk = st["Akk"]
    assert np.all(np.triu(Akk) == 0)
    np.testing.assert_allclose(st["T"], np.linalg.inv(np.eye(64) + Akk), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------ gradient pins
def _loss(o, sf, dO, dS):
    return float(np.sum(o * dO) + np.sum(sf * dS))


@pytest.mark.parametrize("lens", [[13], [5, 9]])
def test_backward_matches_central_differences(lens):
    rng = np.random.default_rng(13)
    H, dk, dv = 2, 4, 3
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv, gate_mean=-1.0)
    N = len(lens)
    s0 = rng.normal(size=(N, H, dk, dv))
    dO = rng.normal(size=(T, H, dv))
    dS = rng.normal(size=(N, H, dk, dv))
    gr = oracle.bwd(q, k, v, g, b, dO, cu_seqlens=cu, initial_state=s0, dS_final=dS)
    inputs = {"q": q, "k": k, "v": v, "g": g, "b": b, "s0": s0}
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "b": "db", "s0": "dS0"}
    h = 1e-6
    for name, x in inputs.items():
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*oracle.fwd(q, k, v, g, b, cu_seqlens=cu, initial_state=s0), dO, dS)
            x[idx] = old - h
            lm = _loss(*oracle.fwd(q, k, v, g, b, cu_seqlens=cu, initial_state=s0), dO, dS)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - gr[names[name]]).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 1e-7, (name, err)


@pytest.mark.parametrize("logit", [-40.0, -30.0, 0.5, 30.0, 40.0])
def test_single_token_beta_gradient_closed_form(logit):
    """One token from the zero state: S_1 = beta kh v^T and o = beta (kh . qh) v,
    so dL/db = sigma'(b) (kh . qh) (v . dO) for L = <dO, o>.  sigma'(b) is taken
    as 1 / (2 + 2 cosh b), which has no cancellation at large |b|, so the pin
    holds to fp64 rounding even where 1 - sigma(b) is below 1e-13."""
    rng = np.random.default_rng(11)
    dk, dv = 8, 6
    q, k, v, g, _ = _rand_case(rng, 1, 1, dk, dv)
    b = np.full((1, 1), logit)
    dO = rng.normal(size=(1, 1, dv))
    qh, kh, _, _ = _prep(q, k, g, b)
    want = (kh[0, 0] @ qh[0, 0]) * (v[0, 0] @ dO[0, 0]) / (2.0 + 2.0 * np.cosh(logit))
    got = oracle.bwd(q, k, v, g, b, dO)["db"][0, 0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_core_backward_matches_central_differences():
    """Gradients with respect to prepared inputs (alpha, beta directly)."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 9, 1, 3, 2
    qh, kh, v = rng.normal(size=(T, H, dk)), rng.normal(size=(T, H, dk)), rng.normal(size=(T, H, dv))
    alpha = rng.uniform(0.3, 1.0, size=(T, H, dk))
    beta = rng.uniform(0.0, 1.0, size=(T, H))
    s0 = rng.normal(size=(1, H, dk, dv))
    dO = rng.normal(size=(T, H, dv))
    dS = rng.normal(size=(1, H, dk, dv))
    gr = oracle.bwd_core(qh, kh, v, alpha, beta, dO, initial_state=s0, dS_final=dS)
    h = 1e-6
    for name, x, key in (("qh", qh, "dqh"), ("kh", kh, "dkh"), ("alpha", alpha, "dalpha"),
                         ("beta", beta, "dbeta"), ("v", v, "dv")):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = x[idx]
            x[idx] = old + h
            lp = _loss(*oracle.fwd_core(qh, kh, v, alpha, beta, initial_state=s0), dO, dS)
            x[idx] = old - h
            lm = _loss(*oracle.fwd_core(qh, kh, v, alpha, beta, initial_state=s0), dO, dS)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        err = np.abs(fd - gr[key]).max() / np.abs(fd).max()
        assert err < 1e-7, (name, err)


def test_adjoint_identity_and_norm_scale_invariance():
    """o and S_T are homogeneous-linear in (v, S_0), so
    <dv, v> + <dS0, S0> = <dO, o> + <dS_T, S_T>.  And each q_t enters only
    through q_t/|q_t| (up to eps), so q_t . dq_t ~ 0 (likewise k)."""
    rng = np.random.default_rng(15)
    lens = [300, 212]
    T, H, dk, dv = sum(lens), 2, 32, 24
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    s0 = 0.1 * rng.normal(size=(2, H, dk, dv))
    dO = rng.normal(size=(T, H, dv))
    dS = 0.1 * rng.normal(size=(2, H, dk, dv))
    o, sf = oracle.fwd(q, k, v, g, b, cu_seqlens=cu, initial_state=s0)
    gr = oracle.bwd(q, k, v, g, b, dO, cu_seqlens=cu, initial_state=s0, dS_final=dS)
    lhs = np.sum(gr["dv"] * v) + np.sum(gr["dS0"] * s0)
    rhs = np.sum(dO * o) + np.sum(dS * sf)
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + abs(rhs))
    for x, dx in ((q, gr["dq"]), (k, gr["dk"])):
        dots = np.abs(np.sum(x * dx, axis=-1))
        scale = np.linalg.norm(x, axis=-1) * np.linalg.norm(dx, axis=-1)
        assert np.all(dots <= 1e-6 * scale + 1e-15)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_backward_matches_token_backward(C):
    """The chunk-level backward (the algebra the GPU kernels implement) equals
    the token-level reverse-mode oracle, itself pinned by finite differences."""
    rng = np.random.default_rng(16)
    H, dk, dv = 2, 8, 6
    lens = [150, 1, 70]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, b = _rand_case(rng, T, H, dk, dv)
    s0 = 0.1 * rng.normal(size=(len(lens), H, dk, dv))
    dO = rng.normal(size=(T, H, dv))
    dS = 0.1 * rng.normal(size=(len(lens), H, dk, dv))
    ref = oracle.bwd(q, k, v, g, b, dO, cu_seqlens=cu, initial_state=s0, dS_final=dS)
    got = chunked.bwd(q, k, v, g, b, dO, cu_seqlens=cu, initial_state=s0, dS_final=dS, chunk=C)
    for name in ("dq", "dk", "dv", "dg", "db", "dS0"):
        err = np.abs(got[name] - ref[name]).max() / np.abs(ref[name]).max()
        assert err < 1e-10, (name, err)
