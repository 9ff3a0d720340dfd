"""Chunked form of the KDA forward in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

The pages organise KDA as intra-chunk processing plus inter-chunk state
passing ("TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
practice", section "KDA pre/post-processing fusion").  The chunking changes only
how the work is grouped, not the result, so this module is checked against the
token recurrence in ``oracle.fwd`` for every chunk size (chunk-size
invariance).  It exists to pin that algebra and to expose the per-chunk
intermediate matrices for stage-by-stage comparison.

For one chunk of C tokens entering with state S (rows r, s = 0..C-1, G the
inclusive cumulative sum of g inside the chunk, Gam = exp(G)):

    Akk[r, s] = beta_r sum_c kh[r,c] kh[s,c] exp(G[r,c] - G[s,c])   (s < r)
    T         = (I + Akk)^{-1}
    W         = T diag(beta) (kh * Gam),     Ut = T diag(beta) v
    U         = Ut - W S
    Aqk[r, s] = sum_c qh[r,c] kh[s,c] exp(G[r,c] - G[s,c])          (s <= r)
    O         = (qh * Gam) S + Aqk U
    S_next    = Diag(Gam[C-1]) S + (kh * exp(G[C-1] - G))^T U

The exponentials of gate differences are evaluated directly (no factoring into
exp(G_r) * exp(-G_s)), and T comes from a plain triangular solve.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def _prep(q, k, b, eps):
    qh = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    kh = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    beta = 1.0 / (1.0 + np.exp(-b))
    return qh, kh, beta


def chunk_step(qh, kh, v, g, beta, S):
    """One chunk.  qh, kh, g: [C, dk]; v: [C, dv]; beta: [C]; S: [dk, dv].

    Returns (O, S_next, stages) with the intermediate matrices in ``stages``."""
    C = qh.shape[0]
    G = np.cumsum(g, axis=0)
    diff = G[:, None, :] - G[None, :, :]                      # [r, s, c] = G_r - G_s
    lower_incl = np.tril(np.ones((C, C), dtype=bool))
    lower_strict = np.tril(np.ones((C, C), dtype=bool), -1)
    E = np.exp(np.where(lower_incl[:, :, None], diff, 0.0))   # only s <= r is used
    kk = np.einsum("rc,sc,rsc->rs", kh, kh, E)
    qk = np.einsum("rc,sc,rsc->rs", qh, kh, E)
    Akk = np.where(lower_strict, beta[:, None] * kk, 0.0)
    Aqk = np.where(lower_incl, qk, 0.0)
    T = solve_triangular(np.eye(C) + Akk, np.eye(C), lower=True, unit_diagonal=True)
    Gam = np.exp(G)
    W = T @ (beta[:, None] * kh * Gam)
    Ut = T @ (beta[:, None] * v)
    U = Ut - W @ S
    O = (qh * Gam) @ S + Aqk @ U
    Ktil = kh * np.exp(G[-1][None, :] - G)
    S_next = np.exp(G[-1])[:, None] * S + Ktil.T @ U
    stages = {"G": G, "Akk": Akk, "T": T, "W": W, "Ut": Ut, "U": U, "Aqk": Aqk, "S_in": S.copy()}
    return O, S_next, stages


def fwd(q, k, v, g, b, cu_seqlens=None, initial_state=None, eps=1e-6, chunk=64, keep_stages=False):
    """Chunked forward from raw inputs (same contract as ``oracle.fwd``).

    Chunks restart at every document start; the last chunk of a document may be
    shorter.  With ``keep_stages`` the per-chunk matrices are returned as a list
    of (seq, head, chunk_start, stages) tuples."""
    q, k, v, g, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    qh, kh, beta = _prep(q, k, b, eps)
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dk, dv))
    kept = []
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                O, S, st = chunk_step(qh[c0:c1, h], kh[c0:c1, h], v[c0:c1, h], g[c0:c1, h], beta[c0:c1, h], S)
                o[c0:c1, h] = O
                if keep_stages:
                    kept.append((n, h, c0, st))
            sf[n, h] = S
    if keep_stages:
        return o, sf, kept
    return o, sf


def chunk_bwd(qh, kh, v, g, beta, S0, dO, dS1):
    """Backward of ``chunk_step`` for one chunk, given the entering state S0,
    the output gradient dO [C, dv] and dS1 = dL/d(state after the chunk).

    Returns (grads, dS0) with grads = dict(dqh, dkh, dv, dg, dbeta) for the
    chunk's tokens (with respect to the prepared inputs: unit qh, kh, the
    log-decay g and beta itself).  Written out step by step from the chunk
    equations in this module's docstring."""
    C = qh.shape[0]
    G = np.cumsum(g, axis=0)
    Gam = np.exp(G)
    GC = G[-1]
    lower_incl = np.tril(np.ones((C, C), dtype=bool))
    lower_strict = np.tril(np.ones((C, C), dtype=bool), -1)
    QG, KG, KI, Kt = qh * Gam, beta[:, None] * kh * Gam, kh / Gam, kh * np.exp(GC[None, :] - G)
    Akk = np.where(lower_strict, KG @ KI.T, 0.0)
    Aqk = np.where(lower_incl, QG @ KI.T, 0.0)
    T = solve_triangular(np.eye(C) + Akk, np.eye(C), lower=True, unit_diagonal=True)
    W = T @ KG
    BV = beta[:, None] * v
    U = T @ BV - W @ S0
    # reverse
    dU = Aqk.T @ dO + Kt @ dS1
    dS0 = np.exp(GC)[:, None] * dS1 + QG.T @ dO - W.T @ dU
    dQG = dO @ S0.T
    dAqk = np.where(lower_incl, dO @ U.T, 0.0)
    dKt = U @ dS1.T
    dGamC = np.sum(S0 * dS1, axis=1)
    dW = -dU @ S0.T
    dT = dU @ BV.T + dW @ KG.T
    dBV = T.T @ dU
    dKG = T.T @ dW
    dAkk = np.where(lower_strict, -T.T @ dT @ T.T, 0.0)
    dKG += dAkk @ KI
    dKI = dAkk.T @ KG + dAqk.T @ QG
    dQG += dAqk @ KI
    dv = beta[:, None] * dBV
    dbeta = np.sum(v * dBV, axis=1) + np.sum(dKG * kh * Gam, axis=1)
    dqh = dQG * Gam
    dkh = beta[:, None] * Gam * dKG + dKI / Gam + dKt * np.exp(GC[None, :] - G)
    dG = dQG * QG + dKG * KG - dKI * KI - dKt * Kt
    dGC = np.sum(dKt * Kt, axis=0) + dGamC * np.exp(GC)
    dG[-1] += dGC
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return {"dqh": dqh, "dkh": dkh, "dv": dv, "dg": dg, "dbeta": dbeta, "dU": dU}, dS0


def bwd(q, k, v, g, b, dO, cu_seqlens=None, initial_state=None, dS_final=None, eps=1e-6, chunk=64):
    """Chunked backward from raw inputs (same contract as ``oracle.bwd``):
    a forward pass records the state entering every chunk, then a reverse pass
    over the chunks applies ``chunk_bwd`` and carries dL/dS backwards.  The
    chain rule through the L2 norm and the sigmoid closes it."""
    q, k, v, g, b, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b, dO))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.size - 1
    nq = np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    nk = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    qh, kh, beta = q / nq, k / nk, 1.0 / (1.0 + np.exp(-b))
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("db", b))}
    dS0_all = np.zeros((N, H, dk, dv))
    dqh = np.zeros_like(q)
    dkh = np.zeros_like(k)
    dbeta = np.zeros_like(b)
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[n, h], dtype=np.float64)
            starts = list(range(t0, t1, chunk))
            states = []
            for c0 in starts:
                c1 = min(c0 + chunk, t1)
                states.append(S)
                _, S, _ = chunk_step(qh[c0:c1, h], kh[c0:c1, h], v[c0:c1, h], g[c0:c1, h], beta[c0:c1, h], S)
            dS = np.zeros((dk, dv)) if dS_final is None else np.array(dS_final[n, h], dtype=np.float64)
            for c0, S0 in zip(starts[::-1], states[::-1]):
                c1 = min(c0 + chunk, t1)
                gr, dS = chunk_bwd(qh[c0:c1, h], kh[c0:c1, h], v[c0:c1, h], g[c0:c1, h], beta[c0:c1, h], S0,
                                   dO[c0:c1, h], dS)
                dqh[c0:c1, h], dkh[c0:c1, h] = gr["dqh"], gr["dkh"]
                out["dv"][c0:c1, h], out["dg"][c0:c1, h], dbeta[c0:c1, h] = gr["dv"], gr["dg"], gr["dbeta"]
            dS0_all[n, h] = dS
    out["dq"] = (dqh - qh * np.sum(qh * dqh, axis=-1, keepdims=True)) / nq
    out["dk"] = (dkh - kh * np.sum(kh * dkh, axis=-1, keepdims=True)) / nk
    out["db"] = dbeta * beta * (1.0 - beta)
    out["dS0"] = dS0_all
    return out
