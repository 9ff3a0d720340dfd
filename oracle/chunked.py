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
