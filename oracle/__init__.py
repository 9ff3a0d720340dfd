"""fp64 CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and it shares no code with the GPU library.

Contents
--------
* ``fwd`` / ``bwd`` -- the token-by-token recurrence and its reverse-mode
  backward in double precision (C, ``kda_oracle.c``; threads over
  (sequence, head) chains).  This is the oracle of record.
* ``fwd_core`` / ``bwd_core`` -- the same recurrence on prepared inputs
  (unit q/k, alpha and beta given directly), so special cases such as
  beta = 0 or alpha = 1 can be pinned exactly.
* ``oracle.chunked`` -- the chunked (intra-chunk + inter-chunk) form written out
  in numpy fp64, for chunk-size invariance and for stage-by-stage comparison.

Sources: "TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
practice" (jinguxun.com news 11080097), sections "Kimi K3.1 Pro model
structure" (KDA is a gated matrix-state recurrence) and "KDA pre/post-processing
fusion" (Q/K normalisation, beta transform and gating in the forward; backward
through the saved normalisation statistics).  The recurrence taken as the
reading of those words is written out in ``kda_oracle.c``.

Layouts: q, k, g ``[T, H, dk]``; v, o ``[T, H, dv]``; b ``[T, H]``;
states ``[N, H, dk, dv]``; ``cu_seqlens`` ``[N + 1]`` (int64).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_ORACLE_LIB names another build of kda_oracle.c (the sanitizer test loads
# an AddressSanitizer / UndefinedBehaviorSanitizer build this way)
_LIB_PATH = os.environ.get("KDA_ORACLE_LIB") or os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.POINTER(ctypes.c_int64)


def build(verbose: bool = False) -> str:
    """Compile ``kda_oracle.c`` into ``libkda_oracle.so`` with gcc."""
    import subprocess

    src = os.path.join(_HERE, "kda_oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", tmp, src, "-lpthread", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    common = [ctypes.c_int64, ctypes.c_int, _I64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.kda_oracle_fwd.argtypes = common + [_D] * 6 + [ctypes.c_double, _D, _D, ctypes.c_int]
    lib.kda_oracle_fwd.restype = ctypes.c_int
    lib.kda_oracle_fwd_core.argtypes = common + [_D] * 6 + [_D, _D, ctypes.c_int]
    lib.kda_oracle_fwd_core.restype = ctypes.c_int
    lib.kda_oracle_bwd.argtypes = common + [_D] * 6 + [ctypes.c_double] + [_D] * 8 + [ctypes.c_int]
    lib.kda_oracle_bwd.restype = ctypes.c_int
    lib.kda_oracle_bwd_core.argtypes = common + [_D] * 6 + [_D] * 8 + [ctypes.c_int]
    lib.kda_oracle_bwd_core.restype = ctypes.c_int
    _lib = lib
    return lib


MAX_THREADS = 16  # the CPU share a one-GPU machine grants, whatever the host reports


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_THREADS))


def _f64(x):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _ptr(a):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return cu


def _shapes(q, v):
    if q.ndim != 3 or v.ndim != 3 or q.shape[:2] != v.shape[:2]:
        raise ValueError("q/k/g must be [T,H,dk] and v [T,H,dv]")
    T, H, dk = q.shape
    return T, H, dk, v.shape[2]


def fwd(q, k, v, g, b, cu_seqlens=None, initial_state=None, eps=1e-6, threads=None):
    """Token-by-token KDA forward in fp64 from raw inputs.

    q, k: raw (the oracle L2-normalises them); g: log-decay (alpha = exp(g));
    b: beta logit (beta = sigmoid(b)).  Returns ``(o, final_state)``."""
    q, k, v, g, b = (_f64(x) for x in (q, k, v, g, b))
    T, H, dk, dv = _shapes(q, v)
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    s0 = _f64(initial_state)
    if s0 is not None and s0.shape != (N, H, dk, dv):
        raise ValueError("initial_state must be [N,H,dk,dv]")
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dk, dv))
    rc = _load().kda_oracle_fwd(T, N, cu.ctypes.data_as(_I64), H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(g), _ptr(b), _ptr(s0), float(eps), _ptr(o), _ptr(sf),
                                int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd failed ({rc})")
    return o, sf


def fwd_core(qh, kh, v, alpha, beta, cu_seqlens=None, initial_state=None, threads=None):
    """Recurrence on prepared inputs: qh, kh used as given, alpha [T,H,dk] and
    beta [T,H] used directly.  Returns ``(o, final_state)``."""
    qh, kh, v, alpha, beta = (_f64(x) for x in (qh, kh, v, alpha, beta))
    T, H, dk, dv = _shapes(qh, v)
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    s0 = _f64(initial_state)
    o = np.zeros((T, H, dv))
    sf = np.zeros((N, H, dk, dv))
    rc = _load().kda_oracle_fwd_core(T, N, cu.ctypes.data_as(_I64), H, dk, dv, _ptr(qh), _ptr(kh),
                                     _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0), _ptr(o), _ptr(sf),
                                     int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_fwd_core failed ({rc})")
    return o, sf


def bwd(q, k, v, g, b, dO, cu_seqlens=None, initial_state=None, dS_final=None, eps=1e-6,
        threads=None):
    """Reverse-mode gradients of ``fwd`` for the loss <dO, o> + <dS_final, S_T>.

    Returns a dict with dq, dk, dv, dg, db (same shapes as the inputs) and
    dS0 ([N,H,dk,dv])."""
    q, k, v, g, b, dO = (_f64(x) for x in (q, k, v, g, b, dO))
    T, H, dk, dv = _shapes(q, v)
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    s0, dsf = _f64(initial_state), _f64(dS_final)
    out = {
        "dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
        "dg": np.zeros((T, H, dk)), "db": np.zeros((T, H)), "dS0": np.zeros((N, H, dk, dv)),
    }
    rc = _load().kda_oracle_bwd(T, N, cu.ctypes.data_as(_I64), H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(g), _ptr(b), _ptr(s0), float(eps), _ptr(dO), _ptr(dsf),
                                _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                _ptr(out["db"]), _ptr(out["dS0"]), int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd failed ({rc})")
    return out


def bwd_core(qh, kh, v, alpha, beta, dO, cu_seqlens=None, initial_state=None, dS_final=None,
             threads=None):
    """Gradients of ``fwd_core`` with respect to qh, kh, v, alpha, beta, S0."""
    qh, kh, v, alpha, beta, dO = (_f64(x) for x in (qh, kh, v, alpha, beta, dO))
    T, H, dk, dv = _shapes(qh, v)
    cu = _cu(cu_seqlens, T)
    N = cu.size - 1
    s0, dsf = _f64(initial_state), _f64(dS_final)
    out = {
        "dqh": np.zeros((T, H, dk)), "dkh": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
        "dalpha": np.zeros((T, H, dk)), "dbeta": np.zeros((T, H)), "dS0": np.zeros((N, H, dk, dv)),
    }
    rc = _load().kda_oracle_bwd_core(T, N, cu.ctypes.data_as(_I64), H, dk, dv, _ptr(qh), _ptr(kh),
                                     _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0), _ptr(dO), _ptr(dsf),
                                     _ptr(out["dqh"]), _ptr(out["dkh"]), _ptr(out["dv"]),
                                     _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dS0"]),
                                     int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd_core failed ({rc})")
    return out
