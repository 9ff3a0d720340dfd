"""Seeded synthetic inputs for the KDA workloads.

This module only draws random numbers and rounds them to the run's storage
type.  It holds none of KDA's arithmetic, so both the GPU path's tests and the
fp64 oracle can consume the same inputs without sharing any method code.

Recipe (every value drawn in float64 with NumPy's PCG64, then rounded
round-to-nearest-even to float32 and, for bf16 runs, to bfloat16):

* generator per (workload seed, tensor id, 65,536-token block):
  ``numpy.random.default_rng([seed, tensor_id, block])`` -- so a long sequence
  can be produced block by block;
* q, k, v, b (beta logit), dO ~ N(0, 1);
* g (log-decay) = -softplus(x), x ~ N(-2, 1), so alpha = exp(g) lies in (0, 1);
* initial state S0 and dS_final ~ N(0, 0.01) (standard deviation 0.1), fp32;
* packed documents: lengths ~ lognormal(6.5, 1), rescaled to the total token
  count (floored, at least 1, remainder to the largest fractional parts);
* gate-range mix (``mix_gates``): per head, one channel in three keeps the
  draw above, one in three has g = 0 (no decay) and one in three fast-forgetting
  g ~ U(-8, -2) per token (a 64-token chunk then decays by e^-128 .. e^-512).

Arrays are returned as float32 whose values are exactly representable in the
run dtype; the oracle upcasts them exactly to float64.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 1 << 16
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "b": 3, "g": 4, "s0": 5, "dO": 6, "dS": 7, "doclen": 8, "gmix": 9}

# The five workloads: shapes, dtypes and which tensors exist.
WORKLOADS = {
    0: dict(name="kda-fwd-fp32-B1-H2-T256-d64", dtype="f32", B=1, H=2, T=256, dk=64, dv=64,
            chunk=64, s0=False, bwd=False, varlen=False),
    1: dict(name="kda-fwd-bf16-B1-H16-T4096-d128", dtype="bf16", B=1, H=16, T=4096, dk=128, dv=128,
            chunk=64, s0=True, bwd=False, varlen=False),
    2: dict(name="kda-fwdbwd-bf16-B4-H32-T8192-d128", dtype="bf16", B=4, H=32, T=8192, dk=128,
            dv=128, chunk=64, s0=True, bwd=True, varlen=False),
    3: dict(name="kda-fwd-bf16-B1-H16-T1048576-d128", dtype="bf16", B=1, H=16, T=1 << 20, dk=128,
            dv=128, chunk=64, s0=True, bwd=False, varlen=False),
    4: dict(name="kda-varlen-fwdbwd-bf16-H32-T65536-64docs-d128", dtype="bf16", B=64, H=32,
            T=65536, dk=128, dv=128, chunk=64, s0=True, bwd=True, varlen=True),
}


def round_bf16(x) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even via float32); returns float32.

    Finite inputs only: the 32-bit sum below cannot carry out of a finite
    float32's bit pattern."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r &= 0xFFFF0000
    return r.view(np.float32).reshape(f.shape)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_tokens(seed, tid, T, tail_shape, dtype, mean=0.0, std=1.0, transform=None):
    """[T, *tail_shape] float32: normals drawn in float64 in 65,536-token
    blocks, each passed through ``transform`` (elementwise, float64) and
    rounded to ``dtype``.  Blocks have their own generators, so they are drawn
    in parallel threads; inside a block the stream is consumed in order through
    one small reused buffer.  The values depend on neither."""
    tail = tuple(tail_shape)
    out = np.empty((T,) + tail, dtype=np.float32)
    step = max(1, (1 << 21) // max(1, int(np.prod(tail, dtype=np.int64))))

    def one(blk):
        a, z = blk * BLOCK, min((blk + 1) * BLOCK, T)
        rng = np.random.default_rng([seed, tid, blk])
        buf = np.empty((min(step, z - a),) + tail, dtype=np.float64)
        for s in range(a, z, step):
            x = buf[: min(step, z - s)]
            rng.standard_normal(out=x)   # the same stream as rng.normal(mean, std, size)
            x *= std
            x += mean
            if transform is not None:
                x = transform(x)
            out[s : s + x.shape[0]] = round_to(x, dtype)

    nblk = (T + BLOCK - 1) // BLOCK
    if nblk <= 1:
        for blk in range(nblk):
            one(blk)
    else:
        with ThreadPoolExecutor(max_workers=min(_workers(), nblk)) as ex:
            list(ex.map(one, range(nblk)))
    return out


def mix_gates(g: np.ndarray, seed: int, dtype: str, offset: int = 0) -> np.ndarray:
    """g [T, H, dk] with the gate-range mix applied per head: channel c with
    (c + h + offset) % 3 == 0 keeps its value, == 1 is set to 0, == 2 is drawn
    from U(-8, -2) (rounded to ``dtype``)."""
    T, H, dk = g.shape
    rng = np.random.default_rng([seed, TENSOR_IDS["gmix"], 0])
    fast = round_to(rng.uniform(-8.0, -2.0, size=g.shape), dtype)
    kind = (np.arange(dk)[None, :] + np.arange(H)[:, None] + offset) % 3   # [H, dk]
    out = np.array(g, dtype=np.float32, copy=True)
    out = np.where(kind[None] == 1, np.float32(0.0), out)
    out = np.where(kind[None] == 2, fast, out)
    return out.astype(np.float32)


def doc_lengths(seed: int, ndocs: int, total: int) -> np.ndarray:
    """Lognormal(6.5, 1) document lengths rescaled to sum exactly to ``total``."""
    rng = np.random.default_rng([seed, TENSOR_IDS["doclen"], 0])
    L = rng.lognormal(6.5, 1.0, size=ndocs)
    x = L * (total / L.sum())
    n = np.maximum(np.floor(x).astype(np.int64), 1)
    rem = int(total - n.sum())
    if rem > 0:
        frac = x - np.floor(x)
        order = sorted(range(ndocs), key=lambda i: (-frac[i], i))
        for i in order[:rem]:
            n[i] += 1
    elif rem < 0:  # only if the floor-at-1 pushed the sum over; take from the longest
        for _ in range(-rem):
            n[int(np.argmax(n))] -= 1
    assert n.sum() == total and n.min() >= 1
    return n


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def generate(seed: int, T: int, H: int, dk: int, dv: int, dtype: str, num_seqs: int = 1,
             with_s0: bool = True, with_grads: bool = False, tensors=None):
    """Inputs for a packed token stream of T tokens over ``num_seqs`` sequences.

    Returns a dict of float32 arrays: q, k, g [T,H,dk]; v [T,H,dv]; b [T,H];
    optionally s0 [N,H,dk,dv], dO [T,H,dv], dS [N,H,dk,dv]."""
    want = set(tensors) if tensors is not None else None

    def need(name):
        return want is None or name in want

    out = {}
    if need("q"):
        out["q"] = _normal_tokens(seed, TENSOR_IDS["q"], T, (H, dk), dtype)
    if need("k"):
        out["k"] = _normal_tokens(seed, TENSOR_IDS["k"], T, (H, dk), dtype)
    if need("v"):
        out["v"] = _normal_tokens(seed, TENSOR_IDS["v"], T, (H, dv), dtype)
    if need("b"):
        out["b"] = _normal_tokens(seed, TENSOR_IDS["b"], T, (H,), dtype)
    if need("g"):
        # -softplus(x), x ~ N(-2, 1)
        out["g"] = _normal_tokens(seed, TENSOR_IDS["g"], T, (H, dk), dtype, mean=-2.0,
                                  transform=lambda x: -np.logaddexp(0.0, x))
    if with_s0 and need("s0"):
        rng = np.random.default_rng([seed, TENSOR_IDS["s0"], 0])
        out["s0"] = rng.normal(0.0, 0.1, size=(num_seqs, H, dk, dv)).astype(np.float32)
    if with_grads:
        if need("dO"):
            out["dO"] = _normal_tokens(seed, TENSOR_IDS["dO"], T, (H, dv), dtype)
        if need("dS"):
            rng = np.random.default_rng([seed, TENSOR_IDS["dS"], 0])
            out["dS"] = rng.normal(0.0, 0.1, size=(num_seqs, H, dk, dv)).astype(np.float32)
    return out


def workload(idx: int, tensors=None, T=None, B=None, H=None):
    """Inputs of workload ``idx`` (0..4).  T, B, H may be overridden to get a
    smaller case with the same distributions.  Returns (spec, cu_seqlens, arrays)."""
    spec = dict(WORKLOADS[idx])
    if T is not None:
        spec["T"] = T
    if B is not None:
        spec["B"] = B
    if H is not None:
        spec["H"] = H
    seed = 1000 + idx
    if spec["varlen"]:
        lengths = doc_lengths(seed, spec["B"], spec["T"])
        cu = cu_from_lengths(lengths)
        total = spec["T"]
    else:
        total = spec["B"] * spec["T"]
        cu = np.arange(spec["B"] + 1, dtype=np.int64) * spec["T"]
    arrs = generate(seed, total, spec["H"], spec["dk"], spec["dv"], spec["dtype"], num_seqs=spec["B"],
                    with_s0=spec["s0"], with_grads=spec["bwd"], tensors=tensors)
    return spec, cu, arrs
