"""libkda for PyTorch-ROCm: Kimi Delta Attention chunked forward/backward on MI355X.

The Python layer only marshals arguments: it checks tensor devices, dtypes and
shapes, allocates outputs with torch (device memory), and passes raw pointers
plus the current HIP stream to the C ABI of libkda.so.  Every step of the
computation (normalisation, gating, intra-chunk solve, inter-chunk state
passing, gradients) runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback.

Layouts follow include/kda.h: q, k, g ``[T, H, dk]``; v ``[T, H, dv]``;
beta ``[T, H]`` (the logit); states ``[N, H, dk, dv]`` fp32; cu_seqlens int32
``[N + 1]`` on the device.
"""
from __future__ import annotations

from typing import Optional

from . import _lib
from ._lib import (KDA_BF16, KDA_F32, KDA_FLAG_SAVE_FOR_BWD, KDA_FLAG_SEQUENTIAL, KdaConfig, KdaError, kda_bwd_workspace_size,
                   kda_fwd_workspace_size, kda_saved_size, make_config)

__all__ = ["kda", "kda_fwd", "kda_fwd_staged", "kda_bwd", "kda_decode", "kda_saved_size", "kda_fwd_workspace_size", "kda_bwd_workspace_size",
           "make_config", "KdaConfig", "KdaError", "KDA_F32", "KDA_BF16", "KDA_FLAG_SAVE_FOR_BWD",
           "KDA_FLAG_SEQUENTIAL"]


def _torch():
    import torch
    return torch


def _dt_code(dtype):
    torch = _torch()
    if dtype == torch.bfloat16:
        return KDA_BF16
    if dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {dtype}")


def _ptr(t):
    return 0 if t is None else int(t.data_ptr())


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _common(q, k, v, g, beta, cu_seqlens, num_seqs):
    torch = _torch()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [T,H,dk] and v [T,H,dv]")
    T, H, dk = q.shape
    dv = v.shape[2]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("libkda runs on the GPU only: tensors must be on a cuda (HIP) device")
    dt = q.dtype
    for name, t, shp in (("k", k, (T, H, dk)), ("v", v, (T, H, dv)), ("g", g, (T, H, dk)), ("beta", beta, (T, H))):
        _check(t, name, shp, dt, dev)
    _check(q, "q", (T, H, dk), dt, dev)
    if cu_seqlens is not None:
        if (cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev
                or not cu_seqlens.is_contiguous()):
            raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor on the same device")
        N = cu_seqlens.numel() - 1
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    return T, H, dk, dv, N, dev, dt


def kda_fwd(q, k, v, g, beta, cu_seqlens=None, initial_state=None, *, num_seqs: Optional[int] = None,
            out_dtype=None, save_for_bwd: bool = False, eps: float = 1e-6, scale: float = 1.0,
            output_final_state: bool = True, sequential: bool = False):
    """KDA forward.  Returns ``(o, final_state, saved)``; ``saved`` is None
    unless ``save_for_bwd``.  ``num_seqs`` splits an un-packed stream into equal
    sequences when ``cu_seqlens`` is None.  ``sequential`` keeps the library
    from splitting long sequences into segments (KDA_FLAG_SEQUENTIAL)."""
    torch = _torch()
    T, H, dk, dv, N, dev, dt = _common(q, k, v, g, beta, cu_seqlens, num_seqs)
    out_dtype = out_dtype or torch.float32
    _check(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    cfg = make_config(H, dk, dv, _dt_code(dt), _dt_code(out_dtype), eps, scale,
                      (KDA_FLAG_SAVE_FOR_BWD if save_for_bwd else 0) | (KDA_FLAG_SEQUENTIAL if sequential else 0))
    o = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    saved = None
    if save_for_bwd:
        saved = torch.empty(max(kda_saved_size(cfg, T, N), 1), dtype=torch.uint8, device=dev)
    wsb = kda_fwd_workspace_size(cfg, T, N)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.check(_lib.kda_fwd_raw(cfg, T, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                    _ptr(initial_state), _ptr(o), _ptr(sf), _ptr(saved),
                                    0 if saved is None else saved.numel(), _ptr(ws), wsb, stream))
    return o, sf, saved


def kda_fwd_staged(q, k, v, g, beta, cu_seqlens=None, initial_state=None, *, num_seqs: Optional[int] = None,
                   out_dtype=None, eps: float = 1e-6, scale: float = 1.0, chunk: int = 64):
    """The staged forward (kda_fwd with KDA_FLAG_STAGED): the correctness path.
    Returns ``(o, final_state, stages)``; ``stages`` maps each name of
    ``_lib.STAGES`` to an fp32 view of the workspace shaped
    ``[slots, H, ...]`` (see kda_stage in include/kda.h): chunk j of
    document n is slot ``cu[n] // chunk + n + j``.  ``chunk`` may be 16, 32
    or 64."""
    torch = _torch()
    T, H, dk, dv, N, dev, dt = _common(q, k, v, g, beta, cu_seqlens, num_seqs)
    out_dtype = out_dtype or torch.float32
    _check(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    cfg = make_config(H, dk, dv, _dt_code(dt), _dt_code(out_dtype), eps, scale, _lib.KDA_FLAG_STAGED)
    cfg.chunk = chunk
    o = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    wsb = kda_fwd_workspace_size(cfg, T, N)
    ws = torch.zeros(max(wsb, 4), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.check(_lib.kda_fwd_raw(cfg, T, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                    _ptr(initial_state), _ptr(o), _ptr(sf), 0, 0, _ptr(ws), wsb, stream))
    slots = T // chunk + N
    C = chunk
    tail = {"G": (C, dk), "Akk": (C, C), "Aqk": (C, C), "T": (C, C), "W": (C, dk), "Ut": (C, dv),
            "U": (C, dv), "S_in": (dk, dv), "QG": (C, dk), "Ktil": (C, dk), "GamC": (dk,)}
    stages = {}
    for i, name in enumerate(_lib.STAGES):
        off = _lib.kda_stage_offset(cfg, T, N, i)
        count = slots * H
        for d in tail[name]:
            count *= d
        stages[name] = ws[off:off + 4 * count].view(torch.float32).view(slots, H, *tail[name])
    return o, sf, stages


def kda_bwd(q, k, v, g, beta, saved, dO, cu_seqlens=None, initial_state=None, dS_final=None, *,
            num_seqs: Optional[int] = None, out_dtype=None, eps: float = 1e-6, scale: float = 1.0,
            output_d_initial_state: bool = True, stage: str = "all", out=None):
    """KDA backward for the loss <dO, o> + <dS_final, final_state>.  Returns a
    dict with dq, dk, dv, dg, dbeta, dS0 (None unless requested) and the
    workspace.

    stage "all" calls kda_bwd; "scan" and "grads" call its two stages
    (kda_bwd_scan, kda_bwd_grads).  Pass the dict returned by the "scan" call as
    `out` to the "grads" call: it carries the outputs and the workspace the
    second stage reads."""
    torch = _torch()
    T, H, dk, dv, N, dev, dt = _common(q, k, v, g, beta, cu_seqlens, num_seqs)
    out_dtype = out_dtype or torch.float32
    _check(dO, "dO", (T, H, dv), dt, dev)
    _check(initial_state, "initial_state", (N, H, dk, dv), torch.float32, dev)
    _check(dS_final, "dS_final", (N, H, dk, dv), torch.float32, dev)
    cfg = make_config(H, dk, dv, _dt_code(dt), _dt_code(out_dtype), eps, scale, 0)
    need = kda_saved_size(cfg, T, N)
    if saved is None or saved.dtype != torch.uint8 or saved.numel() < need or saved.device != dev:
        raise ValueError(f"saved must be a uint8 device tensor of at least {need} bytes from kda_fwd(save_for_bwd=True)")
    if stage not in _lib.BWD_ENTRY:
        raise ValueError(f"stage must be one of {sorted(_lib.BWD_ENTRY)}")
    wsb = kda_bwd_workspace_size(cfg, T, N)
    if out is None:
        out = {
            "dq": torch.empty((T, H, dk), dtype=out_dtype, device=dev),
            "dk": torch.empty((T, H, dk), dtype=out_dtype, device=dev),
            "dv": torch.empty((T, H, dv), dtype=out_dtype, device=dev),
            "dg": torch.empty((T, H, dk), dtype=out_dtype, device=dev),
            "dbeta": torch.empty((T, H), dtype=out_dtype, device=dev),
            "dS0": torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_d_initial_state else None,
            "workspace": torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev),
        }
    ws = out["workspace"]
    if ws.numel() < wsb:
        raise ValueError(f"workspace must hold at least {wsb} bytes")
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.check(_lib.kda_bwd_raw(cfg, T, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                                    _ptr(initial_state), _ptr(saved), saved.numel(), _ptr(dO), _ptr(dS_final), _ptr(out["dq"]),
                                    _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                                    _ptr(out["dS0"]), _ptr(ws), wsb, stream, stage))
    return out


def kda_decode(q, k, v, g, beta, state=None, *, out_state=None, out_dtype=None, eps: float = 1e-6,
               scale: float = 1.0):
    """One decode step: one token per sequence on a resident fp32 state.

    q, k, g ``[N, H, dk]``, v ``[N, H, dv]``, beta ``[N, H]`` (the logit);
    ``state`` ``[N, H, dk, dv]`` fp32 or None (zero state).  ``out_state`` is
    where the state after the token goes: a new tensor if None, or a given
    tensor, which may be ``state`` itself for an in-place update.  Returns
    ``(o, out_state)``."""
    torch = _torch()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [N,H,dk] and v [N,H,dv]")
    N, H, dk = q.shape
    dv = v.shape[2]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("libkda runs on the GPU only: tensors must be on a cuda (HIP) device")
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("v", v, (N, H, dv)), ("g", g, (N, H, dk)),
                         ("beta", beta, (N, H))):
        _check(t, name, shp, dt, dev)
    _check(state, "state", (N, H, dk, dv), torch.float32, dev)
    if out_state is None:
        out_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _check(out_state, "out_state", (N, H, dk, dv), torch.float32, dev)
    out_dtype = out_dtype or torch.float32
    cfg = make_config(H, dk, dv, _dt_code(dt), _dt_code(out_dtype), eps, scale, 0)
    o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        _lib.check(_lib.kda_decode_raw(cfg, N, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                       _ptr(out_state), _ptr(o), stream))
    return o, out_state


def _autograd_function():
    torch = _torch()

    class KDAFunction(torch.autograd.Function):
        """Autograd glue: forward saves the library's saved buffer, backward calls
        kda_bwd.  Gradients flow to q, k, v, g, beta and initial_state."""

        @staticmethod
        def forward(ctx, q, k, v, g, beta, cu_seqlens, initial_state, num_seqs, eps, scale):
            o, sf, saved = kda_fwd(q, k, v, g, beta, cu_seqlens, initial_state, num_seqs=num_seqs, eps=eps,
                                   scale=scale, save_for_bwd=True)
            ctx.save_for_backward(q, k, v, g, beta, saved)
            ctx.cu_seqlens, ctx.initial_state = cu_seqlens, initial_state
            ctx.num_seqs, ctx.eps, ctx.scale = num_seqs, eps, scale
            ctx.out_dtype = o.dtype
            return o, sf

        @staticmethod
        def backward(ctx, d_o, d_sf):
            q, k, v, g, beta, saved = ctx.saved_tensors
            s0 = ctx.initial_state
            d_o = (d_o if d_o is not None else torch.zeros_like(v)).to(q.dtype).contiguous()
            d_sf = d_sf.contiguous() if d_sf is not None else None
            # gradients come out of the kernels in the inputs' dtype (rounded once, as a cast would)
            gr = kda_bwd(q, k, v, g, beta, saved, d_o, ctx.cu_seqlens, s0, d_sf, num_seqs=ctx.num_seqs,
                         out_dtype=q.dtype, eps=ctx.eps, scale=ctx.scale, output_d_initial_state=s0 is not None)
            return (gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["dbeta"], None, gr["dS0"], None, None, None)

    return KDAFunction


_KDA_FN = None


def kda(q, k, v, g, beta, cu_seqlens=None, initial_state=None, *, num_seqs: Optional[int] = None,
        eps: float = 1e-6, scale: float = 1.0):
    """KDA as a differentiable torch op: returns ``(o, final_state)`` (fp32) and,
    under autograd, back-propagates through kda_bwd.  The upstream gradient of o
    is cast to the input dtype (bf16 inputs take a bf16 dO, as kda_bwd does)."""
    global _KDA_FN
    if _KDA_FN is None:
        _KDA_FN = _autograd_function()
    return _KDA_FN.apply(q, k, v, g, beta, cu_seqlens, initial_state, num_seqs, eps, scale)
