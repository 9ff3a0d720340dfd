"""ctypes binding of libkda (include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so.  PyTorch supplies device memory and the stream.  There is
no fallback: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kda.h")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_FLAG_SAVE_FOR_BWD = 1
KDA_FLAG_SEQUENTIAL = 2
KDA_FLAG_STAGED = 4
# kda_stage (include/kda.h), in order
STAGES = ("G", "Akk", "Aqk", "T", "W", "Ut", "U", "S_in", "QG", "Ktil", "GamC")


class KdaConfig(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("l2_eps", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libkda status {status}: {message}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p


def header_functions() -> list[str]:
    """Names of the functions declared in include/kda.h."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def load():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    # One HIP runtime per process.  PyTorch ships its own libamdhip64 and
    # libhsa-runtime64; loading torch first makes libkda.so bind to those (same
    # soname) instead of pulling in a second copy from the ROCm install, and two
    # runtimes in one process compete for the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    cfgp = ctypes.POINTER(KdaConfig)
    lib.kda_config_init.argtypes = [cfgp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.kda_config_init.restype = None
    lib.kda_stage_offset.argtypes = [cfgp, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    lib.kda_stage_offset.restype = ctypes.c_size_t
    for name in ("kda_saved_size", "kda_fwd_workspace_size", "kda_bwd_workspace_size"):
        fn = getattr(lib, name)
        fn.argtypes = [cfgp, ctypes.c_int64, ctypes.c_int32]
        fn.restype = ctypes.c_size_t
    lib.kda_fwd.argtypes = ([cfgp, ctypes.c_int64, ctypes.c_int32] + [_vp] * 10 + [ctypes.c_size_t, _vp]
                            + [ctypes.c_size_t, _vp])
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd_static.argtypes = [cfgp, ctypes.c_int64, ctypes.c_int32] + [_vp] * 10 + [ctypes.c_size_t, _vp]
    lib.kda_fwd_static.restype = ctypes.c_int
    for name in ("kda_bwd", "kda_bwd_scan", "kda_bwd_grads"):
        fn = getattr(lib, name)
        fn.argtypes = ([cfgp, ctypes.c_int64, ctypes.c_int32] + [_vp] * 8 + [ctypes.c_size_t] + [_vp] * 9
                       + [ctypes.c_size_t, _vp])
        fn.restype = ctypes.c_int
    lib.kda_decode.argtypes = [cfgp, ctypes.c_int32] + [_vp] * 9
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def make_config(H, dk, dv, in_dtype=KDA_BF16, out_dtype=KDA_F32, eps=1e-6, scale=1.0, flags=0):
    cfg = KdaConfig()
    load().kda_config_init(ctypes.byref(cfg), H, dk, dv)
    cfg.in_dtype, cfg.out_dtype = in_dtype, out_dtype
    cfg.l2_eps, cfg.scale, cfg.flags = eps, scale, flags
    return cfg


def check(status: int):
    if status != KDA_OK:
        lib = load()
        raise KdaError(status, f"{lib.kda_status_string(status).decode()}: {lib.kda_last_error().decode()}")


def kda_saved_size(cfg: KdaConfig, total_tokens: int, num_seqs: int) -> int:
    return int(load().kda_saved_size(ctypes.byref(cfg), total_tokens, num_seqs))


def kda_fwd_workspace_size(cfg: KdaConfig, total_tokens: int, num_seqs: int) -> int:
    return int(load().kda_fwd_workspace_size(ctypes.byref(cfg), total_tokens, num_seqs))


def kda_stage_offset(cfg: KdaConfig, total_tokens: int, num_seqs: int, stage: int) -> int:
    return int(load().kda_stage_offset(ctypes.byref(cfg), total_tokens, num_seqs, stage))


def kda_bwd_workspace_size(cfg: KdaConfig, total_tokens: int, num_seqs: int) -> int:
    return int(load().kda_bwd_workspace_size(ctypes.byref(cfg), total_tokens, num_seqs))


def kda_fwd_raw(cfg, total_tokens, num_seqs, q, k, v, g, beta, cu_seqlens, initial_state, o,
                final_state, saved, saved_bytes, workspace, workspace_bytes, stream) -> int:
    """Direct call of kda_fwd with integer device addresses (0 = NULL); returns the status."""
    return load().kda_fwd(ctypes.byref(cfg), total_tokens, num_seqs, q, k, v, g, beta, cu_seqlens,
                          initial_state, o, final_state, saved, saved_bytes, workspace, workspace_bytes, stream)


KDA_STATIC_WORKSPACE_BYTES = 128 << 20


def kda_fwd_static_raw(cfg, total_tokens, num_seqs, q, k, v, g, beta, cu_seqlens, initial_state, o,
                       final_state, saved, saved_bytes, stream) -> int:
    """Direct call of kda_fwd_static (the forward on the library's static
    workspace) with integer device addresses (0 = NULL); returns the status."""
    return load().kda_fwd_static(ctypes.byref(cfg), total_tokens, num_seqs, q, k, v, g, beta, cu_seqlens,
                                 initial_state, o, final_state, saved, saved_bytes, stream)


BWD_ENTRY = {"all": "kda_bwd", "scan": "kda_bwd_scan", "grads": "kda_bwd_grads"}


def kda_bwd_raw(cfg, total_tokens, num_seqs, q, k, v, g, beta, cu_seqlens, initial_state, saved, saved_bytes,
                dO, dS_final, dq, dk, dv, dg, dbeta, d_initial_state, workspace, workspace_bytes,
                stream, stage: str = "all") -> int:
    """Direct call of kda_bwd (stage "all"), kda_bwd_scan ("scan") or kda_bwd_grads
    ("grads") with integer device addresses (0 = NULL); returns the status."""
    fn = getattr(load(), BWD_ENTRY[stage])
    return fn(ctypes.byref(cfg), total_tokens, num_seqs, q, k, v, g, beta, cu_seqlens, initial_state, saved,
              saved_bytes, dO, dS_final, dq, dk, dv, dg, dbeta, d_initial_state, workspace, workspace_bytes, stream)


def kda_decode_raw(cfg, num_seqs, q, k, v, g, beta, state_in, state_out, o, stream) -> int:
    """Direct call of kda_decode with integer device addresses (0 = NULL); returns the status."""
    return load().kda_decode(ctypes.byref(cfg), num_seqs, q, k, v, g, beta, state_in, state_out, o, stream)
