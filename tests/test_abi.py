"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, sizes buffers as documented, and rejects bad arguments
on the host with the documented status BEFORE any HIP call (every case below
fails validation, so no pointer is ever dereferenced and nothing is launched)."""
import ctypes

import pytest

from gated_delta_rule_41_amd import _lib
from gated_delta_rule_41_amd._lib import (KDA_BF16, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE,
                                          KDA_F32, KDA_FLAG_SAVE_FOR_BWD, KDA_OK)

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def test_library_exports_every_header_function():
    lib = _lib.load()
    names = _lib.header_functions()
    assert {"kda_fwd", "kda_bwd", "kda_saved_size", "kda_config_init"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.kda_version() >= 100


def test_config_init_defaults():
    cfg = _lib.make_config(4, 128, 64)
    assert (cfg.H, cfg.dk, cfg.dv, cfg.chunk) == (4, 128, 64, 64)
    assert abs(cfg.l2_eps - 1e-6) < 1e-12 and cfg.scale == 1.0


def test_status_strings():
    lib = _lib.load()
    for s in range(5):
        assert lib.kda_status_string(s)
    assert b"unknown" in lib.kda_status_string(99)


def test_sizes():
    cfg = _lib.make_config(32, 128, 128, KDA_BF16, KDA_F32)
    T, N = 4 * 8192, 4
    slots = T // 64 + N
    states = slots * 32 * 128 * 128 * 2   # bf16 inputs: fp16 states, scaled per 16 value columns
    nrm = T * 32 * 4
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    u = slots * 32 * 64 * 128 * 2   # per-chunk U (saved) and dU (workspace) in fp16, bf16 inputs only
    sc = slots * 32 * (128 // 16) * 4   # one fp32 scale per chunk, head and 16-column group
    assert _lib.kda_saved_size(cfg, T, N) == al(states) + 2 * al(nrm) + al(u) + al(sc)
    flags = slots * 32 * 4          # one int per chunk and head: decay past the factorised range
    assert _lib.kda_bwd_workspace_size(cfg, T, N) == al(states) + al(u) + al(sc) + al(flags)
    assert _lib.kda_fwd_workspace_size(cfg, T, N) == 0
    cfg32 = _lib.make_config(2, 64, 64, KDA_F32, KDA_F32)
    assert _lib.kda_saved_size(cfg32, 256, 1) == al(5 * 2 * 64 * 64 * 4) + 2 * al(256 * 2 * 4)
    # fp32 inputs at dk = 128: states and norms only (no per-chunk U)
    cfg128 = _lib.make_config(2, 128, 128, KDA_F32, KDA_F32)
    assert _lib.kda_saved_size(cfg128, 256, 1) == al(5 * 2 * 128 * 128 * 4) + 2 * al(256 * 2 * 4)
    assert _lib.kda_bwd_workspace_size(cfg128, 256, 1) == al(5 * 2 * 128 * 128 * 4) + al(5 * 2 * 4)
    bad = _lib.make_config(2, 96, 64)
    assert _lib.kda_saved_size(bad, 256, 1) == 0


def _fwd(cfg, T=128, N=1, q=FAKE, o=FAKE, cu=0, saved=0, saved_bytes=0, ws=0, wsb=0):
    return _lib.kda_fwd_raw(cfg, T, N, q, FAKE, FAKE, FAKE, FAKE, cu, 0, o, 0, saved, saved_bytes, ws, wsb, 0)


def _err():
    return _lib.load().kda_last_error().decode()


@pytest.mark.parametrize("dk,dv,chunk,ind,expect", [
    (96, 128, 64, KDA_BF16, KDA_ERR_UNSUPPORTED),
    (128, 32, 64, KDA_BF16, KDA_ERR_UNSUPPORTED),
    (128, 128, 32, KDA_BF16, KDA_ERR_UNSUPPORTED),
    (128, 128, 64, 7, KDA_ERR_INVALID_ARG),
])
def test_fwd_rejects_unsupported_configs(dk, dv, chunk, ind, expect):
    cfg = _lib.make_config(2, 64, 64)
    cfg.dk, cfg.dv, cfg.chunk, cfg.in_dtype = dk, dv, chunk, ind
    assert _fwd(cfg) == expect
    assert _err()


def test_fwd_rejects_bad_arguments():
    cfg = _lib.make_config(2, 64, 64, KDA_BF16)
    assert _lib.load().kda_fwd(None, 1, 1, *([None] * 10), 0, None, 0, None) == KDA_ERR_INVALID_ARG
    assert _fwd(cfg, T=-1) == KDA_ERR_INVALID_ARG
    assert _fwd(cfg, T=1 << 31) == KDA_ERR_INVALID_ARG
    assert _fwd(cfg, N=0) == KDA_ERR_INVALID_ARG
    assert _fwd(cfg, T=100, N=3) == KDA_ERR_INVALID_ARG      # no cu_seqlens and T % N != 0
    assert _fwd(cfg, q=0) == KDA_ERR_INVALID_ARG and "q" in _err()
    assert _fwd(cfg, o=0) == KDA_ERR_INVALID_ARG and "o" in _err()
    assert _fwd(cfg, q=FAKE + 2) == KDA_ERR_INVALID_ARG and "aligned" in _err()
    assert _fwd(cfg, cu=FAKE + 4) == KDA_ERR_INVALID_ARG
    cfg.flags = KDA_FLAG_SAVE_FOR_BWD
    assert _fwd(cfg) == KDA_ERR_INVALID_ARG and "saved" in _err()
    need = _lib.kda_saved_size(cfg, 128, 1)
    assert need > 0
    assert _fwd(cfg, saved=FAKE, saved_bytes=need - 1) == KDA_ERR_WORKSPACE and "saved" in _err()
    cfg.flags = 1 << 5
    assert _fwd(cfg) == KDA_ERR_INVALID_ARG
    cfg.flags = 0
    cfg.l2_eps = float("nan")
    assert _fwd(cfg) == KDA_ERR_INVALID_ARG
    cfg.l2_eps = 1e-6
    cfg.scale = float("inf")
    assert _fwd(cfg) == KDA_ERR_INVALID_ARG


def test_bwd_rejects_bad_arguments():
    cfg = _lib.make_config(2, 64, 64, KDA_BF16)
    T, N = 128, 1
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=0, s0=0, saved=FAKE, dO=FAKE, dSf=0, dq=FAKE,
                dk=FAKE, dv=FAKE, dg=FAKE, db=FAKE, dS0=0, ws=FAKE)
    need = _lib.kda_bwd_workspace_size(cfg, T, N)
    assert need > 0

    saved_need = _lib.kda_saved_size(cfg, T, N)
    assert saved_need > 0

    def call(wsb=need, saved_bytes=saved_need, **kw):
        a = dict(args)
        a.update(kw)
        return _lib.kda_bwd_raw(cfg, T, N, a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["s0"], a["saved"],
                                saved_bytes, a["dO"], a["dSf"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dS0"], a["ws"], wsb, 0)

    assert call(wsb=need - 1) == KDA_ERR_WORKSPACE
    assert call(saved_bytes=saved_need - 1) == KDA_ERR_WORKSPACE and "saved" in _err()
    for stage in ("scan", "grads"):
        assert _lib.kda_bwd_raw(cfg, T, N, *([FAKE] * 5), 0, 0, FAKE, saved_need - 256, FAKE, 0, *([FAKE] * 5), 0,
                                FAKE, need, 0, stage=stage) == KDA_ERR_WORKSPACE
    assert call(saved=0) == KDA_ERR_INVALID_ARG and "saved" in _err()
    assert call(dO=0) == KDA_ERR_INVALID_ARG and "dO" in _err()
    assert call(dg=FAKE + 8) == KDA_ERR_INVALID_ARG
    assert call(ws=0) == KDA_ERR_INVALID_ARG
    cfg.dk = 80
    assert call() == KDA_ERR_UNSUPPORTED


def test_python_layer_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import gated_delta_rule_41_amd as kda
    x = torch.zeros(4, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        kda.kda_fwd(x, x, x, x, torch.zeros(4, 1))
    assert KDA_OK == 0
    assert isinstance(_lib.KdaConfig(), ctypes.Structure)


def _decode(cfg, N=2, q=FAKE, s_in=0, s_out=FAKE, o=FAKE):
    return _lib.kda_decode_raw(cfg, N, q, FAKE, FAKE, FAKE, FAKE, s_in, s_out, o, 0)


def test_decode_rejects_bad_arguments():
    lib = _lib.load()
    assert lib.kda_decode(None, 1, *([None] * 9)) == KDA_ERR_INVALID_ARG
    cfg = _lib.make_config(4, 128, 128, KDA_BF16)
    assert _decode(cfg, N=-1) == KDA_ERR_INVALID_ARG
    assert _decode(cfg, q=0) == KDA_ERR_INVALID_ARG and "q" in _err()
    assert _decode(cfg, o=0) == KDA_ERR_INVALID_ARG and "o" in _err()
    assert _decode(cfg, s_out=0) == KDA_ERR_INVALID_ARG and "state_out" in _err()
    assert _decode(cfg, s_out=FAKE + 4) == KDA_ERR_INVALID_ARG and "aligned" in _err()
    assert _decode(cfg, s_in=FAKE + 8) == KDA_ERR_INVALID_ARG and "state_in" in _err()
    # overlapping but distinct state buffers are refused; the same buffer (in place) is not
    assert _decode(cfg, s_in=FAKE, s_out=FAKE + 4096) == KDA_ERR_INVALID_ARG and "overlap" in _err()
    cfg.dk = 96
    assert _decode(cfg) == KDA_ERR_UNSUPPORTED
    cfg.dk, cfg.in_dtype = 128, 9
    assert _decode(cfg) == KDA_ERR_INVALID_ARG
    # nothing to do: returns before any HIP call
    cfg.in_dtype = KDA_F32
    assert _decode(cfg, N=0, q=0, s_out=0, o=0) == KDA_OK


def test_fwd_workspace_for_long_sequences():
    """The forward needs a workspace only when it splits long sequences: bf16
    inputs, few (sequence, head) chains, long documents, no state save and no
    KDA_FLAG_SEQUENTIAL."""
    long_cfg = _lib.make_config(16, 128, 128, KDA_BF16, KDA_F32)
    ws = _lib.kda_fwd_workspace_size(long_cfg, 1 << 20, 1)
    # at least the maps [M | B] (dk x (dk + dv)) and entering states of two segments per head
    assert ws >= 2 * 16 * 128 * (256 + 128) * 4
    assert _lib.kda_fwd_workspace_size(long_cfg, 4 * 8192, 4) == 0          # 256 chains fill the GPU
    assert _lib.kda_fwd_workspace_size(long_cfg, 4096, 1) == 0              # too short to split
    seq = _lib.make_config(16, 128, 128, KDA_BF16, KDA_F32, flags=_lib.KDA_FLAG_SEQUENTIAL)
    assert _lib.kda_fwd_workspace_size(seq, 1 << 20, 1) == 0
    save = _lib.make_config(16, 128, 128, KDA_BF16, KDA_F32, flags=KDA_FLAG_SAVE_FOR_BWD)
    assert _lib.kda_fwd_workspace_size(save, 1 << 20, 1) == 0
    f32 = _lib.make_config(2, 64, 64, KDA_F32, KDA_F32)
    assert _lib.kda_fwd_workspace_size(f32, 1 << 20, 1) == 0
    # too small or missing workspace is refused before any launch
    assert _fwd(long_cfg, T=1 << 20, ws=FAKE, wsb=ws - 1) == KDA_ERR_WORKSPACE
    assert _fwd(long_cfg, T=1 << 20, ws=0, wsb=ws) == KDA_ERR_INVALID_ARG and "workspace" in _err()
    cfg = _lib.make_config(2, 64, 64, KDA_BF16)
    cfg.flags = 8
    assert _fwd(cfg) == KDA_ERR_INVALID_ARG


def test_staged_forward_workspace_and_checks():
    """KDA_FLAG_STAGED: the workspace holds the eleven fp32 stages of kda_stage,
    each [slots, H, ...], 256-byte aligned, in enum order; the flag excludes the
    state save; a short or missing workspace is refused before any launch."""
    T, N, H, dk, dv = 247, 3, 2, 128, 64
    cfg = _lib.make_config(H, dk, dv, KDA_BF16, KDA_F32, flags=_lib.KDA_FLAG_STAGED)
    slots = T // 64 + N
    tails = {"G": 64 * dk, "Akk": 64 * 64, "Aqk": 64 * 64, "T": 64 * 64, "W": 64 * dk, "Ut": 64 * dv,
             "U": 64 * dv, "S_in": dk * dv, "QG": 64 * dk, "Ktil": 64 * dk, "GamC": dk}
    off = [_lib.kda_stage_offset(cfg, T, N, i) for i in range(len(_lib.STAGES) + 1)]
    assert off[0] == 0
    for i, name in enumerate(_lib.STAGES):
        size = slots * H * tails[name] * 4
        assert off[i] % 256 == 0 and off[i + 1] - off[i] == (size + 255) // 256 * 256, name
    need = _lib.kda_fwd_workspace_size(cfg, T, N)
    assert need == off[-1] > 0
    assert _lib.kda_stage_offset(cfg, T, N, len(_lib.STAGES) + 1) == 0
    assert _lib.kda_stage_offset(cfg, T, N, -1) == 0
    assert _fwd(cfg, T=T, N=N, cu=FAKE, ws=FAKE, wsb=need - 1) == KDA_ERR_WORKSPACE
    assert _fwd(cfg, T=T, N=N, cu=FAKE, ws=0, wsb=need) == KDA_ERR_INVALID_ARG and "workspace" in _err()
    both = _lib.make_config(H, dk, dv, KDA_BF16, KDA_F32, flags=_lib.KDA_FLAG_STAGED | KDA_FLAG_SAVE_FOR_BWD)
    need_s = _lib.kda_saved_size(both, T, N)
    assert _fwd(both, T=T, N=N, cu=FAKE, saved=FAKE, saved_bytes=need_s, ws=FAKE, wsb=need) == KDA_ERR_UNSUPPORTED
    assert "STAGED" in _err()
    # chunks of 16 and 32: the staged forward only
    c16 = _lib.make_config(H, dk, dv, KDA_BF16, KDA_F32, flags=_lib.KDA_FLAG_STAGED)
    c16.chunk = 16
    n16 = _lib.kda_fwd_workspace_size(c16, T, N)
    assert n16 == _lib.kda_stage_offset(c16, T, N, len(_lib.STAGES)) > 0
    assert _lib.kda_stage_offset(c16, T, N, 1) == (((T // 16 + N) * H * 16 * dk * 4) + 255) // 256 * 256
    plain = _lib.make_config(H, dk, dv, KDA_BF16, KDA_F32)
    plain.chunk = 16
    assert _fwd(plain, T=T, N=N, cu=FAKE) == KDA_ERR_UNSUPPORTED and "chunk" in _err()
    assert _lib.kda_bwd_raw(c16, T, N, *([FAKE] * 5), FAKE, 0, FAKE, 1 << 30, FAKE, 0, *([FAKE] * 5), 0,
                            FAKE, 1 << 30, 0, "all") == KDA_ERR_UNSUPPORTED


def test_head_count_bound():
    """64 * H * max(dk, dv) must stay below 2^31 (32-bit row offsets in a chunk)."""
    cfg = _lib.make_config(262144, 128, 128, KDA_BF16)       # 64 * 262144 * 128 = 2^31
    assert _fwd(cfg, T=64) == KDA_ERR_UNSUPPORTED and "H too large" in _err()


def test_launch_size_bound():
    """Every launch stays within 2^32 - 1 work-items along x; larger problems are refused on
    the host (checked before any HIP call, so no device is needed)."""
    many_docs = _lib.make_config(1, 64, 64, KDA_BF16)     # 2^23 one-token documents: 2^23 x 512 = 2^32
    assert _fwd(many_docs, T=1 << 23, N=1 << 23) == KDA_ERR_UNSUPPORTED and "one launch" in _err()
    many_chunks = _lib.make_config(1024, 64, 64, KDA_BF16)   # 8193 chunk slots x 1024 heads x 512 > 2^32 - 1
    assert _fwd(many_chunks, T=1 << 19, N=1) == KDA_ERR_UNSUPPORTED and "one launch" in _err()
    dec = _lib.make_config(1, 64, 64, KDA_BF16)            # 2^24 decode workgroups x 256 = 2^32
    assert _decode(dec, N=1 << 24) == KDA_ERR_UNSUPPORTED and "one launch" in _err()
