"""kda_fwd_static, the forward on the library's static device workspace (for
callers that cannot allocate), against kda_fwd with a caller-allocated
workspace, through the C ABI.

The cases take the long-sequence split (kda_fwd_workspace_size > 0), so the
static workspace is used.  Both entry points run the same kernels on the same
plan, so their outputs must agree bit for bit; the first case is also checked
against the fp64 oracle at the bf16 bars of tests/gpu_util.py.  Two calls in a
row, the second smaller, show that a call reads nothing an earlier call left
in the shared array.
"""
import ctypes

import numpy as np
import pytest

import kda_inputs
import oracle

from gated_delta_rule_41_amd import _lib


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)


def test_static_workspace_rejects_oversized_plans():
    # the largest split plans (many documents of short-value heads) need more than the static array
    cfg = _lib.make_config(1, 128, 64, _lib.KDA_BF16, _lib.KDA_F32)
    N = 127
    T = ((1 << 23) - N - 1) * 64      # the most chunk slots one launch covers at H = 1
    T -= T % N
    need = _lib.kda_fwd_workspace_size(cfg, T, N)
    assert need > _lib.KDA_STATIC_WORKSPACE_BYTES
    fake = 1 << 20
    st = _lib.kda_fwd_static_raw(cfg, T, N, fake, fake, fake, fake, fake, 0, 0, fake, 0, 0, 0, 0)
    assert st == _lib.KDA_ERR_WORKSPACE
    assert "static workspace" in _lib.load().kda_last_error().decode()
    # the long-context workload (one 2^20-token sequence, 16 heads of 128 x 128) fits
    cfg16 = _lib.make_config(16, 128, 128, _lib.KDA_BF16, _lib.KDA_F32)
    assert 0 < _lib.kda_fwd_workspace_size(cfg16, 1 << 20, 1) <= _lib.KDA_STATIC_WORKSPACE_BYTES


@pytest.mark.gpu
def test_static_workspace_forward_matches_kda_fwd():
    from gpu_util import BF16_FROB, BF16_MAX_RMS, dev, frob_rel, host, max_over_rms, need_gpu, torch
    need_gpu()
    H, dk, dv = 2, 128, 128
    cfg = _lib.make_config(H, dk, dv, _lib.KDA_BF16, _lib.KDA_F32)
    for call, (T, seed) in enumerate([(16384, 61), (8192, 62)]):
        wsb = _lib.kda_fwd_workspace_size(cfg, T, 1)
        _say(f"call {call}: T={T} H={H} dk={dk} dv={dv} workspace {wsb} bytes")
        assert 0 < wsb <= _lib.KDA_STATIC_WORKSPACE_BYTES
        x = kda_inputs.generate(seed, T, H, dk, dv, "bf16", num_seqs=1, with_s0=True)
        d = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b")}
        s0 = torch.from_numpy(x["s0"]).cuda()
        outs = []
        for static in (False, True):
            o = torch.full((T, H, dv), float("nan"), device="cuda")
            sf = torch.full((1, H, dk, dv), float("nan"), device="cuda")
            ptrs = [d[k].data_ptr() for k in ("q", "k", "v", "g", "b")]
            stream = torch.cuda.current_stream().cuda_stream
            if static:
                st = _lib.kda_fwd_static_raw(cfg, T, 1, *ptrs, 0, s0.data_ptr(), o.data_ptr(), sf.data_ptr(),
                                             0, 0, stream)
            else:
                ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
                st = _lib.kda_fwd_raw(cfg, T, 1, *ptrs, 0, s0.data_ptr(), o.data_ptr(), sf.data_ptr(), 0, 0,
                                      ws.data_ptr(), wsb, stream)
            assert st == _lib.KDA_OK, _lib.load().kda_last_error().decode()
            torch.cuda.synchronize()
            outs.append((o, sf))
        (o1, sf1), (o2, sf2) = outs
        assert torch.equal(o1, o2) and torch.equal(sf1, sf2), f"call {call}"
        if call == 0:
            o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], initial_state=x["s0"])
            e1, e2 = max_over_rms(host(o2), o_ref), frob_rel(host(sf2), sf_ref)
            _say(f"call {call}: o max/rms {e1:.2e} final state frob {e2:.2e}")
            assert e1 <= BF16_MAX_RMS and e2 <= BF16_FROB
