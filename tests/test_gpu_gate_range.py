"""GPU parity over the whole gate range, forward and backward, against the
fp64 oracle through the C ABI.

The decay alpha = exp(g) may be any value in (0, 1] per key channel (the gate
of "TorchTitan Ascend open source: Kimi K3.1 Pro adaptation and training
practice", section "Kimi K3.1 Pro model structure").  Every head mixes three
kinds of channels (kda_inputs.mix_gates): the usual draw, g = 0, and
fast-forgetting channels with g ~ U(-8, -2) per token, whose decay over one
64-token chunk (e^-128 .. e^-512) is far below what the chunk-start
factorisation exp(G_r) exp(-G_s) can hold in fp32.  Such chunks go through the
recurrence token by token (forward, reverse scan) and through the pair-exact
chunk-gradient kernel.  Bars as in the other parity tests.
"""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import dev, frob_rel, host, inf_rel, max_over_rms, need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu

LENS = [200, 64, 1, 130, 77]


def _say(msg):
    print(f"[gpu-gate-range] {msg}", flush=True)


def _err(a, r, dtype, state=False):
    if dtype == "f32":
        return inf_rel(a, r)
    return frob_rel(a, r) if state else max_over_rms(a, r)


def _bar(dtype, state=False):
    return 1e-4 if dtype == "f32" else (1e-2 if state else 2e-2)


def _case(seed, dtype, dk, dv, H, lens, mix=True):
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    x = kda_inputs.generate(seed, T, H, dk, dv, dtype, num_seqs=len(lens), with_s0=True, with_grads=True)
    if mix:
        x["g"] = kda_inputs.mix_gates(x["g"], seed, dtype)
    return cu, x


def _run_and_check(dtype, dk, dv, cu, x, tag):
    d = {k: dev(x[k], dtype) for k in ("q", "k", "v", "g", "b", "dO")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    dS = torch.from_numpy(x["dS"]).cuda()
    cu_t = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, sf, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, save_for_bwd=True)
    o2, sf2, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0)
    gr = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS)
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["dO"], cu_seqlens=cu, initial_state=x["s0"],
                     dS_final=x["dS"])
    got = {"o": host(o), "sf": host(sf), "o_infer": host(o2), "sf_infer": host(sf2), "dq": host(gr["dq"]),
           "dk": host(gr["dk"]), "dv": host(gr["dv"]), "dg": host(gr["dg"]), "db": host(gr["dbeta"]),
           "dS0": host(gr["dS0"])}
    want = {"o": o_ref, "sf": sf_ref, "o_infer": o_ref, "sf_infer": sf_ref, "dq": ref["dq"], "dk": ref["dk"],
            "dv": ref["dv"], "dg": ref["dg"], "db": ref["db"], "dS0": ref["dS0"]}
    states = ("sf", "sf_infer", "dS0")
    errs = {}
    for name, a in got.items():
        assert np.isfinite(a).all(), (tag, name)
        errs[name] = _err(a, want[name], dtype, state=name in states)
    _say(f"{tag}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, e in errs.items():
        assert e <= _bar(dtype, state=name in states), (tag, name, e)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 128), ("bf16", 128, 64),
                                         ("f32", 64, 64), ("f32", 128, 128), ("f32", 64, 128)])
def test_mixed_gate_range_forward_backward(dtype, dk, dv):
    need_gpu()
    _say(f"mixed gates {dtype} dk={dk} dv={dv} lens={LENS}")
    cu, x = _case(101, dtype, dk, dv, 3, LENS)
    _run_and_check(dtype, dk, dv, cu, x, f"{dtype} {dk}x{dv}")


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 128, 128), ("f32", 128, 64)])
def test_fp32_dk128_usual_gates(dtype, dk, dv):
    """fp32 inputs at dk = 128 (token-by-token forward and scan, pair-exact
    gradients) on the usual gate draw."""
    need_gpu()
    _say(f"usual gates {dtype} dk={dk} dv={dv} lens={LENS}")
    cu, x = _case(102, dtype, dk, dv, 2, LENS, mix=False)
    _run_and_check(dtype, dk, dv, cu, x, f"{dtype} {dk}x{dv} usual")


def test_mixed_gate_range_long_sequence_split():
    """A long sequence takes the segment split of the bf16 forward (segment maps
    from the zero state, composed per document, segments rerun); the map pass
    and the rerun meet fast-forgetting chunks too."""
    need_gpu()
    T, H, dk, dv = 16384, 2, 128, 128
    from gated_delta_rule_41_amd import _lib
    cfg = _lib.make_config(H, dk, dv, _lib.KDA_BF16, _lib.KDA_F32)
    assert _lib.kda_fwd_workspace_size(cfg, T, 1) > 0
    _say(f"split T={T} H={H}")
    x = kda_inputs.generate(103, T, H, dk, dv, "bf16", num_seqs=1, with_s0=True)
    x["g"] = kda_inputs.mix_gates(x["g"], 103, "bf16")
    d = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o, sf, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], None, s0)
    torch.cuda.synchronize()
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], initial_state=x["s0"])
    e1, e2 = max_over_rms(host(o), o_ref), frob_rel(host(sf), sf_ref)
    _say(f"split: o max/rms {e1:.2e} final state frob {e2:.2e}")
    assert np.isfinite(host(o)).all() and e1 <= 2e-2 and e2 <= 1e-2
