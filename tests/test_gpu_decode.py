"""GPU parity of the decode step (kda_decode) against the fp64 oracle, through the C ABI.

The oracle's token recurrence is the definition: one decode step of sequence n
is the oracle run on a one-token document n starting from the same state, and a
run of steps after a prefill is the oracle run on the whole sequence.
Tolerances are the ones in tests/gpu_util.py.
"""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import (BF16_FROB, BF16_MAX_RMS, F32_TOL, dev, frob_rel, host, inf_rel, max_over_rms, need_gpu,
                      torch)

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-decode] {msg}", flush=True)


def _step_inputs(seed, N, H, dk, dv, dtype, with_s0=True):
    # one token per sequence: a packed stream of N one-token documents
    return kda_inputs.generate(seed, N, H, dk, dv, dtype, num_seqs=N, with_s0=with_s0)


def _to_dev(x, dtype):
    return {name: dev(x[name], dtype) for name in ("q", "k", "v", "g", "b")}


def _assert_close(o, s, o_ref, s_ref, dtype, tag):
    o, s = host(o), host(s)
    assert np.isfinite(o).all() and np.isfinite(s).all(), tag
    if dtype == "f32":
        e1, e2 = inf_rel(o, o_ref), inf_rel(s, s_ref)
        _say(f"{tag}: o {e1:.2e} state {e2:.2e} (max rel)")
        assert e1 <= F32_TOL and e2 <= F32_TOL, tag
    else:
        e1, e2 = max_over_rms(o, o_ref), frob_rel(s, s_ref)
        _say(f"{tag}: o max/rms {e1:.2e} state frob {e2:.2e}")
        assert e1 <= BF16_MAX_RMS and e2 <= BF16_FROB, tag


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("f32", 128, 128), ("bf16", 128, 128),
                                         ("bf16", 64, 128), ("bf16", 128, 64)])
def test_decode_step_matches_oracle(dtype, dk, dv):
    need_gpu()
    N, H = 37, 6
    _say(f"one step {dtype} N={N} H={H} dk={dk} dv={dv}")
    x = _step_inputs(71, N, H, dk, dv, dtype)
    d = _to_dev(x, dtype)
    s0 = torch.from_numpy(x["s0"]).cuda()
    o, s1 = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], s0)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=np.arange(N + 1),
                              initial_state=x["s0"])
    _assert_close(o, s1, o_ref, s_ref, dtype, f"step {dtype} {dk}x{dv}")


def test_decode_zero_state_and_bf16_output():
    need_gpu()
    N, H, dk, dv = 16, 4, 128, 128
    _say("zero state, bf16 output")
    x = _step_inputs(72, N, H, dk, dv, "bf16", with_s0=False)
    d = _to_dev(x, "bf16")
    o, s1 = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], None, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    o_ref, s_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=np.arange(N + 1))
    # storing o in bf16 adds up to 2^-8 |o| (round to nearest, 8-bit significand); the compute
    # error on top of that storage rounding is held to the bf16 bar
    excess = np.abs(host(o) - o_ref) - 2.0 ** -8 * np.abs(o_ref)
    err = excess.max() / np.sqrt(np.mean(o_ref ** 2))
    e2 = frob_rel(host(s1), s_ref)
    _say(f"zero state: o excess over bf16 rounding {err:.2e}, state frob {e2:.2e}")
    assert err <= BF16_MAX_RMS and e2 <= BF16_FROB


def test_decode_in_place_and_deterministic():
    """An in-place update equals an out-of-place one bitwise; repeated calls are bitwise equal."""
    need_gpu()
    N, H, dk, dv = 24, 8, 128, 128
    _say("in place / determinism")
    x = _step_inputs(73, N, H, dk, dv, "bf16")
    d = _to_dev(x, "bf16")
    s0 = torch.from_numpy(x["s0"]).cuda()
    o1, s1 = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], s0)
    o2, s2 = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], s0)
    sp = s0.clone()
    o3, s3 = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], sp, out_state=sp)
    torch.cuda.synchronize()
    assert s3.data_ptr() == sp.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)
    assert torch.equal(s0, torch.from_numpy(x["s0"]).cuda())   # out-of-place leaves the input state alone


def test_prefill_then_decode_matches_oracle():
    """kda_fwd over a prefix, then one decode step per further token with the
    state updated in place, equals the oracle over the whole sequences."""
    need_gpu()
    lens = [200, 131, 64, 1]
    steps = 40
    H, dk, dv = 4, 128, 128
    N = len(lens)
    _say(f"prefill {lens} then {steps} decode steps")
    total = [L + steps for L in lens]
    cu_full = kda_inputs.cu_from_lengths(total)
    x = kda_inputs.generate(74, int(cu_full[-1]), H, dk, dv, "bf16", num_seqs=N, with_s0=True)
    o_ref, s_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu_full, initial_state=x["s0"])
    # prefill: the first lens[n] tokens of every sequence, packed
    pre = np.concatenate([np.arange(cu_full[n], cu_full[n] + lens[n]) for n in range(N)])
    cu_pre = torch.from_numpy(kda_inputs.cu_from_lengths(lens).astype(np.int32)).cuda()
    dp = {name: dev(x[name][pre], "bf16") for name in ("q", "k", "v", "g", "b")}
    s = torch.from_numpy(x["s0"]).cuda()
    _, s, _ = kda.kda_fwd(dp["q"], dp["k"], dp["v"], dp["g"], dp["b"], cu_pre, s)
    outs = []
    for t in range(steps):
        rows = np.array([cu_full[n] + lens[n] + t for n in range(N)])
        ds = {name: dev(x[name][rows], "bf16") for name in ("q", "k", "v", "g", "b")}
        o, s = kda.kda_decode(ds["q"], ds["k"], ds["v"], ds["g"], ds["b"], s, out_state=s)
        outs.append(host(o))
    torch.cuda.synchronize()
    o_dec = np.stack(outs, axis=1)                      # [N, steps, H, dv]
    ref = np.stack([o_ref[cu_full[n] + lens[n]: cu_full[n + 1]] for n in range(N)])
    e1, e2 = max_over_rms(o_dec, ref), frob_rel(host(s), s_ref)
    _say(f"prefill+decode: o max/rms {e1:.2e} final state frob {e2:.2e}")
    assert e1 <= BF16_MAX_RMS and e2 <= BF16_FROB


def test_decode_serving_shape_sampled():
    """The timed decode shape (256 sequences x 32 heads, d = 128, bf16 inputs,
    fp32 state updated in place), checked on sampled sequences."""
    need_gpu()
    N, H, dk, dv = 256, 32, 128, 128
    _say(f"serving shape N={N} H={H} d={dk}")
    x = _step_inputs(75, N, H, dk, dv, "bf16")
    d = _to_dev(x, "bf16")
    s = torch.from_numpy(x["s0"]).cuda()
    o, s = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], s, out_state=s)
    o, s = host(o), host(s)
    seqs = np.array([0, 1, 97, 128, 255])
    sub = {name: x[name][seqs] for name in ("q", "k", "v", "g", "b")}
    o_ref, s_ref = oracle.fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["b"], cu_seqlens=np.arange(len(seqs) + 1),
                              initial_state=x["s0"][seqs])
    e1, e2 = max_over_rms(o[seqs], o_ref), frob_rel(s[seqs], s_ref)
    _say(f"serving shape sampled: o max/rms {e1:.2e} state frob {e2:.2e}")
    assert e1 <= BF16_MAX_RMS and e2 <= BF16_FROB


def test_decode_empty_batch():
    need_gpu()
    e = torch.empty((0, 2, 64), device="cuda", dtype=torch.bfloat16)
    o, s = kda.kda_decode(e, e, e, e, torch.empty((0, 2), device="cuda", dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64) and s.shape == (0, 2, 64, 64)
