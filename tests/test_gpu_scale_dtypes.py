"""GPU checks of the query scale and of bf16 outputs, through the C ABI.

The oracle has no query scale (the pages' formula has none; the ABI carries
one for callers), so the scale is pinned by exact identities instead:
scaling the normalised query by 1/2 is exact in floating point and o is linear
in it, so o(scale=1/2) = o(scale=1) / 2 bitwise, for the chunked forward and
for the decode step; and the loss <dO, o> with scale s is the loss with scale 1
and upstream gradient s dO, so the gradients agree (up to rounding).
bf16 outputs are compared with the fp32 outputs of the same call: beyond the
storage rounding (round to nearest, at most 2^-8 |x|) they must agree to
1e-5 of the RMS, i.e. the bf16-output kernels compute the same values.
"""
import numpy as np
import pytest

import kda_inputs

from gpu_util import dev, host, max_over_rms, need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu

SAME = 1e-5   # bf16 output vs fp32 output of the same computation, beyond storage rounding


def _say(msg):
    print(f"[gpu-scale] {msg}", flush=True)


def _inputs(seed, lens, H=3, dk=128, dv=128, grads=False):
    cu = kda_inputs.cu_from_lengths(lens)
    x = kda_inputs.generate(seed, int(cu[-1]), H, dk, dv, "bf16", num_seqs=len(lens), with_s0=True,
                            with_grads=grads)
    d = {k: dev(x[k], "bf16") for k in (("q", "k", "v", "g", "b", "dO") if grads else ("q", "k", "v", "g", "b"))}
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    s0 = torch.from_numpy(x["s0"]).cuda()
    return x, d, cu_t, s0


def _storage_excess(x_bf16, x_f32):
    a, r = host(x_bf16), host(x_f32)
    return float((np.abs(a - r) - 2.0 ** -8 * np.abs(r)).max() / np.sqrt(np.mean(r * r)))


def test_forward_scale_half_is_exact():
    need_gpu()
    _say("forward, scale 1/2")
    x, d, cu_t, s0 = _inputs(91, [200, 64, 137])
    o1, sf1, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0)
    oh, sfh, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(oh, 0.5 * o1)
    assert torch.equal(sfh, sf1)      # the state does not see the query


def test_decode_scale_half_is_exact():
    need_gpu()
    _say("decode, scale 1/2")
    x = kda_inputs.generate(92, 16, 4, 128, 128, "bf16", num_seqs=16, with_s0=True)
    d = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o1, s1 = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], s0)
    oh, sh = kda.kda_decode(d["q"], d["k"], d["v"], d["g"], d["b"], s0, scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(oh, 0.5 * o1) and torch.equal(sh, s1)


def test_backward_scale_equals_scaled_upstream_gradient():
    """Gradients with scale s and dO equal those with scale 1 and s dO."""
    need_gpu()
    _say("backward, scale 1/2 vs dO / 2")
    x, d, cu_t, s0 = _inputs(93, [150, 64, 90], grads=True)
    dS = torch.from_numpy(x["dS"]).cuda()
    _, _, sv_h = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, scale=0.5, save_for_bwd=True)
    gh = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], sv_h, d["dO"], cu_t, s0, dS, scale=0.5)
    _, _, sv_1 = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, save_for_bwd=True)
    g1 = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], sv_1, (0.5 * d["dO"].float()).bfloat16(), cu_t, s0, dS)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        e = max_over_rms(host(gh[name]), host(g1[name]))
        _say(f"  {name}: max/rms {e:.2e}")
        assert e <= 1e-3, name


def test_backward_bf16_outputs():
    need_gpu()
    _say("backward, bf16 gradients")
    x, d, cu_t, s0 = _inputs(94, [130, 64, 1, 70], grads=True)
    dS = torch.from_numpy(x["dS"]).cuda()
    _, _, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, save_for_bwd=True)
    gf = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS)
    gb = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert gb[name].dtype == torch.bfloat16
        e = _storage_excess(gb[name], gf[name])
        _say(f"  {name}: excess over bf16 storage {e:.2e}")
        assert e <= SAME, name
    assert torch.equal(gb["dS0"], gf["dS0"])   # d(initial state) is fp32 in both


def test_split_forward_bf16_output():
    """The two-level path (one long sequence, few heads) with bf16 o."""
    need_gpu()
    T, H = 1 << 16, 2
    _say(f"two-level forward T={T} H={H}, bf16 o")
    x = kda_inputs.generate(95, T, H, 128, 128, "bf16", num_seqs=1, with_s0=True)
    d = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    of, sff, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], None, s0)
    ob, sfb, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], None, s0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert ob.dtype == torch.bfloat16
    e = _storage_excess(ob, of)
    _say(f"  o excess over bf16 storage {e:.2e}")
    assert e <= SAME
    assert torch.equal(sfb, sff)
