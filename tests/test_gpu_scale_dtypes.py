"""GPU checks of the query scale and of bf16 outputs, through the C ABI.

The oracle has no query scale (the pages' formula has none; the ABI carries
one for callers), so the scale is pinned by exact identities instead:
scaling the normalised query by 1/2 is exact in floating point and o is linear
in it, so o(scale=1/2) = o(scale=1) / 2 bitwise, for the chunked forward and
for the decode step; and the loss <dO, o> with scale s is the loss with scale 1
and upstream gradient s dO, so the gradients agree (up to rounding).
A non-default eps of the L2 norm is checked against the oracle at that eps.
bf16 outputs are compared with the fp32 outputs of the same call: beyond the
storage rounding (round to nearest, at most 2^-8 |x|) they must agree to
1e-5 of the RMS, i.e. the bf16-output kernels compute the same values.
"""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import dev, frob_rel, host, inf_rel, max_over_rms, need_gpu, torch

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


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("bf16", 128, 128)])
def test_norm_eps_forward_backward_decode(dtype, dk, dv):
    """A non-default eps of the L2 norm reaches the forward, the backward (through the saved
    norms) and the decode step.  q and k are scaled by 1/16 (exact) so |q|^2 is ~dk/256 and
    eps = 0.25 changes every normalised row; the runs are compared with the oracle at the
    same eps, and the default eps is checked to give a different o (the test is not vacuous)."""
    need_gpu()
    eps = 0.25
    _say(f"norm eps {eps} {dtype} dk={dk} dv={dv}")
    lens = [150, 64, 1]
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    x = kda_inputs.generate(97, T, 2, dk, dv, dtype, num_seqs=len(lens), with_s0=True, with_grads=True)
    x["q"] = x["q"] / 16.0
    x["k"] = x["k"] / 16.0
    d = {k: dev(x[k], dtype) for k in ("q", "k", "v", "g", "b", "dO")}
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    s0 = torch.from_numpy(x["s0"]).cuda()
    dS = torch.from_numpy(x["dS"]).cuda()
    o, sf, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, eps=eps, save_for_bwd=True)
    gr = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS, eps=eps)
    o_def, _, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0)
    # decode: the first token of every document as a one-token step from its initial state
    first = cu[:-1][np.asarray(lens) > 0]
    pick = lambda a: a[first]
    dd = {k: dev(pick(x[k]), dtype) for k in ("q", "k", "v", "g", "b")}
    s0d = torch.from_numpy(x["s0"][np.asarray(lens) > 0]).cuda()
    o_dec, st_dec = kda.kda_decode(dd["q"], dd["k"], dd["v"], dd["g"], dd["b"], s0d, eps=eps)
    torch.cuda.synchronize()

    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"],
                               eps=eps)
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["dO"], cu_seqlens=cu, initial_state=x["s0"],
                     dS_final=x["dS"], eps=eps)
    n1 = len(first)
    od_ref, sd_ref = oracle.fwd(pick(x["q"]), pick(x["k"]), pick(x["v"]), pick(x["g"]), pick(x["b"]),
                                cu_seqlens=np.arange(n1 + 1), initial_state=x["s0"][np.asarray(lens) > 0], eps=eps)
    pairs = [("o", host(o), o_ref, False), ("sf", host(sf), sf_ref, True), ("dq", host(gr["dq"]), ref["dq"], False),
             ("dk", host(gr["dk"]), ref["dk"], False), ("dv", host(gr["dv"]), ref["dv"], False),
             ("dg", host(gr["dg"]), ref["dg"], False), ("db", host(gr["dbeta"]), ref["db"], False),
             ("dS0", host(gr["dS0"]), ref["dS0"], True), ("o_dec", host(o_dec), od_ref, False),
             ("state_dec", host(st_dec), sd_ref, True)]
    errs = {}
    for name, a, r, state in pairs:
        assert np.isfinite(a).all(), name
        errs[name] = inf_rel(a, r) if dtype == "f32" else (frob_rel(a, r) if state else max_over_rms(a, r))
    _say(" ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for name, a, r, state in pairs:
        bar = 1e-4 if dtype == "f32" else (1e-2 if state else 2e-2)
        assert errs[name] <= bar, (name, errs[name])
    # the default eps gives a visibly different output on these rows
    assert max_over_rms(host(o_def), o_ref) > 0.1


def test_fp32_inputs_bf16_outputs():
    """fp32 inputs with o and the gradients written in bf16: the same values as the fp32-output
    call of the fp32-input kernels, beyond the storage rounding."""
    need_gpu()
    _say("fp32 inputs, bf16 outputs (forward and backward)")
    lens = [130, 64, 1, 70]
    cu = kda_inputs.cu_from_lengths(lens)
    x = kda_inputs.generate(98, int(cu[-1]), 3, 64, 64, "f32", num_seqs=len(lens), with_s0=True, with_grads=True)
    d = {k: dev(x[k], "f32") for k in ("q", "k", "v", "g", "b", "dO")}
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    s0 = torch.from_numpy(x["s0"]).cuda()
    dS = torch.from_numpy(x["dS"]).cuda()
    of, sff, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, save_for_bwd=True)
    ob, sfb, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, out_dtype=torch.bfloat16)
    gf = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS)
    gb = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert ob.dtype == torch.bfloat16
    assert torch.equal(sfb, sff)       # the final state is fp32 in both
    e = _storage_excess(ob, of)
    _say(f"  o: excess over bf16 storage {e:.2e}")
    assert e <= SAME
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert gb[name].dtype == torch.bfloat16
        e = _storage_excess(gb[name], gf[name])
        _say(f"  {name}: excess over bf16 storage {e:.2e}")
        assert e <= SAME, name
    assert torch.equal(gb["dS0"], gf["dS0"])
