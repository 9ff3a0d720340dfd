"""The autograd wrapper (gated_delta_rule_41_amd.kda) against the oracle and
against direct kda_fwd / kda_bwd calls, through the C ABI."""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import BF16_FROB, BF16_MAX_RMS, dev, frob_rel, host, max_over_rms, need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu


def test_autograd_matches_direct_calls_and_oracle():
    need_gpu()
    print("[gpu-autograd] kda() under autograd", flush=True)
    lens = [150, 64, 33]
    H, d = 3, 128
    cu = kda_inputs.cu_from_lengths(lens)
    x = kda_inputs.generate(720, int(cu[-1]), H, d, d, "bf16", num_seqs=len(lens), with_s0=True, with_grads=True)
    leaves = {n: dev(x[n], "bf16").requires_grad_(True) for n in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda().requires_grad_(True)
    dO = dev(x["dO"], "bf16")
    dS = torch.from_numpy(x["dS"]).cuda()
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, sf = kda.kda(leaves["q"], leaves["k"], leaves["v"], leaves["g"], leaves["b"], cu_t, s0)
    loss = (o * dO.float()).sum() + (sf * dS).sum()
    loss.backward()
    torch.cuda.synchronize()
    # direct calls
    d = {n: t.detach() for n, t in leaves.items()}
    o2, sf2, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0.detach(), save_for_bwd=True)
    gr = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, dO, cu_t, s0.detach(), dS)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2) and torch.equal(sf.detach(), sf2)
    for n, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("b", "dbeta")):
        assert torch.equal(leaves[n].grad, gr[gname].to(torch.bfloat16)), n
    assert torch.equal(s0.grad, gr["dS0"])
    # and against the oracle (bf16 gradients: storage rounding allowed on top of the bar)
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["dO"], cu_seqlens=cu, initial_state=x["s0"],
                     dS_final=x["dS"])
    for n, rname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("b", "db")):
        a, r = host(leaves[n].grad), ref[rname]
        e = float((np.abs(a - r) - 2.0 ** -8 * np.abs(r)).max() / np.sqrt(np.mean(r * r)))
        print(f"[gpu-autograd]   d{n}: excess over bf16 storage / rms {e:.2e}", flush=True)
        assert e <= BF16_MAX_RMS, n
    assert frob_rel(host(s0.grad), ref["dS0"]) <= BF16_FROB
    o_ref, _ = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    assert max_over_rms(host(o), o_ref) <= BF16_MAX_RMS
