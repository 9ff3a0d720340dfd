"""Oracle-free invariants of the KDA forward and backward at full size, through
the C ABI.

KDA as the pages describe it ("TorchTitan Ascend open source: Kimi K3.1 Pro
adaptation and training practice", sections "Kimi K3.1 Pro model structure"
and "KDA pre/post-processing fusion"), read as the gated delta rule
S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
o_t = S_t^T q_t with q and k L2-normalised, fixes two properties that hold at
any size, so they are checked on whole workloads the oracle cannot finish:

  * linearity: for fixed q, k, g, beta, the outputs (o, S_T) are linear in
    (v, S_0), and the gradients (dq, dk, dv, dg, dbeta, dS_0) are linear in the
    cotangents (dO, dS_T).  Inputs are split into two parts with disjoint
    support (alternate tokens, alternate key rows), so that both parts and their
    sum are exact in the input dtype;
  * scale invariance of the normalisation: o depends on q only through
    q / sqrt(|q|^2 + eps), so q_t . dq_t = eps / (|q_t|^2 + eps) * (qhat_t . dqhat_t),
    which is below 1e-6 of |q_t| |dq_t| at these input norms (|q|^2 ~ dk); the
    same holds for k.

Bars.  Each GPU result is within the parity bar of its exact value (bf16
inputs: max error 2e-2 of the rms, states 1e-2 in the Frobenius norm), and
the exact values satisfy linearity exactly, so the defect
x(a + b) - x(a) - x(b) is bounded by the sum of the three bars.  The
projection that makes q . dq vanish is applied by the kernel in fp32 to fp32
values, so the per-token cosine between q_t and dq_t stays near fp32 rounding;
1e-4 leaves room for the 128-term dot products.
"""
import numpy as np
import pytest

import kda_inputs

from gpu_util import need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dg", "dbeta")


def _say(msg):
    print(f"[gpu-invariants] {msg}", flush=True)


def _load(idx):
    spec, cu, x = kda_inputs.workload(idx)
    bf = lambda a: torch.from_numpy(a).to("cuda", torch.bfloat16)
    d = {n: bf(x[n]) for n in ("q", "k", "v", "g", "b", "dO")}
    d["s0"] = torch.from_numpy(x["s0"]).cuda()
    d["dS"] = torch.from_numpy(x["dS"]).cuda()
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda() if spec["varlen"] else None
    return spec, cu_t, d


def _rms(t):
    return float(torch.sqrt(torch.mean(t.double() ** 2)))


def _frob(t):
    return float(torch.linalg.vector_norm(t.double()))


def _halves(T, dk, dev):
    """Token and key-row masks of two disjoint halves (even / odd)."""
    tok = (torch.arange(T, device=dev) % 2 == 0).view(T, 1, 1)
    row = (torch.arange(dk, device=dev) % 2 == 0).view(1, 1, dk, 1)
    return tok, row


@pytest.mark.parametrize("idx", [2, 4])
def test_forward_linear_in_v_and_initial_state(idx):
    need_gpu()
    spec, cu, d = _load(idx)
    N = spec["B"]
    _say(f"forward linearity, workload {idx} ({spec['name']})")
    T, dk = d["q"].shape[0], d["q"].shape[2]
    tok, row = _halves(T, dk, d["q"].device)
    zero_v, zero_s = torch.zeros_like(d["v"]), torch.zeros_like(d["s0"])
    va, vb = torch.where(tok, d["v"], zero_v), torch.where(tok, zero_v, d["v"])
    sa, sb = torch.where(row, d["s0"], zero_s), torch.where(row, zero_s, d["s0"])
    assert torch.equal(va + vb, d["v"]) and torch.equal(sa + sb, d["s0"])

    def run(v, s0):
        o, sf, _ = kda.kda_fwd(d["q"], d["k"], v, d["g"], d["b"], cu, s0, num_seqs=None if cu is not None else N)
        return o, sf

    o, sf = run(d["v"], d["s0"])
    oa, sfa = run(va, sa)
    ob, sfb = run(vb, sb)
    torch.cuda.synchronize()
    e_o = float((o.double() - oa.double() - ob.double()).abs().max())
    bar_o = 2e-2 * (_rms(o) + _rms(oa) + _rms(ob))
    e_s = _frob(sf.double() - sfa.double() - sfb.double())
    bar_s = 1e-2 * (_frob(sf) + _frob(sfa) + _frob(sfb))
    _say(f"  o defect {e_o:.3e} (bar {bar_o:.3e}), final state defect {e_s:.3e} (bar {bar_s:.3e})")
    assert e_o <= bar_o and e_s <= bar_s


@pytest.mark.parametrize("idx", [2, 4])
def test_backward_linear_in_cotangents(idx):
    need_gpu()
    spec, cu, d = _load(idx)
    N = spec["B"]
    ns = None if cu is not None else N
    _say(f"backward linearity in (dO, dS_T), workload {idx}")
    T, dk = d["q"].shape[0], d["q"].shape[2]
    tok, row = _halves(T, dk, d["q"].device)
    zero_o, zero_s = torch.zeros_like(d["dO"]), torch.zeros_like(d["dS"])
    da, db = torch.where(tok, d["dO"], zero_o), torch.where(tok, zero_o, d["dO"])
    sa, sb = torch.where(row, d["dS"], zero_s), torch.where(row, zero_s, d["dS"])
    _, _, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu, d["s0"], num_seqs=ns, save_for_bwd=True)

    def run(dO, dS):
        r = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, dO, cu, d["s0"], dS, num_seqs=ns)
        return {n: r[n] for n in GRADS + ("dS0",)}

    g = run(d["dO"], d["dS"])
    ga = run(da, sa)
    gb = run(db, sb)
    torch.cuda.synchronize()
    for n in GRADS:
        e = float((g[n].double() - ga[n].double() - gb[n].double()).abs().max())
        bar = 2e-2 * (_rms(g[n]) + _rms(ga[n]) + _rms(gb[n]))
        _say(f"  {n} defect {e:.3e} (bar {bar:.3e})")
        assert e <= bar, n
    e = _frob(g["dS0"].double() - ga["dS0"].double() - gb["dS0"].double())
    bar = 1e-2 * (_frob(g["dS0"]) + _frob(ga["dS0"]) + _frob(gb["dS0"]))
    _say(f"  dS0 defect {e:.3e} (bar {bar:.3e})")
    assert e <= bar


def test_normalisation_scale_invariance():
    """q_t . dq_t and k_t . dk_t vanish per token (workload 2, every token)."""
    need_gpu()
    spec, cu, d = _load(2)
    N = spec["B"]
    _say("q . dq and k . dk per token, workload 2")
    _, _, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], None, d["s0"], num_seqs=N, save_for_bwd=True)
    r = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], None, d["s0"], d["dS"], num_seqs=N)
    torch.cuda.synchronize()
    for x, dx, name in ((d["q"], r["dq"], "q"), (d["k"], r["dk"], "k")):
        xd, gd = x.double(), dx.double()
        dot = (xd * gd).sum(-1).abs()
        den = torch.linalg.vector_norm(xd, dim=-1) * torch.linalg.vector_norm(gd, dim=-1)
        assert bool(torch.all(den > 0)), name
        cos = float((dot / den).max())
        _say(f"  max |{name}.d{name}| / (|{name}| |d{name}|) over {dot.numel()} tokens x heads: {cos:.2e}")
        assert cos <= 1e-4, name
