"""GPU parity of the three full-size workloads on every chain, against the
fp64 oracle through the C ABI.

  workload 2  bf16 B=4 H=32 T=8192 d=128: forward and backward, every tensor
  workload 3  bf16 B=1 H=16 T=1048576 d=128: forward (two-level split), every
              head; the oracle runs in two groups of eight heads to bound host
              memory
  workload 4  bf16 H=32 T=65536, 64 packed documents: forward and backward,
              every tensor

Every output and gradient is compared whole against the bf16 bars:
max|x - r| / rms(r) <= 2e-2 and ||x - r||_F / ||r||_F <= 1e-2.  Each tensor's
two errors are printed (run with -s to see them).
"""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import dev, host, need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu

MAX_RMS, FROB = 2e-2, 1e-2


def _say(msg):
    print(f"[gpu-full] {msg}", flush=True)


class Err:
    """max|x - r|, sum (x - r)^2 and sum r^2 accumulated over pieces of a tensor."""

    def __init__(self):
        self.mx, self.se, self.sr, self.n = 0.0, 0.0, 0.0, 0

    def add(self, x, r):
        x = np.asarray(x, dtype=np.float64)
        r = np.asarray(r, dtype=np.float64)
        assert np.isfinite(x).all()
        d = x - r
        self.mx = max(self.mx, float(np.abs(d).max(initial=0.0)))
        self.se += float(np.sum(d * d))
        self.sr += float(np.sum(r * r))
        self.n += r.size
        return self

    def max_over_rms(self):
        return self.mx / max(np.sqrt(self.sr / max(self.n, 1)), 1e-30)

    def frob(self):
        return np.sqrt(self.se) / max(np.sqrt(self.sr), 1e-30)


def _check(tag, errs):
    _say(tag + ": " + "  ".join(f"{k} max/rms={e.max_over_rms():.2e} frob={e.frob():.2e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert e.max_over_rms() <= MAX_RMS and e.frob() <= FROB, (tag, k, e.max_over_rms(), e.frob())


def _gpu_fwd_bwd(x, cu, num_seqs, bwd):
    d = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b") + (("dO",) if bwd else ())}
    s0 = torch.from_numpy(x["s0"]).cuda()
    cu_t = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda() if cu is not None else None
    o, sf, saved = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, num_seqs=num_seqs,
                               save_for_bwd=bwd)
    gr = None
    if bwd:
        dS = torch.from_numpy(x["dS"]).cuda()
        gr = kda.kda_bwd(d["q"], d["k"], d["v"], d["g"], d["b"], saved, d["dO"], cu_t, s0, dS, num_seqs=num_seqs)
    torch.cuda.synchronize()
    del d
    return o, sf, gr


@pytest.mark.timeout(900)
@pytest.mark.parametrize("idx", [2, 4])
def test_full_workload_forward_backward(idx):
    need_gpu()
    spec, cu, x = kda_inputs.workload(idx)
    _say(f"workload {idx} ({spec['name']}): forward + backward, every tensor")
    N = spec["B"]
    o, sf, gr = _gpu_fwd_bwd(x, cu, N, True)
    got = {"o": host(o), "sf": host(sf)}
    got.update({k: host(gr[n]) for k, n in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("db", "dbeta"),
                                           ("dS0", "dS0"))})
    del o, sf, gr
    _say(f"workload {idx}: GPU done, oracle running")
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    ref = oracle.bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["dO"], cu_seqlens=cu, initial_state=x["s0"],
                     dS_final=x["dS"])
    want = {"o": o_ref, "sf": sf_ref, "dq": ref["dq"], "dk": ref["dk"], "dv": ref["dv"], "dg": ref["dg"],
            "db": ref["db"], "dS0": ref["dS0"]}
    _check(f"workload {idx}", {k: Err().add(got[k], want[k]) for k in got})


@pytest.mark.timeout(1200)
def test_full_workload3_long_context_forward():
    need_gpu()
    spec, cu, x = kda_inputs.workload(3)
    _say(f"workload 3 ({spec['name']}): forward on every head; inputs generated")
    o, sf, _ = _gpu_fwd_bwd(x, cu, 1, False)
    _say("workload 3: GPU forward done, oracle running in two groups of 8 heads")
    errs = {"o": Err(), "sf": Err()}
    H = spec["H"]
    for h0 in range(0, H, 8):
        heads = list(range(h0, min(h0 + 8, H)))
        sub = {k: np.ascontiguousarray(x[k][:, heads]) for k in ("q", "k", "v", "g", "b")}
        o_ref, sf_ref = oracle.fwd(sub["q"], sub["k"], sub["v"], sub["g"], sub["b"], cu_seqlens=cu,
                                   initial_state=np.ascontiguousarray(x["s0"][:, heads]), threads=len(heads))
        del sub
        errs["o"].add(host(o[:, h0:h0 + len(heads)]), o_ref)
        errs["sf"].add(host(sf[:, h0:h0 + len(heads)]), sf_ref)
        del o_ref, sf_ref
        _say(f"workload 3: heads {heads[0]}..{heads[-1]} compared")
    _check("workload 3", errs)
