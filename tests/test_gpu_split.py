"""GPU parity of the two-level forward for long sequences, through the C ABI.

With few (sequence, head) chains and long documents, kda_fwd cuts every
document into segments, computes each segment's affine map in parallel,
composes the maps per document and reruns the segments from their entering
states.  These cases are sized so that the library takes that path (the
workspace it asks for is non-zero); they compare it with the fp64 oracle
and with the one-pass forward (KDA_FLAG_SEQUENTIAL).  Tolerances are the ones
in tests/gpu_util.py.
"""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import (BF16_FROB, BF16_MAX_RMS, dev, frob_rel, host, max_over_rms, need_gpu, torch)

import gated_delta_rule_41_amd as kda
from gated_delta_rule_41_amd import _lib

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-split] {msg}", flush=True)


def _splits(T, N, H, dk, dv):
    cfg = _lib.make_config(H, dk, dv, _lib.KDA_BF16, _lib.KDA_F32)
    return _lib.kda_fwd_workspace_size(cfg, T, N) > 0


def _run(x, cu, N, sequential=False, with_s0=True):
    d = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b")}
    cu_t = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda() if cu is not None else None
    s0 = torch.from_numpy(x["s0"]).cuda() if with_s0 else None
    o, sf, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], cu_t, s0, num_seqs=N, sequential=sequential)
    torch.cuda.synchronize()
    return host(o), host(sf)


def _check(o, sf, o_ref, sf_ref, tag):
    assert np.isfinite(o).all() and np.isfinite(sf).all(), tag
    e1, e2 = max_over_rms(o, o_ref), frob_rel(sf, sf_ref)
    _say(f"{tag}: o max/rms {e1:.2e} final state frob {e2:.2e}")
    assert e1 <= BF16_MAX_RMS and e2 <= BF16_FROB, tag


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_split_one_long_sequence(dk, dv):
    need_gpu()
    T, H = 1 << 17, 2
    assert _splits(T, 1, H, dk, dv)
    _say(f"one sequence T={T} H={H} dk={dk} dv={dv}")
    x = kda_inputs.generate(81, T, H, dk, dv, "bf16", num_seqs=1, with_s0=True)
    o, sf = _run(x, None, 1)
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], initial_state=x["s0"])
    _check(o, sf, o_ref, sf_ref, f"split {dk}x{dv}")
    # against the one-pass forward: same chunks, different rounding only
    o1, sf1 = _run(x, None, 1, sequential=True)
    e1, e2 = max_over_rms(o, o1), frob_rel(sf, sf1)
    _say(f"split vs one-pass: o max/rms {e1:.2e} final state frob {e2:.2e}")
    assert e1 <= BF16_MAX_RMS and e2 <= BF16_FROB


def test_split_documents_of_mixed_length_and_zero_state():
    """Packed documents of very different lengths (one empty, one of a single
    token, others spanning many segments with ragged ends), no initial state."""
    need_gpu()
    lens = [50000, 1, 0, 69999, 10240]
    N, H, dk, dv = len(lens), 2, 128, 128
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    assert _splits(T, N, H, dk, dv)
    _say(f"documents {lens} H={H}")
    x = kda_inputs.generate(82, T, H, dk, dv, "bf16", num_seqs=N, with_s0=False)
    o, sf = _run(x, cu, N, with_s0=False)
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu)
    _check(o, sf, o_ref, sf_ref, "mixed documents")
    assert np.all(sf[2] == 0.0)   # the empty document ends in its (zero) initial state


def test_split_initial_state_reaches_every_document():
    """Each document starts from its own initial state: with a gate close to 1
    (slow decay) the state carries across many segments, so a wrong entering
    state would show in outputs far from the document start."""
    need_gpu()
    lens = [40000, 30000]
    N, H, dk, dv = len(lens), 2, 64, 64
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    assert _splits(T, N, H, dk, dv)
    _say(f"slow decay, documents {lens}")
    x = kda_inputs.generate(83, T, H, dk, dv, "bf16", num_seqs=N, with_s0=True)
    x["g"] = kda_inputs.round_bf16(x["g"] * 1e-3)   # alpha = exp(g) within 1e-3 of 1
    x["b"] = kda_inputs.round_bf16(x["b"] - 4.0)    # small beta: the state changes slowly
    x["s0"] = x["s0"] * 10.0
    o, sf = _run(x, cu, N)
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    _check(o, sf, o_ref, sf_ref, "slow decay")


def test_split_deterministic():
    need_gpu()
    T, H, dk, dv = 1 << 16, 2, 128, 128
    assert _splits(T, 1, H, dk, dv)
    _say("split determinism")
    x = kda_inputs.generate(84, T, H, dk, dv, "bf16", num_seqs=1, with_s0=True)
    o1, sf1 = _run(x, None, 1)
    o2, sf2 = _run(x, None, 1)
    assert np.array_equal(o1, o2) and np.array_equal(sf1, sf2)
