"""GPU parity of the fused KDA forward against the fp64 oracle, through the C ABI.

Every case prints its name before it touches the GPU.  Inputs come from the
seeded generator shared with the oracle (kda_inputs).  Tolerances are the ones
in tests/gpu_util.py.  The full-size workloads 2-4 are compared on every
chain in test_gpu_full_configs.py.
"""
import numpy as np
import pytest

import kda_inputs
import oracle

from gpu_util import assert_fwd_close, dev, host, need_gpu, run_fwd, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-fwd] {msg}", flush=True)


def test_w0_fp32_full():
    need_gpu()
    _say("workload 0: fp32 B=1 H=2 T=256 d=64")
    spec, cu, x = kda_inputs.workload(0)
    o, sf, *_ = run_fwd(x, "f32", cu=cu)
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu)
    e = assert_fwd_close(o, sf, o_ref, sf_ref, "f32", "w0")
    _say(f"w0 errors {e}")


def test_w1_bf16_full():
    need_gpu()
    _say("workload 1: bf16 B=1 H=16 T=4096 d=128")
    spec, cu, x = kda_inputs.workload(1)
    o, sf, *_ = run_fwd(x, "bf16", cu=cu)
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    e = assert_fwd_close(o, sf, o_ref, sf_ref, "bf16", "w1")
    _say(f"w1 errors {e}")


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 64), ("bf16", 64, 64), ("bf16", 128, 128), ("bf16", 64, 128),
                                         ("bf16", 128, 64)])
def test_ragged_varlen_small(dtype, dk, dv):
    """Several chunks and ragged tails; documents of length 1, 63, 64, 65, 0, 130."""
    need_gpu()
    _say(f"ragged varlen {dtype} dk={dk} dv={dv}")
    lens = [1, 63, 64, 65, 0, 130, 7]
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    x = kda_inputs.generate(77, T, 3, dk, dv, dtype, num_seqs=len(lens), with_s0=True)
    for out_dtype in (torch.float32, torch.bfloat16):
        o, sf, *_ = run_fwd(x, dtype, cu=cu, out_dtype=out_dtype)
        o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
        if out_dtype == torch.bfloat16:
            # storing o in bf16 adds up to 2^-8 |o| (round to nearest, 8-bit significand); the compute
            # error on top of that storage rounding is held to the bf16 bar
            excess = np.abs(host(o) - o_ref) - 2.0 ** -8 * np.abs(o_ref)
            err = excess.max() / np.sqrt(np.mean(o_ref ** 2))
            assert err <= 2e-2, err
        else:
            assert_fwd_close(o, sf, o_ref, sf_ref, dtype, f"ragged {dtype} {dk}x{dv}")
        # the empty document passes its initial state through unchanged
        np.testing.assert_array_equal(host(sf)[4], x["s0"][4].astype(np.float64))


def test_equal_sequences_without_cu_seqlens():
    need_gpu()
    _say("num_seqs=3 equal sequences, cu_seqlens NULL")
    x = kda_inputs.generate(78, 3 * 192, 2, 128, 128, "bf16", num_seqs=3, with_s0=True)
    o, sf, *_ = run_fwd(x, "bf16", num_seqs=3)
    cu = np.array([0, 192, 384, 576])
    o_ref, sf_ref = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    assert_fwd_close(o, sf, o_ref, sf_ref, "bf16", "equal seqs")


def test_empty_input():
    need_gpu()
    _say("T=0")
    z = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((0, 2), dtype=torch.bfloat16, device="cuda")
    s0 = torch.randn(1, 2, 64, 64, device="cuda")
    o, sf, _ = kda.kda_fwd(z, z, z, z, b, None, s0)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64)
    assert torch.equal(sf, s0)


def test_state_carry_and_determinism():
    """Two calls chained through the state at a chunk boundary equal one call
    bitwise, and repeated calls are bitwise identical."""
    need_gpu()
    _say("state carry / determinism")
    x = kda_inputs.generate(79, 1024, 4, 128, 128, "bf16", with_s0=True)
    o, sf, _, d, s0, _ = run_fwd(x, "bf16")
    o2, sf2, _ = kda.kda_fwd(d["q"], d["k"], d["v"], d["g"], d["b"], None, s0)
    a = 512
    oa, sa, _ = kda.kda_fwd(d["q"][:a].contiguous(), d["k"][:a].contiguous(), d["v"][:a].contiguous(),
                            d["g"][:a].contiguous(), d["b"][:a].contiguous(), None, s0)
    ob, sb, _ = kda.kda_fwd(d["q"][a:].contiguous(), d["k"][a:].contiguous(), d["v"][a:].contiguous(),
                            d["g"][a:].contiguous(), d["b"][a:].contiguous(), None, sa)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(sf, sf2)
    assert torch.equal(torch.cat([oa, ob]), o) and torch.equal(sb, sf)


def test_causality_and_document_isolation():
    need_gpu()
    _say("causality / isolation")
    lens = [300, 200, 100]
    cu = kda_inputs.cu_from_lengths(lens)
    x = kda_inputs.generate(80, 600, 2, 128, 128, "bf16", num_seqs=3, with_s0=True)
    o1, sf1, *_ = run_fwd(x, "bf16", cu=cu)
    y = {k: v.copy() for k, v in x.items()}
    y["v"][400:500] = 1000.0       # second document, tokens 100..199
    y["q"][400:500] = np.nan       # NaN must not leak into other documents or earlier tokens
    o2, sf2, *_ = run_fwd(y, "bf16", cu=cu)
    # Every token before the chunk that holds token 400 (the second document's
    # chunks start at 300, 364, 428, ...) is bitwise unchanged.  Inside that
    # chunk, tokens 364..399 may differ by rounding only: a chunk's fp16 operands
    # share one power-of-two scale, chosen from the whole chunk's values.
    assert torch.equal(o1[:364], o2[:364])
    a, b = host(o1[364:400]), host(o2[364:400])
    assert np.isfinite(b).all()
    assert np.abs(a - b).max() <= 1e-2 * np.sqrt(np.mean(a * a))
    assert torch.equal(o1[500:], o2[500:])
    assert torch.equal(sf1[0], sf2[0]) and torch.equal(sf1[2], sf2[2])


