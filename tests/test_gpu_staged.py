"""The staged forward (KDA_FLAG_STAGED) stage by stage against the chunked
fp64 reference, through the C ABI.

The staged path writes every intermediate of the chunk form of the pages'
intra-chunk processing plus inter-chunk state passing ("TorchTitan Ascend open
source: Kimi K3.1 Pro adaptation and training practice", section "KDA
pre/post-processing fusion"): G, Akk, Aqk, T, W, Ut, U and the state entering
each chunk.  oracle/chunked.py computes the same matrices in fp64 (its own
pins tie it to the token recurrence).  Both sides see the same inputs (bf16
values are exact in fp64), so the only difference is fp32 arithmetic: every
stage must match to 1e-4 of its largest entry, and o and the final state the
token-recurrence oracle to 1e-4 (inf-norm relative), whatever the gates.
"""
import numpy as np
import pytest

import kda_inputs
import oracle
from oracle import chunked

from gpu_util import dev, host, inf_rel, need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu

LENS = [150, 64, 33]     # a partial last chunk in two documents
STAGE_BAR = 1e-4
OUT_BAR = 1e-4


def _say(msg):
    print(f"[gpu-staged] {msg}", flush=True)


def _stage_err(a, r):
    scale = max(float(np.abs(r).max()), 1e-30)
    return float(np.abs(a - r).max()) / scale


def _run(seed, lens, H, dk, dv, dtype, gates=None, out_dtype=None, chunk=64):
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    x = kda_inputs.generate(seed, T, H, dk, dv, dtype, num_seqs=len(lens), with_s0=True)
    if gates == "mixed":
        x["g"] = kda_inputs.mix_gates(x["g"], seed, dtype)
    t = {n: dev(x[n], dtype) for n in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    o, sf, st = kda.kda_fwd_staged(t["q"], t["k"], t["v"], t["g"], t["b"], cu_t, s0, out_dtype=out_dtype,
                                   chunk=chunk)
    torch.cuda.synchronize()
    return cu, x, host(o), host(sf), {n: host(a) for n, a in st.items()}


@pytest.mark.parametrize("dk,dv,dtype,chunk", [(64, 64, "bf16", 64), (128, 128, "bf16", 64), (64, 128, "f32", 64),
                                              (128, 64, "f32", 64), (128, 128, "bf16", 16), (64, 64, "f32", 32)])
def test_stages_match_chunked_reference(dk, dv, dtype, chunk):
    need_gpu()
    H = 2
    _say(f"stages dk={dk} dv={dv} {dtype} chunk={chunk} lens={LENS}")
    cu, x, o, sf, st = _run(910 + dk + dv, LENS, H, dk, dv, dtype, chunk=chunk)
    ro, rsf, kept = chunked.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"],
                                chunk=chunk, keep_stages=True)
    worst = {}
    for n, h, c0, ref in kept:
        slot = int(cu[n]) // chunk + n + (c0 - int(cu[n])) // chunk
        C = ref["Akk"].shape[0]
        got = {"G": st["G"][slot, h, :C], "Akk": st["Akk"][slot, h, :C, :C], "Aqk": st["Aqk"][slot, h, :C, :C],
               "T": st["T"][slot, h, :C, :C], "W": st["W"][slot, h, :C], "Ut": st["Ut"][slot, h, :C],
               "U": st["U"][slot, h, :C], "S_in": st["S_in"][slot, h]}
        for name, a in got.items():
            e = _stage_err(a, ref[name])
            worst[name] = max(worst.get(name, 0.0), e)
        # rows past the document's end are zero in every stage
        assert not np.any(st["Akk"][slot, h, C:]) and not np.any(st["U"][slot, h, C:])
    _say("  worst stage error / max|ref|: " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))
    for name, e in worst.items():
        assert e <= STAGE_BAR, name
    eo, es = inf_rel(o, ro), inf_rel(sf, rsf)
    _say(f"  o {eo:.1e}  final state {es:.1e} (against the chunked reference)")
    assert eo <= OUT_BAR and es <= OUT_BAR


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_staged_outputs_match_token_oracle_over_the_gate_range(dtype):
    """Fast-forgetting channels (per-token g down to -8) beside g = 0: the staged
    path forms every pair decay directly, so it stays within the fp32 bar."""
    need_gpu()
    H, d = 2, 128
    lens = [200, 64, 1, 130]
    _say(f"gate range {dtype}")
    cu, x, o, sf, _ = _run(930, lens, H, d, d, dtype, gates="mixed")
    ro, rsf = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    eo, es = inf_rel(o, ro), inf_rel(sf, rsf)
    _say(f"  o {eo:.1e}  final state {es:.1e}")
    assert eo <= OUT_BAR and es <= OUT_BAR


def test_staged_equal_sequences_and_bf16_output():
    """cu_seqlens = NULL (equal sequences) and bf16 o: o within bf16 storage
    rounding of the fp32 result, the final state as with fp32 output."""
    need_gpu()
    H, d, N, L = 2, 64, 2, 96
    T = N * L
    x = kda_inputs.generate(940, T, H, d, d, "bf16", num_seqs=N, with_s0=True)
    t = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    o32, sf32, _ = kda.kda_fwd_staged(t["q"], t["k"], t["v"], t["g"], t["b"], None, s0, num_seqs=N)
    o16, sf16, _ = kda.kda_fwd_staged(t["q"], t["k"], t["v"], t["g"], t["b"], None, s0, num_seqs=N,
                                      out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(sf16, sf32)
    cu = kda_inputs.cu_from_lengths([L] * N)
    ro, rsf = oracle.fwd(x["q"], x["k"], x["v"], x["g"], x["b"], cu_seqlens=cu, initial_state=x["s0"])
    assert inf_rel(host(o32), ro) <= OUT_BAR and inf_rel(host(sf32), rsf) <= OUT_BAR


def test_chunk_size_invariance():
    """The chunking changes only rounding (the chunk form reaches the token
    recurrence's result exactly): chunks of 16, 32 and 64 give o and the final
    state within fp32 rounding of each other."""
    need_gpu()
    H, d = 2, 64
    lens = [150, 64, 33]
    res = {}
    for chunk in (16, 32, 64):
        _, _, o, sf, _ = _run(960, lens, H, d, d, "bf16", chunk=chunk)
        res[chunk] = (o, sf)
    for chunk in (16, 32):
        eo, es = inf_rel(res[chunk][0], res[64][0]), inf_rel(res[chunk][1], res[64][1])
        _say(f"chunk {chunk} against 64: o {eo:.1e}, final state {es:.1e}")
        assert eo <= 1e-5 and es <= 1e-5


def test_staged_against_fused_forward():
    """The fused forward within its own bar of the staged one (a cross-check of
    the fast path that needs no oracle, here on the headline dims)."""
    need_gpu()
    H, d = 4, 128
    lens = [300, 77, 256]
    cu = kda_inputs.cu_from_lengths(lens)
    T = int(cu[-1])
    x = kda_inputs.generate(950, T, H, d, d, "bf16", num_seqs=len(lens), with_s0=True)
    t = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "g", "b")}
    s0 = torch.from_numpy(x["s0"]).cuda()
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    os_, sfs, _ = kda.kda_fwd_staged(t["q"], t["k"], t["v"], t["g"], t["b"], cu_t, s0)
    of, sff, _ = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["b"], cu_t, s0)
    torch.cuda.synchronize()
    a, r = host(of), host(os_)
    e = float(np.abs(a - r).max() / np.sqrt(np.mean(r * r)))
    es = float(np.linalg.norm(host(sff) - host(sfs)) / np.linalg.norm(host(sfs)))
    _say(f"fused vs staged: o max/rms {e:.1e}, final state frob {es:.1e}")
    assert e <= 2e-2 and es <= 1e-2
