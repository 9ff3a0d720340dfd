"""The library under HIP graph capture (torch.cuda.CUDAGraph on ROCm), through the C ABI.

The entry points enqueue kernels only (no allocation, no memset, no host
synchronisation), so a serving loop or a training step can be captured once
and replayed.  Each test captures a sequence of calls, replays the graph
several times with eager work and synchronisations in between, and checks
every replay bitwise against the same calls made eagerly.  A last test runs
independent calls concurrently on three streams and checks them bitwise
against the same calls made one after another.
"""
import numpy as np
import pytest

import kda_inputs

from gpu_util import dev, need_gpu, torch

import gated_delta_rule_41_amd as kda

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)


def test_decode_steps_in_a_graph():
    """Eight decode steps on a resident state, captured once and replayed."""
    need_gpu()
    N, H, d, steps = 32, 8, 128, 8
    _say(f"decode: {steps} steps, N={N} H={H} d={d}")
    xs = [kda_inputs.generate(700 + t, N, H, d, d, "bf16", num_seqs=N, with_s0=(t == 0)) for t in range(steps)]
    toks = [{k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b")} for x in xs]
    s_init = torch.from_numpy(xs[0]["s0"]).cuda()

    def run(state, outs):
        for t in range(steps):
            o, _ = kda.kda_decode(toks[t]["q"], toks[t]["k"], toks[t]["v"], toks[t]["g"], toks[t]["b"], state,
                                  out_state=state)
            outs[t].copy_(o)

    # eager reference
    s_ref = s_init.clone()
    o_ref = [torch.empty((N, H, d), device="cuda") for _ in range(steps)]
    run(s_ref, o_ref)
    torch.cuda.synchronize()
    # capture (warm up on a side stream first, as torch requires)
    s_g = s_init.clone()
    o_g = [torch.empty((N, H, d), device="cuda") for _ in range(steps)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(s_g, o_g)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(s_g, o_g)
    for rep in range(3):
        s_g.copy_(s_init)
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for t in range(steps):
            assert torch.equal(o_g[t], o_ref[t]), (rep, t)
        assert torch.equal(s_g, s_ref), rep
    _say("decode replays bitwise equal to eager")


def test_forward_backward_in_a_graph():
    """One training step (forward with the state save, backward) captured and replayed."""
    need_gpu()
    lens = [300, 64, 129]
    H, d = 4, 128
    _say(f"fwd+bwd: lens={lens} H={H} d={d}")
    cu = kda_inputs.cu_from_lengths(lens)
    x = kda_inputs.generate(710, int(cu[-1]), H, d, d, "bf16", num_seqs=len(lens), with_s0=True, with_grads=True)
    t = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b", "dO")}
    cu_t = torch.from_numpy(cu.astype(np.int32)).cuda()
    s0 = torch.from_numpy(x["s0"]).cuda()
    dS = torch.from_numpy(x["dS"]).cuda()
    names = ("dq", "dk", "dv", "dg", "dbeta", "dS0")

    def step():
        o, sf, saved = kda.kda_fwd(t["q"], t["k"], t["v"], t["g"], t["b"], cu_t, s0, save_for_bwd=True)
        gr = kda.kda_bwd(t["q"], t["k"], t["v"], t["g"], t["b"], saved, t["dO"], cu_t, s0, dS)
        return [o, sf] + [gr[n] for n in names]

    ref = [a.clone() for a in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rep in range(3):
        for a in outs:
            a.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for name, a, r in zip(("o", "final_state") + names, outs, ref):
            assert torch.equal(a, r), (rep, name)
    _say("fwd+bwd replays bitwise equal to eager")


def test_concurrent_streams_share_no_state():
    """Three independent calls in flight at once on three streams (a training step, a
    two-level long-sequence forward, decode steps) give bitwise the results of the same
    calls made one after another: the library keeps no state between calls."""
    need_gpu()
    _say("concurrent streams: fwd+bwd, two-level forward, decode")
    lens = [300, 64, 129]
    cu = kda_inputs.cu_from_lengths(lens)
    x = kda_inputs.generate(720, int(cu[-1]), 4, 128, 128, "bf16", num_seqs=len(lens), with_s0=True,
                            with_grads=True)
    a = {k: dev(x[k], "bf16") for k in ("q", "k", "v", "g", "b", "dO")}
    cu_a = torch.from_numpy(cu.astype(np.int32)).cuda()
    s0a = torch.from_numpy(x["s0"]).cuda()
    dSa = torch.from_numpy(x["dS"]).cuda()
    T_long = 40960                                    # one document, 2 heads: the library splits it
    y = kda_inputs.generate(721, T_long, 2, 128, 128, "bf16", num_seqs=1, with_s0=True)
    b = {k: dev(y[k], "bf16") for k in ("q", "k", "v", "g", "b")}
    s0b = torch.from_numpy(y["s0"]).cuda()
    z = kda_inputs.generate(722, 64, 8, 128, 128, "bf16", num_seqs=64, with_s0=True)
    c = {k: dev(z[k], "bf16") for k in ("q", "k", "v", "g", "b")}
    s0c = torch.from_numpy(z["s0"]).cuda()
    names = ("dq", "dk", "dv", "dg", "dbeta", "dS0")

    def train():
        o, sf, saved = kda.kda_fwd(a["q"], a["k"], a["v"], a["g"], a["b"], cu_a, s0a, save_for_bwd=True)
        gr = kda.kda_bwd(a["q"], a["k"], a["v"], a["g"], a["b"], saved, a["dO"], cu_a, s0a, dSa)
        return [o, sf] + [gr[n] for n in names]

    def long_fwd():
        o, sf, _ = kda.kda_fwd(b["q"], b["k"], b["v"], b["g"], b["b"], None, s0b)
        return [o, sf]

    def decode():
        st = s0c.clone()
        outs = []
        for t in range(4):   # the same token four times: the state moves on each step
            o, st = kda.kda_decode(c["q"], c["k"], c["v"], c["g"], c["b"], st, out_state=st)
            outs.append(o)
        return outs + [st]

    ref = [[r.clone() for r in f()] for f in (train, long_fwd, decode)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = []
    for s, f in zip(streams, (train, long_fwd, decode)):
        with torch.cuda.stream(s):
            got.append(f())
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i, (g_list, r_list) in enumerate(zip(got, ref)):
        for j, (g_t, r_t) in enumerate(zip(g_list, r_list)):
            assert torch.equal(g_t, r_t), (i, j)
    _say("concurrent results bitwise equal to sequential")
