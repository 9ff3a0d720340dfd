"""Benchmark: KDA forward + backward on one MI355X.

Workload: B=4 packed sequences x T=8192 tokens, H=32 heads, dk=dv=128, chunk 64,
bf16 inputs (q, k, v, g, beta logit, dO), fp32 state, fp32 outputs and
gradients; seeded synthetic inputs from kda_inputs (the same recipe the parity
tests use).  One step = one training pass of the whole hot path: kda_fwd with
the state save, then kda_bwd as its two stages (kda_bwd_scan: reverse state
scan; kda_bwd_grads: chunk-parallel gradients), one kernel each.

Prints ONE JSON line.  `value` is whole-job tokens/s of the fwd+bwd step with
inputs already resident in HBM.  `roofline` reports the step's dominant kernel
against the HBM roofline, timed with HIP events on the stream the library
launches on; `roofline_fwd` reports the fused forward on its own (inference
call, no state save), also against the bandwidth of a plain 1 GiB device copy
measured in the same run (`hbm_copy_gbs`) and as a fraction of the dense bf16
MFMA peak (`mfma_frac`, useful FLOPs of the chunked form; see alg_flops_fwd).
`bf16_outputs` times the same step with o and the gradients written in bf16.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same workload
on the host cores.

Algorithmic bytes (inputs read once, outputs written once; what the
implementation saves or recomputes is not counted), per kernel:
  forward         per token-head: q, k, g (dk bf16 each) + v (dv bf16) + beta
                  (bf16) + o (dv fp32); per (sequence, head): initial + final state
  chunk gradients per token-head: q, k, g, v, beta, dO (bf16) + dq, dk, dg, dv,
                  dbeta (fp32)
  state scan      per (sequence, head): dS_final in, d(initial state) out
  decode step     per (sequence, head): the fp32 state read and written once,
                  q, k, g (dk bf16 each) + v (dv bf16) + beta in, o (dv fp32) out

`decode` reports the serving step on its own: 256 sequences x 32 heads, d = 128,
bf16 token inputs, the fp32 state updated in place, one token per call.

`long_context` reports the inference forward on one 1,048,576-token sequence x
16 heads (d = 128, bf16), which takes the library's two-level path, next to
the one-pass forward on the same inputs.  Its inputs are drawn on the device
with a seeded torch generator in the workload's distributions (q, k, v, beta
logit ~ N(0, 1); g = -softplus(N(-2, 1)); initial state ~ N(0, 0.01)), since
drawing 2^31 values per tensor on the host takes minutes.  Its parity against
the oracle is a test case (the same shape, host-drawn inputs).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published


def alg_bytes(B, T, H, dk, dv, kernel):
    th = B * T * H
    state = dk * dv * 4
    return {
        "fwd": th * (3 * dk * 2 + dv * 2 + 2 + dv * 4) + B * H * 2 * state,
        "grads": th * (3 * dk * 2 + dv * 2 + 2 + dv * 2) + th * (3 * dk * 4 + dv * 4 + 4),
        "scan": B * H * 2 * state,
    }[kernel]


def alg_flops_fwd(B, T, H, dk, dv, C=64):
    """Useful multiply-adds x 2 of the chunked forward (no recompute, triangular
    halves counted once): per chunk and head, Akk (strict lower) and Aqk (lower)
    over dk, the unit-lower solve for T, W = T (beta kh Gam) and Ut = T (beta v)
    (lower), U = Ut - W S and O = (qh Gam) S (C x dk x dv each), Aqk U (lower)
    and the state update (dk x C x dv)."""
    lo, st = C * (C + 1) // 2, C * (C - 1) // 2
    macs = st * dk + lo * dk + C * (C - 1) * (C - 2) // 6 + lo * dk + lo * dv + 3 * C * dk * dv + lo * dv
    return 2.0 * macs * (B * T // C) * H


def traffic_record(kernel):
    """Counter-measured HBM bytes per launch of `kernel`, from the committed
    rocprofv3 summary (profiles/traffic.json), if it was taken on the current
    source of that kernel; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec:
        return None
    with open(os.path.join(ROOT, rec["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec["bytes_per_launch"]


DECODE_N = 256   # sequences in the timed decode batch (H, dk, dv as the workload)


def decode_bytes(N, H, dk, dv):
    return N * H * (2 * dk * dv * 4 + (3 * dk + dv + 1) * 2 + dv * 4)


FWD_GRID = 4 * 32 * 2 * 512   # threads in one launch of the workload's fused forward (one per chain and slice)

KERNELS = {   # traffic.json key -> (substring of the dispatched kernel name, source file, grid size or None)
    "grads": ("kda_bwd_grads_kernel<float, 128, 128>", "gated_delta_rule_41_amd/csrc/kda_bwd.hip", None),
    "scan": ("kda_bwd_scan16_kernel", "gated_delta_rule_41_amd/csrc/kda_scan16.hip", None),
    "fwd": ("kda_fwd16_kernel<float, 128, true, false>", "gated_delta_rule_41_amd/csrc/kda_fwd16.hip", FWD_GRID),
    # the long-context run's second level launches the same kernel on another grid
    "fwd_infer": ("kda_fwd16_kernel<float, 128, false, false>", "gated_delta_rule_41_amd/csrc/kda_fwd16.hip",
                  FWD_GRID),
    "decode": ("kda_decode_kernel", "gated_delta_rule_41_amd/csrc/kda_decode.hip", None),
}


def pmc_summary(fetch_csv, write_csv, probe_mib):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the bench kernels, each
    scaled by the same counter's reading for the copy probe (the run's last
    dispatch), whose true traffic is known: probe_mib MiB read and as many
    written.  Writes profiles/traffic.json (keyed to the kernels' source
    hashes) and prints a markdown summary."""
    import csv
    import hashlib

    def per_dispatch(path, counter):
        sums = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    key = (int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]))
                    sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
        return sums

    probe_bytes = probe_mib * (1 << 20)
    rec, scale = {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        sums = per_dispatch(path, counter)
        last = max(sums)
        scale[counter] = probe_bytes / (sums[last] * 1024.0)
        rec.setdefault("_probe", {"bytes_read": probe_bytes, "bytes_written": probe_bytes})[counter] = {
            "kernel": last[1][:100], "kib": sums[last], "scale": scale[counter]}
        for key, (needle, src, grid) in KERNELS.items():
            vals = [v for (_, name, gs), v in sums.items() if needle in name and (grid is None or gs == grid)]
            if vals:
                rec.setdefault(key, {"kernel": needle, "source": src, "dispatches": len(vals)})[counter + "_kib"] = \
                    sum(vals) / len(vals)
    for key, r in rec.items():
        if key.startswith("_") or "FETCH_SIZE_kib" not in r or "WRITE_SIZE_kib" not in r:
            continue
        r["fetch_bytes"] = r["FETCH_SIZE_kib"] * 1024.0 * scale["FETCH_SIZE"]
        r["write_bytes"] = r["WRITE_SIZE_kib"] * 1024.0 * scale["WRITE_SIZE"]
        r["bytes_per_launch"] = r["fetch_bytes"] + r["write_bytes"]
        with open(os.path.join(ROOT, r["source"]), "rb") as f:
            r["source_sha256"] = hashlib.sha256(f.read()).hexdigest()
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) |")
    print("|---|---|---|---|")
    for key, r in rec.items():
        if "bytes_per_launch" in r:
            print(f"| {r['kernel']} | {r['FETCH_SIZE_kib']:.0f} | {r['WRITE_SIZE_kib']:.0f} | {r['bytes_per_launch']:.4g} |")
    p = rec["_probe"]
    print(f"\ncopy probe ({p['FETCH_SIZE']['kernel']}): {probe_mib} MiB read + written; FETCH_SIZE "
          f"{p['FETCH_SIZE']['kib']:.0f} KiB (scale {p['FETCH_SIZE']['scale']:.4f}), WRITE_SIZE "
          f"{p['WRITE_SIZE']['kib']:.0f} KiB (scale {p['WRITE_SIZE']['scale']:.4f})")


def counter_summary(paths):
    """Per-dispatch averages of every SQ counter in rocprofv3 --pmc CSV files
    for the bench kernels (no GPU work), with the derived busy fractions:
      waves issuing   SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES
      VALU issuing    SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES   (per wave; a SIMD
                      runs two waves of these kernels)
      MFMA busy       SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES)
                      (reading the first as summed over the four SIMDs of a CU)
      LDS conflicts   SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE"""
    import csv
    vals = {}
    for path in paths:
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]), r["Counter_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (_, name, gs, counter), v in per.items():
            for k, (needle, _, grid) in KERNELS.items():
                if needle in name and (grid is None or gs == grid):
                    vals.setdefault(k, {}).setdefault(counter, []).append(v)
    out = {}
    for k, cs in vals.items():
        a = {c: sum(v) / len(v) for c, v in cs.items()}

        def ratio(num, den, mul=1.0):
            return a[num] / (mul * a[den]) if num in a and den in a and a[den] else None
        out[k] = {"counters": a,
                  "waves_issuing": ratio("SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
                  "valu_issuing_per_wave": ratio("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
                  "mfma_busy": ratio("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", 4.0),
                  "lds_conflict_share": ratio("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")}
    print("| kernel | waves issuing | VALU issuing (per wave) | MFMA busy | LDS cycles in bank conflicts |")
    print("|---|---|---|---|---|")
    fmt = lambda x: "-" if x is None else f"{100 * x:.1f}%"   # noqa: E731
    for k, r in out.items():
        print(f"| {KERNELS[k][0]} | {fmt(r['waves_issuing'])} | {fmt(r['valu_issuing_per_wave'])} | "
              f"{fmt(r['mfma_busy'])} | {fmt(r['lds_conflict_share'])} |")
    return out


def cpu_baseline(x, cu, spec, seqs, heads):
    """fp64 oracle, forward + backward, on the first `seqs` sequences and the
    first `heads` heads of the workload (one oracle thread per (sequence, head)
    chain, at most the cores this process may use)."""
    import numpy as np

    import oracle

    T = spec["T"]
    n = seqs * T
    sel = {k: np.ascontiguousarray(x[k][:n, :heads]) for k in ("q", "k", "v", "g", "b", "dO")}
    s0 = np.ascontiguousarray(x["s0"][:seqs, :heads])
    dS = np.ascontiguousarray(x["dS"][:seqs, :heads])
    cu_s = np.asarray(cu[:seqs + 1], dtype=np.int64)
    threads = min(oracle.default_threads(), seqs * heads)
    t0 = time.perf_counter()
    oracle.fwd(sel["q"], sel["k"], sel["v"], sel["g"], sel["b"], cu_seqlens=cu_s, initial_state=s0, threads=threads)
    oracle.bwd(sel["q"], sel["k"], sel["v"], sel["g"], sel["b"], sel["dO"], cu_seqlens=cu_s, initial_state=s0,
               dS_final=dS, threads=threads)
    dt = time.perf_counter() - t0
    full_tokens = n * heads / spec["H"]   # token-heads processed, as whole tokens of the workload
    return {"value": full_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fwd+bwd of sequences 0..{seqs - 1}, heads 0..{heads - 1}, T={T} ({n * heads} token-heads), "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-heads", type=int, default=32, help="heads in the oracle's CPU sample (0: skip)")
    ap.add_argument("--cpu-seqs", type=int, default=4, help="sequences in the oracle's CPU sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed run, one plain device copy of this many MiB (the reference "
                         "kernel that scales rocprofv3's FETCH_SIZE / WRITE_SIZE to bytes)")
    ap.add_argument("--counter-summary", nargs="+", metavar="CSV",
                    help="no GPU work: per-kernel averages and busy fractions of the SQ counters in "
                         "rocprofv3 --pmc counter files of a bench run")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE counter files of "
                         "a run with --copy-probe-mib into profiles/traffic.json and print a summary")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.pmc_summary:
        if args.copy_probe_mib <= 0:
            ap.error("--pmc-summary needs the --copy-probe-mib value of the profiled run")
        pmc_summary(*args.pmc_summary, args.copy_probe_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_delta_rule_41_amd as kda
    import kda_inputs

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda", 0)
    spec, cu, x = kda_inputs.workload(2)
    B, T, H, dk, dv = spec["B"], spec["T"], spec["H"], spec["dk"], spec["dv"]

    def to_dev(a):
        return torch.from_numpy(a).to(dev, torch.bfloat16)

    q, k, v, g, b, dO = (to_dev(x[n]) for n in ("q", "k", "v", "g", "b", "dO"))
    s0 = torch.from_numpy(x["s0"]).to(dev)
    dS = torch.from_numpy(x["dS"]).to(dev)
    cu_t = torch.from_numpy(cu.astype(np.int32)).to(dev)

    def fwd_train():
        return kda.kda_fwd(q, k, v, g, b, cu_t, s0, save_for_bwd=True)

    def bwd(saved, stage="all", out=None):
        return kda.kda_bwd(q, k, v, g, b, saved, dO, cu_t, s0, dS, stage=stage, out=out)

    for _ in range(args.warmup):
        _, _, saved = fwd_train()
        bwd(saved)
    torch.cuda.synchronize()
    _, _, saved = fwd_train()
    out = bwd(saved)          # outputs and workspace, reused by every timed step
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)   # the library launches on this stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_wall0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        _, _, saved = fwd_train()
        ev[i][1].record(stream)
        bwd(saved, "scan", out)
        ev[i][2].record(stream)
        bwd(saved, "grads", out)
        ev[i][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    ms_step = start.elapsed_time(end) / args.steps
    kms = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
           for j, name in enumerate(("fwd", "scan", "grads"))}

    # the same step with o and the gradients written in bf16, the inputs' dtype
    # (what the autograd wrapper returns); state, saves and accumulation stay fp32
    out16 = kda.kda_bwd(q, k, v, g, b, saved, dO, cu_t, s0, dS, out_dtype=torch.bfloat16)
    for _ in range(2):
        _, _, saved16 = kda.kda_fwd(q, k, v, g, b, cu_t, s0, save_for_bwd=True, out_dtype=torch.bfloat16)
        kda.kda_bwd(q, k, v, g, b, saved16, dO, cu_t, s0, dS, out_dtype=torch.bfloat16, out=out16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        _, _, saved16 = kda.kda_fwd(q, k, v, g, b, cu_t, s0, save_for_bwd=True, out_dtype=torch.bfloat16)
        kda.kda_bwd(q, k, v, g, b, saved16, dO, cu_t, s0, dS, out_dtype=torch.bfloat16, out=out16)
    e1.record(stream)
    torch.cuda.synchronize()
    ms16 = e0.elapsed_time(e1) / args.steps
    del out16, saved16

    # the inference forward on its own (no state save): the fused forward kernel alone
    n_inf = max(5, args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        kda.kda_fwd(q, k, v, g, b, cu_t, s0)
    e0.record(stream)
    for _ in range(n_inf):
        kda.kda_fwd(q, k, v, g, b, cu_t, s0)
    e1.record(stream)
    torch.cuda.synchronize()
    inf_ms = e0.elapsed_time(e1) / n_inf

    # attainable HBM bandwidth on this GPU: one plain 1 GiB device copy (read + write)
    cn = (1 << 30) // 4
    csrc = torch.ones(cn, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    for _ in range(2):
        cdst.copy_(csrc)
    e0.record(stream)
    for _ in range(5):
        cdst.copy_(csrc)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * cn * 4 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del csrc, cdst

    # the decode step on its own: one token per sequence, state updated in place
    xd = kda_inputs.generate(1005, DECODE_N, H, dk, dv, "bf16", num_seqs=DECODE_N, with_s0=True)
    dq_, dk_, dv_, dg_, db_ = (to_dev(xd[n]) for n in ("q", "k", "v", "g", "b"))
    sd = torch.from_numpy(xd["s0"]).to(dev)
    del xd
    od = torch.empty((DECODE_N, H, dv), dtype=torch.float32, device=dev)
    kda.kda_decode(dq_, dk_, dv_, dg_, db_, sd, out_state=sd)   # checks shapes once
    # the timed loop calls the C ABI directly with prepared arguments, so host
    # overhead per call stays well under the kernel's duration
    from gated_delta_rule_41_amd import _lib
    dcfg = _lib.make_config(H, dk, dv, kda.KDA_BF16, kda.KDA_F32)
    dargs = (dcfg, DECODE_N) + tuple(int(t.data_ptr()) for t in (dq_, dk_, dv_, dg_, db_, sd, sd, od)) + \
        (stream.cuda_stream,)
    for _ in range(3):
        _lib.check(_lib.kda_decode_raw(*dargs))
    n_dec = max(20, 2 * args.steps)
    e0.record(stream)
    for _ in range(n_dec):
        _lib.kda_decode_raw(*dargs)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / n_dec
    dec_bytes = decode_bytes(DECODE_N, H, dk, dv)
    del sd

    # one long sequence: the two-level forward, and the one-pass forward beside it
    lc_T, lc_H = 1 << 20, 16
    gen = torch.Generator(device=dev).manual_seed(1003)
    lq, lk, lv = (torch.randn(lc_T, lc_H, dk, device=dev, generator=gen).bfloat16() for _ in range(3))
    lg = (-torch.nn.functional.softplus(torch.randn(lc_T, lc_H, dk, device=dev, generator=gen) - 2.0)).bfloat16()
    lb = torch.randn(lc_T, lc_H, device=dev, generator=gen).bfloat16()
    ls0 = 0.1 * torch.randn(1, lc_H, dk, dv, device=dev, generator=gen)
    lc_ms = {}
    for mode in ("split", "one_pass"):
        seq = mode == "one_pass"
        kda.kda_fwd(lq, lk, lv, lg, lb, None, ls0, sequential=seq)
        e0.record(stream)
        for _ in range(3):
            kda.kda_fwd(lq, lk, lv, lg, lb, None, ls0, sequential=seq)
        e1.record(stream)
        torch.cuda.synchronize()
        lc_ms[mode] = e0.elapsed_time(e1) / 3
    lc_bytes = alg_bytes(1, lc_T, lc_H, dk, dv, "fwd")
    del lq, lk, lv, lg, lb, ls0

    tokens = B * T
    names = {"fwd": "kda_fwd16_kernel (training forward, state save)",
             "scan": "kda_bwd_scan16_kernel (reverse state scan)",
             "grads": "kda_bwd_grads_kernel (chunk-parallel gradients)"}
    dom = max(kms, key=kms.get)
    dbytes = alg_bytes(B, T, H, dk, dv, dom)
    ach = dbytes / (kms[dom] * 1e-3) / 1e9
    traffic = traffic_record(dom)
    f_bytes = alg_bytes(B, T, H, dk, dv, "fwd")
    step_bytes = sum(alg_bytes(B, T, H, dk, dv, kname) for kname in kms)
    line = {
        "metric": "KDA fwd+bwd tokens/s (H=32, d=128, T=8192)",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, kda_inputs workload 2)",
        "config": {"workload": spec["name"], "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": 64,
                   "global_batch": B, "seq_len": T, "state": "fp32", "outputs": "fp32"},
        "kernel_ms": kms,
        "bf16_outputs": {"ms_per_step": ms16, "tokens_per_s": tokens / (ms16 * 1e-3),
                         "note": "same step, o and gradients written in bf16"},
        "fwd_infer_ms": inf_ms,
        "fwd_infer_tokens_per_s": tokens / (inf_ms * 1e-3),
        "step_hbm_frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": ach, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": traffic, "alg_bytes_per_launch": dbytes, "ms_per_launch": kms[dom]},
        "roofline_fwd": {"bound": "hbm", "kernel": "kda_fwd16_kernel (inference, no save)",
                         "achieved": f_bytes / (inf_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": f_bytes / (inf_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": traffic_record("fwd_infer"), "alg_bytes_per_launch": f_bytes,
                         "frac_of_copy_bw": f_bytes / (inf_ms * 1e-3) / 1e9 / copy_gbs,
                         "mfma_frac": alg_flops_fwd(B, T, H, dk, dv) / (inf_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "alg_flop_per_launch": alg_flops_fwd(B, T, H, dk, dv)},
        "hbm_copy_gbs": copy_gbs,
        "decode": {"workload": f"decode-bf16-N{DECODE_N}-H{H}-d{dk} (fp32 state in place)",
                   "us_per_step": dec_ms * 1e3, "tokens_per_s": DECODE_N / (dec_ms * 1e-3),
                   "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel", "achieved": dec_bytes / (dec_ms * 1e-3) / 1e9,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                "traffic": traffic_record("decode"), "alg_bytes_per_launch": dec_bytes}},
        "long_context": {"workload": f"kda-fwd-bf16-B1-H{lc_H}-T{lc_T}-d{dk} (inference, two-level)",
                         "ms": lc_ms["split"], "tokens_per_s": lc_T / (lc_ms["split"] * 1e-3),
                         "one_pass_ms": lc_ms["one_pass"],
                         "roofline": {"bound": "hbm", "achieved": lc_bytes / (lc_ms["split"] * 1e-3) / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": lc_bytes / (lc_ms["split"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                      "alg_bytes_per_call": lc_bytes}},
        "timed_wall_s": wall,
    }
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = 2 * n * 4
    if args.cpu_heads > 0:
        line["cpu_baseline"] = cpu_baseline(x, cu, spec, max(1, min(args.cpu_seqs, spec["B"])),
                                            min(args.cpu_heads, spec["H"]))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
