"""Benchmark of the gated delta rule forward pass on one MI355X.

Headline: chunkwise prefill (gdr_chunk_fwd) tokens/s on the Gated DeltaNet
workload B=4, H=16, T=4096, d_k=d_v=128, chunk 64, bf16 q/k/v/o, fp32 gates and
state, seeded synthetic inputs resident in HBM.  One step = one gdr_chunk_fwd
call over the whole batch.  The same line also carries the decode step
(gdr_decode_step, B=256, H=32, d=128, fp32 state) as achieved HBM GB/s.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk-fwd tokens/s + % bf16 MFMA peak; decode-step HBM GB/s % peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def prefill_algorithmic(B, T, H, d, C, io_bytes=2, s0=False):
    """Bytes: q,k,v read and o written once (io dtype), log_alpha and beta (fp32)
    read once, S_T written (and S0 read) once.  FLOPs: 6d^2 + 3Cd + C^2 per
    head-token (the FG2-GDN page's per-head kernel accounting, section 3.6)."""
    ht = B * T * H
    per_ht = 4 * d * io_bytes + 4 + 4
    state = B * H * d * d * 4
    nbytes = ht * per_ht + state * (2 if s0 else 1)
    flops = ht * (6 * d * d + 3 * C * d + C * C)
    return nbytes, flops


def decode_algorithmic(B, H, d, io_bytes=4):
    """State read + written once (fp32), q,k,v read, o written, gates read."""
    bh = B * H
    return bh * (2 * d * d * 4 + 4 * d * io_bytes + 8)


def cpu_baseline(inp, threads):
    import oracle
    t = time.perf_counter()
    oracle.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], None,
                     threads=threads)
    return time.perf_counter() - t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (this path has no multi-GPU part); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_sequence_03_amd import gdr_chunk_fwd, gdr_decode_step, synth
    from linear_attention_sequence_03_amd.gdr import (GDR_BF16, GDR_GATE_SCALAR,
                                                      gdr_chunk_fwd_workspace_size)

    assert torch.cuda.is_available(), "no GPU visible"
    devn = torch.device("cuda:0")
    w = synth.WORKLOADS[1]
    inp = synth.workload_inputs(w)
    B, T, H, d, C = w.B, w.T, w.H, w.d, w.chunk
    bf = torch.bfloat16
    q = torch.from_numpy(inp["q"]).to(devn).to(bf)
    k = torch.from_numpy(inp["k"]).to(devn).to(bf)
    v = torch.from_numpy(inp["v"]).to(devn).to(bf)
    la = torch.from_numpy(inp["log_alpha"]).to(devn)
    be = torch.from_numpy(inp["beta"]).to(devn)
    o = torch.empty((B, T, H, d), dtype=bf, device=devn)
    st = torch.empty((B, H, d, d), dtype=torch.float32, device=devn)
    ws = torch.empty(gdr_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, GDR_GATE_SCALAR),
                     dtype=torch.uint8, device=devn)

    def step():
        gdr_chunk_fwd(q, k, v, la, be, None, chunk=C, o=o, S_T=st, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Whole-job timing: K back-to-back steps bracketed by synchronisation.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-launch duration with HIP events on the launch stream, inputs evicted
    # from the caches between launches by a 512 MiB write (not timed).
    stream = torch.cuda.current_stream(devn)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=devn)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        flush.fill_(1)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    cold = [a.elapsed_time(b) for a, b in ev]
    ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in ev2:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    warm = [a.elapsed_time(b) for a, b in ev2]
    del flush

    nbytes, flops = prefill_algorithmic(B, T, H, d, C)
    launch_ms = float(np.mean(warm))
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    tflops = flops / (launch_ms * 1e-3) / 1e12

    # Decode step, in place on a resident 512 MiB state.
    wd = synth.WORKLOADS[4]
    dinp = synth.workload_inputs(wd)
    dq, dk_, dv_, dla, dbe = (torch.from_numpy(dinp[n]).to(devn)
                              for n in ("q", "k", "v", "log_alpha", "beta"))
    S = torch.from_numpy(dinp["S"]).to(devn)
    do = torch.empty((wd.B, wd.H, wd.d), dtype=torch.float32, device=devn)
    for _ in range(3):
        gdr_decode_step(dq, dk_, dv_, dla, dbe, S, o=do, inplace=True)
    torch.cuda.synchronize()
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.decode_steps)]
    for a, b in dev_ev:
        a.record(stream)
        gdr_decode_step(dq, dk_, dv_, dla, dbe, S, o=do, inplace=True)
        b.record(stream)
    torch.cuda.synchronize()
    dms = float(np.mean([a.elapsed_time(b) for a, b in dev_ev]))
    dbytes = decode_algorithmic(wd.B, wd.H, wd.d)
    dgbs = dbytes / (dms * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": B * T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k unit-norm N(0,1), v N(0,1), beta sigmoid(N(0,1)), "
                "log_alpha U(-0.1,-0.001))",
        "config": {"workload": w.name, "call": "gdr_chunk_fwd", "gate": "scalar",
                   "B": B, "T": T, "H": H, "d_k": d, "d_v": d, "chunk": C,
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "gdr_chunk_fwd (wy_prep + state_pass)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes,
                     "launch_ms_mean": launch_ms,
                     "launch_ms_cold_cache_mean": float(np.mean(cold))},
        "prefill_mfma": {"algorithmic_flops_per_launch": flops, "tflops": tflops,
                         "peak_tflops": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS},
        "decode": {"workload": wd.name, "call": "gdr_decode_step", "ms_per_step": dms,
                   "tokens_per_s": wd.B / (dms * 1e-3),
                   "algorithmic_bytes": dbytes, "achieved_GBs": dgbs,
                   "peak_GBs": HBM_PEAK_GBS, "frac": dgbs / HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        import oracle.gdr_oracle as og
        threads = min(16, og.default_threads())
        secs = cpu_baseline(inp, threads)
        out["cpu_baseline"] = {"value": B * T / secs, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "the whole prefill workload (B=4,T=4096,H=16,d=128) "
                                         "in the fp64 token-by-token oracle, %.1f s" % secs}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
