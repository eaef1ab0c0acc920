"""Benchmark of the gated delta rule forward pass on one MI355X.

Headline: chunkwise prefill (gdr_chunk_fwd) tokens/s on the largest prefill
workload that fits one GPU, the long-context Gated DeltaNet call B=1, H=32,
T=32768, d_k=d_v=128, chunk 64, bf16 q/k/v/o, fp32 gates, an fp32 start state
S0 and the final state S_T; seeded synthetic inputs resident in HBM.  One step
= one gdr_chunk_fwd call over the whole batch.  The same line carries the
other two prefill workloads (B=4,H=16,T=4096 scalar gate; B=2,H=32,T=8192
channel gate), the decode step (gdr_decode_step, B=256, H=32, d=128, fp32
state) as achieved HBM GB/s, and the CPU oracle's throughput.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
    python bench.py --workload 1     # another prefill workload as the headline
                                     # (1: GDN B=4,H=16,T=4096; 2: KDA B=2,H=32,T=8192)
    python bench.py --workload 2 --fg2   # channel-wise write rates (FG2-GDN+) on that
                                         # shape, with the overhead over the KDA call
    python bench.py --workload 2 --gdn2  # decoupled erase / write gates (Gated
                                         # DeltaNet-2, chunkwise) on that shape, with
                                         # the token-sequential scan beside it
    python bench.py --prologue           # raw q, k and beta logits: the gate prologue
                                         # fused into the kernels, against torch
                                         # normalising first
    python bench.py --traffic [--workload N]  # HBM bytes per call (rocprofv3 counters);
                                              # N = 4 is the decode step
    python bench.py --mfma [--workload N]     # issued MFMA FLOPs and MFMA-busy % per call
    python bench.py --sweep          # every chunkwise call over 2k x 16 ... 32k x 1 (H=32)

Prints ONE JSON line.  Only one GPU is used; --gpus above 1 exits.

Timing: `value` is whole-job tokens/s over K back-to-back calls bracketed by
synchronisation.  `roofline` uses the median duration of K launches timed
with HIP events on the launch stream, each launch after a 512 MiB write that
evicts the inputs from the caches (the warm median is reported beside it).
`roofline.traffic` is the HBM bytes one call moves, from two rocprofv3 --pmc
passes (FETCH_SIZE, then WRITE_SIZE) over the call's kernels, each scaled by
what the same counter reads for a plain 256 MiB device copy (libgdr_calib.so:
16-byte loads and stores); it is reported only while the summary in profiles/
was taken from the current kernel sources (hash match), else null.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk-fwd tokens/s + % bf16 MFMA peak; decode-step HBM GB/s % peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def prefill_algorithmic(B, T, H, d, C, io_bytes=2, s0=False, channel=False, fg2=False):
    """Bytes: q,k,v read and o written once (io dtype), log_alpha (fp32, one per
    head-token, or d_k of them for the channel gate) and beta (fp32) read once,
    S_T written (and S0 read) once.  With ``fg2`` the scalar beta is replaced by
    two fp32 d-vectors per head-token (FG2's key and value rates, or Gated
    DeltaNet-2's erase and write gates).  FLOPs: 6d^2 + 3Cd + C^2 per head-token
    (the FG2-GDN page's per-head kernel accounting, section 3.6)."""
    ht = B * T * H
    per_ht = 4 * d * io_bytes + (4 * d if channel else 4) + (2 * 4 * d if fg2 else 4)
    state = B * H * d * d * 4
    nbytes = ht * per_ht + state * (2 if s0 else 1)
    flops = ht * (6 * d * d + 3 * C * d + C * C)
    return nbytes, flops


def decode_algorithmic(B, H, d, io_bytes=4):
    """State read + written once (fp32), q,k,v read, o written, gates read."""
    bh = B * H
    return bh * (2 * d * d * 4 + 4 * d * io_bytes + 8)


COPY_BYTES = 256 << 20
PREFILL_KERNELS = ("fused_chunk", "wy_prep", "state_pass")
DECODE_KERNELS = ("decode_kernel",)
# rocprofv3 derived counters: issued MFMA FLOPs by operand type (MOPS x 512) and
# the MFMA-busy share of the SIMDs over the dispatch
MFMA_COUNTERS = ("MfmaFlopsBF16", "MfmaFlopsF16", "MfmaUtil")
HEADLINE = 3
ROOFLINE_KERNEL = {
    1: "gdr_chunk_fwd (single kernel: fused_chunk<128, 2>)",
    2: "gdr_chunk_fwd (wy_prep_channel_bf16<128, 64> + state_pass<bf16, 128, 64, 2, channel>)",
    3: "gdr_chunk_fwd (single kernel: fused_chunk<128, 1>)",
}
PROFILE_STEM = {
    1: "gdr_chunk_fwd_gdn_B4_H16_T4096_d128",
    2: "gdr_chunk_fwd_kda_B2_H32_T8192_d128",
    3: "gdr_chunk_fwd_gdn_s0_B1_H32_T32768_d128",
    4: "gdr_decode_step_B256_H32_d128",
}


def profile_file(workload, kind):
    """profiles/<call and workload>.<kind>.txt (kind: traffic or mfma)."""
    return os.path.join(ROOT, "profiles", "%s.%s.txt" % (PROFILE_STEM[workload], kind))


def read_summary(workload, kind):
    """The key=value lines of a counter summary, or None when it is absent or
    was taken from other kernel sources."""
    path = profile_file(workload, kind)
    if not os.path.exists(path):
        return None
    kv = dict(l.strip().split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))
    return kv if kv.get("source_hash") == kernel_source_hash(workload) else None


# The sources that build the kernels each workload's summary measures (plus the
# calibration copy): a summary counts only while these are unchanged.
KERNEL_SOURCES = {
    1: ("gdr_fused.hip",), 3: ("gdr_fused.hip",), 2: ("gdr_chunk.hip",), 4: ("gdr_decode.hip",),
}


def kernel_source_hash(workload):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_03_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[workload] + ("gdr_device.hpp", "gdr_launch.hpp", "gdr_calib.hip")):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(inp, threads, min_seconds=10.0, max_reps=40, S0=None):
    """The oracle over the whole workload, repeated until ~min_seconds."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], S0,
                         threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    return reps, time.perf_counter() - t0


def host_threads():
    """Host threads for the CPU baseline: the cores this process may run on,
    limited to the per-GPU share the host sets in OMP_NUM_THREADS when it does."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def traffic_probe(workload):
    """Program run under rocprofv3 --pmc: 3 calls of the workload (a prefill
    call, or for workload 4 a decode step), then 3 plain copies."""
    import ctypes
    import torch
    from linear_attention_sequence_03_amd import gdr_chunk_fwd, gdr_decode_step, synth
    w = synth.WORKLOADS[workload]
    inp = synth.workload_inputs(w)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(a).to(dev) for n, a in inp.items() if a is not None}
    if w.io == "bf16":
        for n in ("q", "k", "v"):
            t[n] = t[n].to(torch.bfloat16)
    for _ in range(3):
        if w.call == "chunk":
            gdr_chunk_fwd(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t.get("S0"), chunk=w.chunk)
        else:
            gdr_decode_step(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], t["S"], inplace=True)
    calib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_sequence_03_amd", "libgdr_calib.so"))
    calib.gdr_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for _ in range(3):
        assert calib.gdr_calib_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, stream) == 0
    torch.cuda.synchronize()


def copy_ceiling():
    """A plain 16-byte device copy (libgdr_calib.so) and torch's copy at a few
    sizes: bytes read + written per second, the practical ceiling for a
    read-modify-write stream such as the decode step."""
    import ctypes
    import torch
    dev = torch.device("cuda:0")
    calib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_sequence_03_amd", "libgdr_calib.so"))
    calib.gdr_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]
    res = {}
    for mib in (256, 512, 1024):
        n = mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        for name, fn in (("calib", lambda: calib.gdr_calib_copy(src.data_ptr(), dst.data_ptr(), n,
                                                                  stream)),
                         ("torch", lambda: dst.copy_(src))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(10)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            t = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
            res["%s_%dMiB_TBs" % (name, mib)] = 2 * n / t / 1e12
        del src, dst
    print(json.dumps(res))


def _pmc_rows(outdir, counters, workload):
    d = tempfile.mkdtemp(prefix="pmc_", dir=outdir)
    cmd = (["rocprofv3", "--pmc"] + list(counters) + ["--output-format", "csv", "-d", d, "-o", "run",
                                                      "--", sys.executable, os.path.abspath(__file__),
                                                      "--traffic-probe", "--workload", str(workload)])
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL, timeout=240)
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def measure_traffic(outdir, workload):
    """Two rocprofv3 --pmc passes over traffic_probe(); returns bytes per call."""
    kernels = DECODE_KERNELS if workload == 4 else PREFILL_KERNELS
    res = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        per = {}
        for r in _pmc_rows(outdir, [ctr], workload):
            name = r["Kernel_Name"]
            key = next((k for k in kernels if k in name), None)
            if key is None and "gdr_calib_copy_kernel" in name:
                key = "copy"
            if key:
                per.setdefault(key, []).append(float(r["Counter_Value"]))
        kib_copy = sum(per["copy"]) / len(per["copy"])
        factor = (COPY_BYTES / 1024.0) / kib_copy
        kib_call = sum(sum(per[k]) / len(per[k]) for k in kernels if k in per)
        res.setdefault("kernels", sorted(k for k in kernels if k in per))
        res[ctr] = dict(kib_per_call=kib_call, copy_kib=kib_copy, factor=factor,
                        bytes_per_call=kib_call * factor * 1024.0)
    return res


def measure_mfma(outdir, workload):
    """One rocprofv3 --pmc pass (MFMA counters) over traffic_probe(); returns the
    per-call sum over the prefill kernels of each counter's per-dispatch mean
    (MfmaUtil: the mean over every prefill dispatch)."""
    per = {}
    for r in _pmc_rows(outdir, MFMA_COUNTERS, workload):
        key = next((k for k in PREFILL_KERNELS if k in r["Kernel_Name"]), None)
        if key:
            d = per.setdefault(r["Counter_Name"], {}).setdefault(key, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    out = {}
    for c, by_kernel in per.items():
        if c == "MfmaUtil":
            out[c] = float(np.mean([v for d in by_kernel.values() for v in d.values()]))
        else:
            out[c] = float(sum(np.mean(list(d.values())) for d in by_kernel.values()))
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


# The pages' prefill sweep ("FG2-GDN" page, section 4.5, Figure 3): one batch of
# 32k tokens split as 2k x 16 ... 32k x 1, here at H = 32 heads, d = 128.
SWEEP = ((16, 2048), (8, 4096), (4, 8192), (2, 16384), (1, 32768))


def run_sweep(steps: int, warmup: int):
    """Prefill tokens/s of every chunkwise call over the pages' B x T sweep.
    One set of seeded inputs [1, 32768, 32, 128] serves every split (a view)."""
    import torch
    from linear_attention_sequence_03_amd import (gdr_chunk_fwd, gdr_fg2_chunk_fwd, gdr_gdn2_chunk_fwd,
                                                  synth)
    from linear_attention_sequence_03_amd.gdr import (GDR_BF16, GDR_GATE_CHANNEL, GDR_GATE_SCALAR,
                                                      gdr_chunk_fwd_workspace_size,
                                                      gdr_fg2_chunk_fwd_workspace_size,
                                                      gdr_gdn2_chunk_fwd_workspace_size)
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    H, d, C, N = 32, 128, 64, 32768
    seed = 1100
    inp = synth.chunk_inputs(1, N, H, d, d, "channel", "bf16", seed=seed)
    bk, bv = synth.write_rates((1, N, H, d), d, seed=seed)
    eb, ww = synth.gdn2_gates(1, N, H, d, d, seed=seed)
    bf = torch.bfloat16
    t = lambda a, dt=None: (torch.from_numpy(a).to(dev) if dt is None  # noqa: E731
                            else torch.from_numpy(a).to(dev).to(dt))
    q, k, v = t(inp["q"], bf), t(inp["k"], bf), t(inp["v"], bf)
    la_c = t(inp["log_alpha"])
    la_s = la_c[..., 0].contiguous()
    be, bk, bv, eb, ww = t(inp["beta"]), t(bk), t(bv), t(eb), t(ww)
    del inp
    o = torch.empty((1, N, H, d), dtype=bf, device=dev)
    st = torch.empty((16, H, d, d), dtype=torch.float32, device=dev)
    nws = max(gdr_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, g) for B, T in SWEEP
              for g in (GDR_GATE_SCALAR, GDR_GATE_CHANNEL))
    nws = max([nws] + [gdr_fg2_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, GDR_GATE_CHANNEL)
                       for B, T in SWEEP]
              + [gdr_gdn2_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, GDR_GATE_CHANNEL)
                 for B, T in SWEEP])
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def shaped(x, B, T):
        return x.view((B, T) + tuple(x.shape[2:]))

    calls = {
        "gdn": lambda B, T: gdr_chunk_fwd(
            shaped(q, B, T), shaped(k, B, T), shaped(v, B, T), shaped(la_s, B, T), shaped(be, B, T),
            None, chunk=C, o=shaped(o, B, T), S_T=st[:B], workspace=ws),
        "kda": lambda B, T: gdr_chunk_fwd(
            shaped(q, B, T), shaped(k, B, T), shaped(v, B, T), shaped(la_c, B, T), shaped(be, B, T),
            None, chunk=C, o=shaped(o, B, T), S_T=st[:B], workspace=ws),
        "fg2_gdn": lambda B, T: gdr_fg2_chunk_fwd(
            shaped(q, B, T), shaped(k, B, T), shaped(v, B, T), shaped(la_c, B, T), shaped(bk, B, T),
            None, None, chunk=C, o=shaped(o, B, T), S_T=st[:B], workspace=ws),
        "fg2_gdn_plus": lambda B, T: gdr_fg2_chunk_fwd(
            shaped(q, B, T), shaped(k, B, T), shaped(v, B, T), shaped(la_c, B, T), shaped(bk, B, T),
            shaped(bv, B, T), None, chunk=C, o=shaped(o, B, T), S_T=st[:B], workspace=ws),
        "gdn2": lambda B, T: gdr_gdn2_chunk_fwd(
            shaped(q, B, T), shaped(k, B, T), shaped(v, B, T), shaped(la_c, B, T), shaped(eb, B, T),
            shaped(ww, B, T), None, chunk=C, o=shaped(o, B, T), S_T=st[:B], workspace=ws),
    }
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, fn in calls.items():
        res[name] = {}
        for B, T in SWEEP:
            for _ in range(warmup):
                fn(B, T)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for a, b in ev:
                a.record(stream)
                fn(B, T)
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            res[name]["%dkx%d" % (T // 1024, B)] = {"ms": ms, "tokens_per_s": B * T / (ms * 1e-3)}
        print("sweep %s done" % name, file=sys.stderr, flush=True)
    first, last = "%dkx%d" % (SWEEP[0][1] // 1024, SWEEP[0][0]), "%dkx%d" % (SWEEP[-1][1] // 1024, SWEEP[-1][0])
    out = {
        "metric": "prefill tokens/s over the B x T sweep (32k tokens per call)",
        "unit": "tokens/s", "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded)",
        "config": {"H": H, "d_k": d, "d_v": d, "chunk": C, "splits": [list(x) for x in SWEEP]},
        "results": res,
        "ratio_last_over_first": {n: res[n][last]["tokens_per_s"] / res[n][first]["tokens_per_s"]
                                  for n in res},
        "overhead_vs_kda": {n: {c: res[n][c]["ms"] / res["kda"][c]["ms"] - 1.0 for c in res[n]}
                            for n in ("fg2_gdn", "fg2_gdn_plus", "gdn2")},
    }
    print(json.dumps(out))


def prefill_tensors(w, devn):
    """A prefill workload's seeded inputs on the device, outputs and workspace."""
    import torch
    from linear_attention_sequence_03_amd import synth
    from linear_attention_sequence_03_amd.gdr import (GDR_BF16, GDR_GATE_CHANNEL, GDR_GATE_SCALAR,
                                                      gdr_chunk_fwd_workspace_size)
    inp = synth.workload_inputs(w)
    B, T, H, d, C = w.B, w.T, w.H, w.d, w.chunk
    bf = torch.bfloat16
    t = {n: torch.from_numpy(inp[n]).to(devn) for n in ("log_alpha", "beta")}
    for n in ("q", "k", "v"):
        t[n] = torch.from_numpy(inp[n]).to(devn).to(bf)
    t["S0"] = torch.from_numpy(inp["S0"]).to(devn) if inp.get("S0") is not None else None
    t["o"] = torch.empty((B, T, H, d), dtype=bf, device=devn)
    t["S_T"] = torch.empty((B, H, d, d), dtype=torch.float32, device=devn)
    channel = inp["log_alpha"].ndim == 4
    gate = GDR_GATE_CHANNEL if channel else GDR_GATE_SCALAR
    t["ws"] = torch.empty(gdr_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, gate),
                          dtype=torch.uint8, device=devn)
    return inp, t, channel, gate


def event_times(step, n, stream, flush=None):
    """Durations (ms) of n launches of step(), HIP events on the launch stream;
    with ``flush``, a 512 MiB write (not timed) evicts the caches before each."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        if flush is not None:
            flush.fill_(1)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def roofline_entry(nbytes, cold, warm, traffic, kernel):
    med = float(np.median(cold))
    achieved = nbytes / (med * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
            "launch_ms_cold_median": med, "launch_ms_cold_min": float(np.min(cold)),
            "launch_ms_cold_mean": float(np.mean(cold)), "launch_ms_warm_median": float(np.median(warm)),
            "timing": "median of %d launches, each after a 512 MiB cache-evicting write; HIP events "
                      "on the launch stream" % len(cold)}


def traffic_of(workload):
    kv = read_summary(workload, "traffic")
    return float(kv["traffic_bytes_per_call"]) if kv else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--workload", type=int, default=HEADLINE, choices=(1, 2, 3, 4),
                    help="prefill workload of the line (3, the largest, is the headline); "
                         "with --traffic / --mfma, 4 selects the decode step")
    ap.add_argument("--fg2", action="store_true",
                    help="time gdr_fg2_chunk_fwd with key and value rates (FG2-GDN+) instead")
    ap.add_argument("--gdn2", action="store_true",
                    help="time gdr_gdn2_chunk_fwd (decoupled erase / write gates) instead, "
                         "with gdr_gdn2_fwd (the scan) beside it")
    ap.add_argument("--prologue", action="store_true",
                    help="raw q, k and beta logits: time the fused gate prologue instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other prefill workloads in the line")
    ap.add_argument("--sweep", action="store_true",
                    help="prefill tokens/s of every chunkwise call over the B x T sweep 2k x 16 ... "
                         "32k x 1 (H=32, d=128), one JSON line of its own")
    ap.add_argument("--traffic", action="store_true",
                    help="measure HBM bytes per call with rocprofv3 and write a summary")
    ap.add_argument("--traffic-probe", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--mfma", action="store_true",
                    help="issued MFMA FLOPs and MFMA-busy share of one prefill call from rocprofv3 "
                         "counters; writes a summary")
    ap.add_argument("--copy", action="store_true",
                    help="time a plain device copy (the practical HBM read+write ceiling)")
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out"))
    args = ap.parse_args()
    if args.sweep:
        run_sweep(args.steps, args.warmup)
        return
    if args.traffic_probe:
        traffic_probe(args.workload)
        return
    if args.copy:
        copy_ceiling()
        return
    from linear_attention_sequence_03_amd import synth
    wname = synth.WORKLOADS[args.workload].name
    if args.traffic:
        os.makedirs(args.out, exist_ok=True)
        res = measure_traffic(args.out, args.workload)
        total = res["FETCH_SIZE"]["bytes_per_call"] + res["WRITE_SIZE"]["bytes_per_call"]
        path = os.path.join(args.out, os.path.basename(profile_file(args.workload, "traffic")))
        with open(path, "w") as fh:
            fh.write("# HBM traffic of one %s call, workload %s\n"
                     % ("gdr_decode_step" if args.workload == 4 else "gdr_chunk_fwd", wname))
            fh.write("# command: python bench.py --traffic --workload %d   (rocprofv3 --pmc FETCH_SIZE, "
                     "then WRITE_SIZE, over 3 calls and 3 plain copies)\n" % args.workload)
            fh.write("# kernels: %s; calibration: plain %d MiB device copy (libgdr_calib.so)\n"
                     % (", ".join(res.get("kernels", ())), COPY_BYTES >> 20))
            fh.write("source_hash=%s\n" % kernel_source_hash(args.workload))
            for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
                r = res[ctr]
                fh.write("%s_kib_per_call=%.1f\n%s_copy_kib=%.1f\n%s_factor=%.4f\n"
                         % (ctr, r["kib_per_call"], ctr, r["copy_kib"], ctr, r["factor"]))
            fh.write("traffic_bytes_per_call=%.0f\n" % total)
        print(json.dumps({"traffic_bytes_per_call": total, "summary": path, **res}))
        return
    if args.mfma:
        os.makedirs(args.out, exist_ok=True)
        res = measure_mfma(args.out, args.workload)
        path = os.path.join(args.out, os.path.basename(profile_file(args.workload, "mfma")))
        with open(path, "w") as fh:
            fh.write("# Issued MFMA work of one gdr_chunk_fwd call, workload %s\n" % wname)
            fh.write("# command: python bench.py --mfma --workload %d   (rocprofv3 --pmc %s)\n"
                     % (args.workload, " ".join(MFMA_COUNTERS)))
            fh.write("# kernels: %s; per-dispatch means over the probe's calls, summed over the "
                     "call's kernels (MfmaUtil: mean over its dispatches)\n" % ", ".join(PREFILL_KERNELS))
            fh.write("source_hash=%s\n" % kernel_source_hash(args.workload))
            for c, v in res.items():
                fh.write("%s=%.6g\n" % (c, v))
        print(json.dumps({"summary": path, **res}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (this path has no multi-GPU part); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.workload == 4:
        print("--workload 4 (the decode step) is part of every line; pick a prefill workload",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_sequence_03_amd import (gdr_chunk_fwd, gdr_decode_step, gdr_fg2_chunk_fwd,
                                                  gdr_gdn2_fwd)
    from linear_attention_sequence_03_amd.gdr import GDR_BF16, gdr_fg2_chunk_fwd_workspace_size

    assert torch.cuda.is_available(), "no GPU visible"
    devn = torch.device("cuda:0")
    stream = torch.cuda.current_stream(devn)
    w = synth.WORKLOADS[args.workload]
    B, T, H, d, C = w.B, w.T, w.H, w.d, w.chunk
    inp, t, channel, gate = prefill_tensors(w, devn)
    q, k, v, la, be, S0, o, st, ws = (t[n] for n in ("q", "k", "v", "log_alpha", "beta", "S0", "o",
                                                      "S_T", "ws"))
    bf = torch.bfloat16

    def plain_step():
        gdr_chunk_fwd(q, k, v, la, be, S0, chunk=C, o=o, S_T=st, workspace=ws)

    step = plain_step
    if args.fg2:
        bk, bv = synth.write_rates((B, T, H, d), d, seed=w.seed)
        bk, bv = torch.from_numpy(bk).to(devn), torch.from_numpy(bv).to(devn)
        ws2 = torch.empty(gdr_fg2_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, gate),
                          dtype=torch.uint8, device=devn)

        def step():
            gdr_fg2_chunk_fwd(q, k, v, la, bk, bv, S0, chunk=C, o=o, S_T=st, workspace=ws2)
    elif args.prologue:
        from linear_attention_sequence_03_amd.gdr import (GDR_PROLOGUE_BETA_SIGMOID,
                                                          GDR_PROLOGUE_L2NORM_QK)
        rin = synth.raw_prologue_inputs(inp, "bf16", seed=w.seed)
        rq = torch.from_numpy(rin["q"]).to(devn).to(bf)
        rk = torch.from_numpy(rin["k"]).to(devn).to(bf)
        rbe = torch.from_numpy(rin["beta"]).to(devn)
        flags = GDR_PROLOGUE_L2NORM_QK | GDR_PROLOGUE_BETA_SIGMOID

        def step():
            gdr_chunk_fwd(rq, rk, v, la, rbe, S0, chunk=C, o=o, S_T=st, workspace=ws, prologue=flags)

        def torch_then_plain():
            # the same result with the prologue done by torch before the call
            qn = (rq.float() * torch.rsqrt((rq.float() ** 2).sum(-1, keepdim=True) + 1e-6)).to(bf)
            kn = (rk.float() * torch.rsqrt((rk.float() ** 2).sum(-1, keepdim=True) + 1e-6)).to(bf)
            gdr_chunk_fwd(qn, kn, v, la, torch.sigmoid(rbe), S0, chunk=C, o=o, S_T=st, workspace=ws)
    elif args.gdn2:
        from linear_attention_sequence_03_amd import (gdr_gdn2_chunk_fwd,
                                                      gdr_gdn2_chunk_fwd_workspace_size)
        eb, ww = synth.gdn2_gates(B, T, H, d, d, seed=w.seed)
        eb, ww = torch.from_numpy(eb).to(devn), torch.from_numpy(ww).to(devn)
        ws3 = torch.empty(gdr_gdn2_chunk_fwd_workspace_size(B, T, H, d, d, C, GDR_BF16, gate),
                          dtype=torch.uint8, device=devn)

        def step():
            gdr_gdn2_chunk_fwd(q, k, v, la, eb, ww, S0, chunk=C, o=o, S_T=st, workspace=ws3)

        def scan_step():
            gdr_gdn2_fwd(q, k, v, la, eb, ww, S0, o=o, S_T=st)

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
    print("headline workload timed: %.4f ms per call" % ms_per_step, file=sys.stderr, flush=True)

    # Per-launch durations: cold (caches evicted before each launch) and warm.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=devn)
    cold = event_times(step, args.steps, stream, flush)
    warm = event_times(step, args.steps, stream)

    variant = args.fg2 or args.gdn2 or args.prologue
    nbytes, flops = prefill_algorithmic(B, T, H, d, C, s0=S0 is not None, channel=channel,
                                        fg2=args.fg2 or args.gdn2)
    launch_ms = float(np.median(cold))
    has_s0 = S0 is not None
    extra_info = {}
    if args.prologue:
        for _ in range(3):
            torch_then_plain()
        tms = float(np.median(event_times(torch_then_plain, args.steps, stream, flush)))
        extra_info["prologue"] = {
            "call": "gdr_chunk_fwd_prologue (L2 norm of q, k + sigmoid of beta, fused)",
            "launch_ms_cold_median": launch_ms,
            "unfused_call": "torch normalisation + sigmoid, then gdr_chunk_fwd",
            "unfused_ms_cold_median": tms, "speedup": tms / launch_ms}
    if args.fg2:
        for _ in range(3):
            plain_step()
        base_ms = float(np.median(event_times(plain_step, args.steps, stream, flush)))
        base_bytes, _ = prefill_algorithmic(B, T, H, d, C, s0=S0 is not None, channel=channel)
        extra_info["fg2"] = {
            "call": "gdr_fg2_chunk_fwd (key and value rates: FG2-GDN+)",
            "launch_ms_cold_median": launch_ms, "base_call": "gdr_chunk_fwd (scalar rate)",
            "base_launch_ms_cold_median": base_ms, "overhead": launch_ms / base_ms - 1.0,
            "algorithmic_bytes": nbytes, "base_algorithmic_bytes": base_bytes,
            "bytes_overhead": nbytes / base_bytes - 1.0}
    if args.gdn2:
        scan_step()
        sms = float(np.median(event_times(scan_step, min(args.steps, 5), stream, flush)))
        extra_info["gdn2"] = {"call": "gdr_gdn2_chunk_fwd (gdn2_prep + gdn2_state_pass)",
                              "launch_ms_cold_median": launch_ms,
                              "scan_call": "gdr_gdn2_fwd (gdn2_scan, token-sequential)",
                              "scan_launch_ms_cold_median": sms, "speedup": sms / launch_ms}
    traffic = None if variant else traffic_of(args.workload)
    kernel = ("gdr_gdn2_chunk_fwd (gdn2_prep<128, channel> + gdn2_state_pass<128, 2>)" if args.gdn2 else
              ("gdr_fg2_chunk_fwd (fg2_scale prologue + " if args.fg2 else "")
              + ROOFLINE_KERNEL[args.workload] + (")" if args.fg2 else ""))
    roofline = roofline_entry(nbytes, cold, warm, traffic, kernel)
    tflops = flops / (launch_ms * 1e-3) / 1e12
    issued = {}
    kv = None if variant else read_summary(args.workload, "mfma")
    if kv:
        iflops = float(kv.get("MfmaFlopsBF16", 0.0)) + float(kv.get("MfmaFlopsF16", 0.0))
        issued = {"issued_flops_per_launch": iflops,
                  "issued_tflops": iflops / (launch_ms * 1e-3) / 1e12,
                  "issued_frac": iflops / (launch_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                  "mfma_busy_pct": float(kv["MfmaUtil"]) if "MfmaUtil" in kv else None}

    # The other prefill workloads, timed the same way (one entry each).
    others = {}
    if not (variant or args.no_extra):
        del q, k, v, la, be, S0, o, st, ws, t
        torch.cuda.empty_cache()
        for wi in (1, 2, 3):
            if wi == args.workload:
                continue
            w2 = synth.WORKLOADS[wi]
            _, t2, ch2, _ = prefill_tensors(w2, devn)

            def step2(t2=t2, w2=w2):
                gdr_chunk_fwd(t2["q"], t2["k"], t2["v"], t2["log_alpha"], t2["beta"], t2["S0"],
                              chunk=w2.chunk, o=t2["o"], S_T=t2["S_T"], workspace=t2["ws"])

            for _ in range(args.warmup):
                step2()
            c2 = event_times(step2, args.steps, stream, flush)
            w2t = event_times(step2, args.steps, stream)
            nb2, fl2 = prefill_algorithmic(w2.B, w2.T, w2.H, w2.d, w2.chunk, s0=t2["S0"] is not None,
                                           channel=ch2)
            r2 = roofline_entry(nb2, c2, w2t, traffic_of(wi), ROOFLINE_KERNEL[wi])
            m2 = r2["launch_ms_cold_median"]
            others[w2.name] = {"tokens_per_s": w2.B * w2.T / (m2 * 1e-3), "roofline": r2,
                               "algorithmic_tflops": fl2 / (m2 * 1e-3) / 1e12,
                               "algorithmic_mfma_frac": fl2 / (m2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
            del t2
            torch.cuda.empty_cache()
            print("workload %d timed: %.4f ms per call" % (wi, m2), file=sys.stderr, flush=True)
    del flush
    torch.cuda.empty_cache()

    # Decode step, in place on a resident 512 MiB state.
    wd = synth.WORKLOADS[4]
    dinp = synth.workload_inputs(wd)
    dq, dk_, dv_, dla, dbe = (torch.from_numpy(dinp[n]).to(devn)
                              for n in ("q", "k", "v", "log_alpha", "beta"))
    S = torch.from_numpy(dinp["S"]).to(devn)
    do = torch.empty((wd.B, wd.H, wd.d), dtype=torch.float32, device=devn)

    def dstep():
        gdr_decode_step(dq, dk_, dv_, dla, dbe, S, o=do, inplace=True)

    for _ in range(3):
        dstep()
    torch.cuda.synchronize()
    dtimes = event_times(dstep, args.decode_steps, stream)
    dms = float(np.median(dtimes))
    dbytes = decode_algorithmic(wd.B, wd.H, wd.d)
    dgbs = dbytes / (dms * 1e-3) / 1e9

    # Several tokens per sequence on the same resident state (speculative
    # decoding): a read-only pass scoring Td draft tokens, then the commit of
    # the accepted prefixes in place.
    from linear_attention_sequence_03_amd import gdr_decode_multi
    Td = 4
    mi = synth.chunk_inputs(wd.B, Td, wd.H, wd.d, wd.d, "scalar", "f32", seed=wd.seed + 1)
    mq, mk, mv, mla, mbe = (torch.from_numpy(mi[n]).to(devn)
                            for n in ("q", "k", "v", "log_alpha", "beta"))
    macc = torch.from_numpy(np.random.Generator(np.random.PCG64(wd.seed)).integers(
        0, Td + 1, wd.B).astype(np.int32)).to(devn)
    mo = torch.empty((wd.B, Td, wd.H, wd.d), dtype=torch.float32, device=devn)

    def verify():
        gdr_decode_multi(mq, mk, mv, mla, mbe, S, o=mo)

    def commit():
        gdr_decode_multi(mq, mk, mv, mla, mbe, S, accepted=macc, want_o=False, inplace=True)

    mres = {}
    for name, fn in (("verify", verify), ("commit", commit)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        mres[name] = float(np.median(event_times(fn, args.decode_steps, stream)))
    # A draft tree per sequence on the same state: 16 nodes (a random tree),
    # every node verified in one pass, then the accepted node's state rebuilt
    # in place from the written values.
    from linear_attention_sequence_03_amd import gdr_decode_tree, gdr_decode_tree_commit
    Tt = 16
    ti = synth.chunk_inputs(wd.B, Tt, wd.H, wd.d, wd.d, "scalar", "f32", seed=wd.seed + 2)
    tq, tk, tv, tla, tbe = (torch.from_numpy(ti[n]).to(devn) for n in ("q", "k", "v", "log_alpha", "beta"))
    tpar = torch.from_numpy(synth.draft_tree("random", wd.B, Tt, seed=wd.seed)).to(devn)
    tacc = torch.from_numpy(np.random.Generator(np.random.PCG64(wd.seed + 1)).integers(
        -1, Tt, wd.B).astype(np.int32)).to(devn)
    to_ = torch.empty((wd.B, Tt, wd.H, wd.d), dtype=torch.float32, device=devn)
    tD = torch.empty_like(to_)

    def tverify():
        gdr_decode_tree(tq, tk, tv, tla, tbe, S, tpar, o=to_, D=tD)

    def tcommit():
        gdr_decode_tree_commit(tk, tla, tpar, tD, tacc, S, inplace=True)

    for name, fn in (("tree_verify", tverify), ("tree_commit", tcommit)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        mres[name] = float(np.median(event_times(fn, args.decode_steps, stream)))
    state_bytes = wd.B * wd.H * wd.d * wd.d * 4
    vec_bytes = wd.B * Td * wd.H * (4 * wd.d * 4 + 8)
    tv_bytes = state_bytes + wd.B * Tt * wd.H * (5 * wd.d * 4 + 8) + wd.B * Tt * 4
    tc_bytes = 2 * state_bytes
    mv_bytes = state_bytes + vec_bytes                      # read the state once
    mc_bytes = 2 * state_bytes + vec_bytes - wd.B * Td * wd.H * wd.d * 4   # no o written

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
                "log_alpha U(-0.1,-0.001)%s)" % (", S0 N(0,0.02^2)" if has_s0 else ""),
        "config": {"workload": w.name + ("_fg2plus" if args.fg2 else "_gdn2" if args.gdn2
                                         else "_raw_prologue" if args.prologue else ""),
                   "call": ("gdr_fg2_chunk_fwd" if args.fg2 else "gdr_gdn2_chunk_fwd" if args.gdn2
                            else "gdr_chunk_fwd"),
                   "gate": "channel" if channel else "scalar",
                   "B": B, "T": T, "H": H, "d_k": d, "d_v": d, "chunk": C,
                   "global_batch": B, "seq_len": T, "parallelism": "single GPU"},
        "roofline": roofline,
        "prefill_mfma": {"algorithmic_flops_per_launch": flops, "tflops": tflops,
                         "peak_tflops": BF16_PEAK_TFLOPS, "frac": tflops / BF16_PEAK_TFLOPS, **issued},
        "decode": {"workload": wd.name, "call": "gdr_decode_step", "ms_per_step_median": dms,
                   "tokens_per_s": wd.B / (dms * 1e-3),
                   "algorithmic_bytes": dbytes, "achieved_GBs": dgbs,
                   "peak_GBs": HBM_PEAK_GBS, "frac": dgbs / HBM_PEAK_GBS, "traffic": traffic_of(4),
                   "timing": "median of %d in-place steps, HIP events" % len(dtimes)},
        "decode_multi": {"call": "gdr_decode_multi", "draft_tokens": Td,
                         "verify_ms": mres["verify"], "verify_bytes": mv_bytes,
                         "verify_GBs": mv_bytes / (mres["verify"] * 1e-3) / 1e9,
                         "commit_ms": mres["commit"], "commit_bytes": mc_bytes,
                         "commit_GBs": mc_bytes / (mres["commit"] * 1e-3) / 1e9,
                         "note": "verify: state read once, o for all draft tokens; commit: "
                                 "state of the accepted prefix written in place"},
        "decode_tree": {"call": "gdr_decode_tree + gdr_decode_tree_commit", "nodes": Tt, "tree": "random",
                        "verify_ms": mres["tree_verify"], "verify_bytes": tv_bytes,
                        "verify_GBs": tv_bytes / (mres["tree_verify"] * 1e-3) / 1e9,
                        "commit_ms": mres["tree_commit"], "commit_bytes": tc_bytes,
                        "commit_GBs": tc_bytes / (mres["tree_commit"] * 1e-3) / 1e9,
                        "note": "verify: every node's o and written value from one pass over the state "
                                "(bytes: the state, q, k, v, o, written values, gates, parents); commit: "
                                "the accepted node's state rebuilt in place (bytes: state read and "
                                "written; its path's keys and values are a few KiB)"},
    }
    if others:
        out["other_prefill"] = others
    out.update(extra_info)
    if not args.no_cpu_baseline and not variant:
        import oracle.gdr_oracle as og  # noqa: F401  (builds the oracle on first use)
        threads = host_threads()
        reps, secs = cpu_baseline(inp, threads, S0=inp.get("S0"))
        out["cpu_baseline"] = {"value": reps * B * T / secs, "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": "the whole prefill workload (B=%d,T=%d,H=%d,d=%d) "
                                         "through the fp64 token-by-token oracle, %d times, "
                                         "%.1f s on %d threads of %s (the host cores this process "
                                         "may use, within the per-GPU share OMP_NUM_THREADS=%s); "
                                         "the GPU call is %.0fx its throughput"
                                         % (B, T, H, d, reps, secs, threads, cpu_model(),
                                            os.environ.get("OMP_NUM_THREADS", "unset"),
                                            out["value"] / (reps * B * T / secs))}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
