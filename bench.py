#!/usr/bin/env python3
"""Benchmark of the MTP draft step on one MI355X.

A step is one pass of the whole hot path for one batch of synthetic input:
one mtp_draft_step call (embedding gather, two RMSNorms, concat, fc [h, 2h],
final RMSNorm, the draft lm_head sweep with the fused argmax), the draft token
left on the device. Default workload: vocab 154,880,
hidden 4,096, BF16 weights, b = 1 (the draft-head shape the pages time).

Prints ONE JSON line. `value` is the step's algorithmic HBM bytes divided by
the step time (GB/s); `drafts_per_s` is b / step time. `roofline` rates the
dominant kernel (the lm_head sweep) from HIP events around K back-to-back
launches of it on its own stream, after the timed steps. `lmhead_by_dtype`
times the lm_head + argmax at 154,880 x 4,096, b = 1, in each of the three
weight precisions the same way (weights quantized on the GPU, rotated copies),
with p10 / p50 / p90 over batches of 10 back-to-back launches;
`quantize_us` the load-time quantizers on those weights (not part of the
metric); `step_by_batch` (default workload only) the draft step in BF16 at
b = 2, 4, 8 and in FP8 / NVFP4 at b = 1 and 8, timed as the main step is;
`stream_read_ceiling` a bare streaming read of the BF16 and NVFP4
heads' weight bytes with the sweeps' load pattern (mtp_stream_read), the
ceiling their fractions are set against. `cpu_baseline` times the oracle (test infrastructure) on the host on
the same input, with all its threads and with one.

Inputs are resident in HBM before timing. Weights are rotated over enough
copies that a copy is re-read only after more traffic than the 256 MB Infinity
Cache holds.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--dtype bf16|fp8|nvfp4] [--batch B] [--no-cpu-baseline]
  python bench.py --sweep-report     # lm_head + argmax on every head workload (one JSON line each)
  python bench.py --pmc-summary FETCH.csv WRITE.csv [--workload/--dtype/--batch as profiled]
  python bench.py --next-report      # the sweep with log-probability / grammar mask, chained drafts,
                                     # and the combine variants (one JSON line each)

`roofline.traffic` is the lm_head kernel's HBM bytes per launch from two
rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) of this script with
--calibrate-copy, each counter scaled by what it reads for a plain 1 GiB device
copy in the same run. --pmc-summary turns the two counter CSVs into the lines
kept in profiles/lmhead_argmax_hbm_traffic.txt; they carry a digest of the
kernel's sources and count only while the sources still match (else null).
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "draft lm_head+argmax GB/s (frac of HBM peak) and drafts/sec, 154880x4096"
MALL_BYTES = 256 << 20
# the lm_head kernel of each form (mtp_lmhead_kernel_form: 0 VALU sweep, 1 matrix-core sweep)
LM_KERNELS = {0: "lmhead_argmax_kernel", 1: "lmhead_mfma_kernel"}
KERNEL_SOURCES = tuple("mtp_draft_head_02_amd/csrc/" + f for f in (
    "sweep_impl.h", "mfma_impl.h", "sweep.hip", "lm_bf16.hip", "lm_fp8.hip", "lm_nvfp4.hip", "mfma_bf16.hip",
    "mfma_fp8.hip", "mfma_nvfp4.hip", "mtp_device.h", "mtp_kernels.h"))


def lm_kernel(wl) -> str:
    """Name of the lm_head kernel this workload's calls launch."""
    import mtp_draft_head_02_amd as m

    return LM_KERNELS[m.mtp_lmhead_kernel_form(wl.batch, wl.hidden, m.parse_wdtype(wl.wdtype))]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lmhead_argmax_hbm_traffic.txt")
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="step_154880x4096")
    ap.add_argument("--dtype", default=None, help="override the workload's weight precision")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-by-dtype", action="store_true",
                    help="skip the per-precision lm_head timings, the quantizer timings and the wider-batch steps")
    ap.add_argument("--sweep-report", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (the reference kernel for HBM byte counters)")
    ap.add_argument("--next-report", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script")
    return ap.parse_args()


def sources_digest() -> str:
    """sha256 (first 16 hex digits) over the lm_head kernel's source files."""
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_key(wl) -> str:
    n = min(wl.mtp_vocab_size, wl.vocab) if wl.mtp_vocab_size > 0 else wl.vocab
    return f"{wl.wdtype}:{wl.vocab}x{wl.hidden}:n{n}:b{wl.batch}"


def load_traffic(wl):
    """(fetch, write) HBM bytes per launch recorded for this workload with the
    current kernel sources, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    key, dig = traffic_key(wl), sources_digest()
    for line in open(TRAFFIC_FILE):
        f = line.split()
        if len(f) >= 5 and f[0] == "traffic" and f[1] == key and f[2] == dig:
            return int(f[3]), int(f[4])
    return None


def pmc_summary(fetch_csv: str, write_csv: str, wl) -> None:
    """Per-launch HBM bytes of the lm_head kernel from two counter CSVs, scaled by
    the 1 GiB copy's reading of the same counter."""
    import csv

    import mtp_draft_head_02_amd as m

    # the workload's own instantiation: the kernel templates start <format, batch, ...>
    LM_KERNEL = f"{lm_kernel(wl)}<{m.parse_wdtype(wl.wdtype)}, {wl.batch},"

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        # the calibration copy is the process's first copy (before any weights exist)
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        lm = [float(r["Counter_Value"]) for r in rows if LM_KERNEL in r["Kernel_Name"]]
        if not copy or not lm:
            raise SystemExit(f"{path}: need the calibration copyBuffer dispatch and >=1 {LM_KERNEL} dispatch "
                             f"(got {len(copy)}, {len(lm)})")
        factor = COPY_BYTES / (copy[0] * 1024.0)
        mean_kib = sum(lm) / len(lm)
        return factor, mean_kib, len(lm)

    ff, fk, nf = read(fetch_csv, "FETCH_SIZE")
    wf, wk, nw = read(write_csv, "WRITE_SIZE")
    fb, wb = round(fk * 1024 * ff), round(wk * 1024 * wf)
    n_eff = min(wl.mtp_vocab_size, wl.vocab) if wl.mtp_vocab_size > 0 else wl.vocab
    alg = lm_bytes(m.parse_wdtype(wl.wdtype), n_eff, wl.hidden, wl.batch)
    print(f"# {traffic_key(wl)}: {nf} dispatches, FETCH_SIZE {fk:.1f} KiB x {ff:.4f} (copy calibration) = "
          f"{fb} B; {nw} dispatches, WRITE_SIZE {wk:.1f} KiB x {wf:.4f} = {wb} B; algorithmic {alg} B; "
          f"(fetch + write) / algorithmic = {(fb + wb) / alg:.4f}")
    print(f"traffic {traffic_key(wl)} {sources_digest()} {fb} {wb} {alg}")


def lm_bytes(wd: int, n: int, h: int, b: int) -> int:
    """Algorithmic bytes of one lm_head + argmax launch: weight codes and scales
    for the n swept rows, x, and the tokens written."""
    if wd == 0:
        w = n * h * 2
    elif wd == 1:
        w = n * h + n * 4
    else:
        w = n * h // 2 + n * h // 16 + 4
    return w + b * h * 2 + b * 4


def combine_bytes(b: int, h: int) -> int:
    """Embedding rows + target hidden + 3 gammas + fc [h, 2h] + x out (BF16)."""
    return b * h * 2 + b * h * 2 + 3 * h * 2 + h * 2 * h * 2 + b * h * 2


class Stepper:
    """Holds resident inputs (rotated copies) and prepared C-ABI arguments."""

    def __init__(self, wl, seed: int, with_combine: bool):
        import numpy as np
        import torch

        import mtp_draft_head_02_amd as m
        import synthetic_inputs as si

        self.m, self.torch, self.si, self.wl = m, torch, si, wl
        dev = "cuda:0"
        self.dev = dev
        b, h, V = wl.batch, wl.hidden, wl.vocab
        self.b, self.h, self.V = b, h, V
        self.wd = m.parse_wdtype(wl.wdtype)
        self.n_eff = min(wl.mtp_vocab_size, V) if wl.mtp_vocab_size > 0 else V
        self.lm_bytes = lm_bytes(self.wd, self.n_eff, h, b)
        self.with_combine = with_combine
        self.step_bytes = self.lm_bytes + (combine_bytes(b, h) if with_combine else 0)
        per_copy = self.step_bytes
        self.ncopies = max(2, -(-2 * MALL_BYTES // max(per_copy, 1)) + 1)
        self.ncopies = min(self.ncopies, 8)
        W0 = si.lm_weight(wl, seed, device=dev)
        self.W_host_src = W0  # BF16 source of copy 0 (for the oracle)
        heads = []
        for i in range(self.ncopies):
            Wi = W0 if i == 0 else si.lm_weight(wl, seed + 1000 * i, device=dev)
            heads.append(m.quantize_head(Wi, wl.wdtype))
            if i:
                del Wi
        self.heads = heads
        if with_combine:
            inps = [si.step_inputs(wl, seed if i == 0 else seed + 1000 * i, device=dev) for i in range(self.ncopies)]
            self.inps = inps
            self.x = [torch.empty((b, h), dtype=torch.bfloat16, device=dev) for _ in range(self.ncopies)]
            self.cws = [m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(b, h), dev)
                        for _ in range(self.ncopies)]
        else:
            self.inps = None
            self.x = [si.lm_x(wl, seed if i == 0 else seed + 1000 * i, device=dev) for i in range(self.ncopies)]
        self.lws = [m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(V, h, b, self.wd), dev)
                    for _ in range(self.ncopies)]
        self.sws = [m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(b, h), dev) for _ in range(self.ncopies)] \
            if with_combine else None
        self.tok = [torch.zeros(b, dtype=torch.int32, device=dev) for _ in range(self.ncopies)]
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        self._prepare()

    def _prepare(self):
        m, torch = self.m, self.torch
        vp = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        s = C.c_void_p(self.stream.cuda_stream)
        self.lm_args, self.cb_args, self.step_args = [], [], []
        self._tok_host = []
        for i in range(self.ncopies):
            hd = self.heads[i]
            ws = self.lws[i]
            self.lm_args.append((vp(self.x[i]), self.b, self.h, self.wd, vp(hd.w), vp(hd.scale), vp(hd.gscale),
                                 self.V, self.wl.mtp_vocab_size, vp(self.tok[i]), None, vp(ws),
                                 ws.numel(), s))
            if self.with_combine:
                inp = self.inps[i]
                import numpy as np

                t = np.ascontiguousarray(inp["tokens"], dtype=np.int32)
                self._tok_host.append(t)
                cws = self.cws[i]
                self.cb_args.append((vp(inp["embed"]), self.V, C.c_void_p(t.ctypes.data), vp(inp["hidden"]),
                                     vp(inp["gamma_e"]), vp(inp["gamma_h"]), vp(inp["fc"]), vp(inp["gamma_f"]),
                                     self.b, self.h, C.c_float(self.wl.eps), C.c_float(self.wl.gamma_offset),
                                     vp(self.x[i]), vp(cws), cws.numel(), s))
                sws = self.sws[i]
                self.step_args.append((vp(inp["embed"]), self.V, C.c_void_p(t.ctypes.data), 0, vp(inp["hidden"]),
                                       vp(inp["gamma_e"]), vp(inp["gamma_h"]), vp(inp["fc"]), vp(inp["gamma_f"]),
                                       self.b, self.h, C.c_float(self.wl.eps), C.c_float(self.wl.gamma_offset),
                                       self.wd, vp(hd.w), vp(hd.scale), vp(hd.gscale), self.V,
                                       self.wl.mtp_vocab_size, vp(self.tok[i]), vp(self.x[i]), None, None, vp(sws),
                                       sws.numel(), s))

    def step(self, i: int):
        k = i % self.ncopies
        if self.with_combine:
            st = self.m.lib.mtp_draft_step(*self.step_args[k])
            if st:
                raise RuntimeError(f"mtp_draft_step failed: {self.m.status_string(st)}")
        else:
            self.step_lmhead(i)

    def step_lmhead(self, i: int):
        st = self.m.lib.mtp_lmhead_argmax(*self.lm_args[i % self.ncopies])
        if st:
            raise RuntimeError(f"mtp_lmhead_argmax failed: {self.m.status_string(st)}")


BATCH = 10  # launches per timing window of the percentile figures


def windowed_us(fn, k: int, stream, batch: int = BATCH) -> dict:
    """k back-to-back calls (after a short warm-up) in windows of `batch`, each
    window between two events on `stream` (no event sits between two launches
    of a window): the mean per-call microseconds over all k, and p10 / p50 /
    p90 of the per-window means."""
    import numpy as np
    import torch

    for i in range(max(3, batch)):
        fn(i)
    torch.cuda.synchronize()
    nwin = max(1, k // batch)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nwin)]
    for w in range(nwin):
        ev[2 * w].record(stream)
        for j in range(batch):
            fn(w * batch + j)
        ev[2 * w + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[2 * w].elapsed_time(ev[2 * w + 1]) * 1e3 / batch for w in range(nwin)])
    return {"mean": float(per.mean()), "p10": float(np.percentile(per, 10)), "p50": float(np.percentile(per, 50)),
            "p90": float(np.percentile(per, 90)), "windows": int(nwin), "launches_per_window": batch}


def time_steps(sp: Stepper, steps: int, warmup: int):
    """W untimed steps (at least W, and continued until 0.3 s of them have run:
    a GPU that was idle runs its first launches several percent slower), then
    exactly K timed steps between two events on the launch stream
    (synchronized on both sides). Then, for the roofline, K back-to-back
    lm_head launches (the same rotated inputs) between two events on the same
    stream: the kernel's average launch duration, dispatch gap included. No
    events sit between the kernels of either loop: an event marker between two
    kernels adds a few microseconds of idle GPU."""
    torch = sp.torch
    t0, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t0 < 0.3:
        for _ in range(20):
            sp.step(i)
            i += 1
        torch.cuda.synchronize()

    def loop(fn, k):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(sp.stream)
        for i in range(k):
            fn(i)
        end.record(sp.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / k, (time.perf_counter() - t0) * 1e3 / k

    gpu_ms, wall_ms = loop(sp.step, steps)
    lm_ms, _ = loop(sp.step_lmhead, steps)
    step_w = windowed_us(sp.step, steps, sp.stream)
    lm_w = windowed_us(sp.step_lmhead, steps, sp.stream)
    return {"wall_ms_per_step": wall_ms, "gpu_ms_per_step": gpu_ms, "lm_ms_mean": lm_ms, "step_windows": step_w,
            "lm_windows": lm_w}


def lmhead_by_dtype(args) -> dict:
    """lm_head + argmax at 154,880 x 4,096, b = 1, in BF16, FP8 and NVFP4 (the
    same seeded weights quantized on the GPU, rotated copies, K back-to-back
    launches between two events, then the windowed percentiles); and the
    quantizers' time on those weights."""
    import torch

    import mtp_draft_head_02_amd as m
    import synthetic_inputs as si

    out, quant = {}, {}
    for dt in ("bf16", "fp8", "nvfp4"):
        wl = si.WORKLOADS[f"{dt}_154880x4096_b1"]
        sp = Stepper(wl, args.seed, with_combine=False)
        # warm-up of at least 0.3 s of back-to-back launches (an idle GPU first
        # runs the sweep several percent slower)
        t0, i = time.perf_counter(), 0
        while i < args.warmup or time.perf_counter() - t0 < 0.3:
            for _ in range(50):
                sp.step_lmhead(i)
                i += 1
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(sp.stream)
        for i in range(args.steps):
            sp.step_lmhead(i)
        b.record(sp.stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / args.steps
        w = windowed_us(sp.step_lmhead, args.steps, sp.stream)
        gbs = sp.lm_bytes / us / 1e3
        out[dt] = {"workload": wl.name, "kernel": lm_kernel(wl), "us_per_launch": round(us, 2),
                   "bytes_per_launch": sp.lm_bytes, "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                   "p10_us": round(w["p10"], 2), "p50_us": round(w["p50"], 2), "p90_us": round(w["p90"], 2),
                   "frac_at_p50": round(sp.lm_bytes / w["p50"] / 1e3 / HBM_PEAK_GBS, 4),
                   "weight_copies": sp.ncopies}
        if dt != "bf16":
            W = sp.W_host_src
            V, h = W.shape
            reps = 5
            if dt == "fp8":
                codes = torch.empty((V, h), dtype=torch.uint8, device=sp.dev)
                sc = torch.empty(V, dtype=torch.float32, device=sp.dev)
                fn = lambda: m.mtp_quantize_fp8(W, codes, sc)
                nbytes = V * h * 2 + V * h + 4 * V
            else:
                codes = torch.empty((V, h // 2), dtype=torch.uint8, device=sp.dev)
                bs = torch.empty((V, h // 16), dtype=torch.uint8, device=sp.dev)
                g = torch.empty(1, dtype=torch.float32, device=sp.dev)
                qws = torch.empty(m.mtp_quantize_nvfp4_workspace_bytes(V, h), dtype=torch.uint8, device=sp.dev)
                fn = lambda: m.mtp_quantize_nvfp4(W, codes, bs, g, qws)
                nbytes = 2 * V * h * 2 + V * h // 2 + V * h // 16 + 4  # the absmax pass reads W once more
            fn()
            torch.cuda.synchronize()
            a.record(sp.stream)
            for _ in range(reps):
                fn()
            b.record(sp.stream)
            torch.cuda.synchronize()
            qus = a.elapsed_time(b) * 1e3 / reps
            quant[dt] = {"shape": f"{V}x{h}", "us_per_call": round(qus, 1), "bytes_per_call": nbytes,
                         "GBps": round(nbytes / qus / 1e3, 1)}
        del sp
        torch.cuda.empty_cache()
    return {"lmhead_by_dtype": out, "quantize_us": quant}


STREAM_SHAPES = ("4 waves x 8 KB units", "4 waves x 4 KB", "8 waves x 4 KB", "8 waves x 8 KB",
                 "4 waves x 4 KB in 8 KB runs", "8 waves x 4 KB in 8 KB runs")


def stream_ceiling(args, sizes) -> dict:
    """The streaming-read reference kernel (mtp_stream_read: the sweeps' load
    pattern, no compute) over the lm_head's weight bytes at each size, two
    rotated buffers, K back-to-back launches between two events, the best of
    its six launch shapes: the read ceiling the sweeps' fraction of peak is
    set against."""
    import torch

    import mtp_draft_head_02_amd as m

    dev = torch.device("cuda", 0)
    stream = torch.cuda.Stream(device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    with torch.cuda.stream(stream):
        for name, nbytes in sizes.items():
            nbytes -= nbytes % 8192
            bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(2)]
            torch.cuda.synchronize()
            best = None
            for shape, sname in enumerate(STREAM_SHAPES):
                for i in range(max(args.warmup, 20)):
                    m.mtp_stream_read(bufs[i % 2], nbytes, 0, sink, stream, shape)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for i in range(args.steps):
                    m.mtp_stream_read(bufs[i % 2], nbytes, 0, sink, stream, shape)
                b.record(stream)
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / args.steps
                if best is None or us < best[0]:
                    best = (us, sname)
            us, sname = best
            gbs = nbytes / us / 1e3
            out[name] = {"bytes": nbytes, "us_per_launch": round(us, 2), "GBps": round(gbs, 1),
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "best_shape": sname}
            del bufs
            torch.cuda.empty_cache()
    return out


def cpu_baseline(sp: Stepper, budget_s: float = 20.0):
    """The oracle, as it stands, on the host: the same step on copy 0's inputs.
    Returns the baseline dict and the oracle's token (checked against the GPU's)."""
    import numpy as np

    import oracle
    import synthetic_inputs as si

    threads = oracle.default_threads()
    wl = sp.wl
    Wb = si.bits(sp.W_host_src)
    if sp.wd == 1:
        w, s = oracle.quantize_fp8(Wb, threads)
        g = None
    elif sp.wd == 2:
        w, s, g = oracle.quantize_nvfp4(Wb, threads)
    else:
        w, s, g = Wb, None, None
    if sp.with_combine:
        inp = sp.inps[0]
        host = {k: (si.bits(v) if k != "tokens" else v) for k, v in inp.items()}
    else:
        xb = si.bits(sp.x[0])
    reps, t_total, tok = 0, 0.0, None
    while True:
        t0 = time.perf_counter()
        if sp.with_combine:
            xb = oracle.draft_combine(host["embed"], host["tokens"], host["hidden"], host["gamma_e"],
                                      host["gamma_h"], host["fc"], host["gamma_f"], wl.eps, wl.gamma_offset)
        tok, L = oracle.lmhead_argmax(xb, wl.wdtype, w, s, g, vocab=sp.V, mtp_vocab_size=wl.mtp_vocab_size,
                                      threads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
        if t_total >= budget_s / 2 or reps >= 5:
            break
    per = t_total / reps
    ctx = (xb, wl.wdtype, w, s, g, L)
    # the same step once more with one thread
    t0 = time.perf_counter()
    if sp.with_combine:
        xb1 = oracle.draft_combine(host["embed"], host["tokens"], host["hidden"], host["gamma_e"],
                                   host["gamma_h"], host["fc"], host["gamma_f"], wl.eps, wl.gamma_offset)
    else:
        xb1 = xb
    tok1, _ = oracle.lmhead_argmax(xb1, wl.wdtype, w, s, g, vocab=sp.V, mtp_vocab_size=wl.mtp_vocab_size, threads=1)
    per1 = time.perf_counter() - t0
    assert np.array_equal(tok1, tok), "the oracle's result depends on its thread count"
    base = {
        "value": round(sp.step_bytes / per / 1e9, 3),
        "unit": "GB/s",
        "drafts_per_s": round(sp.b / per, 3),
        "ms_per_step": round(per * 1e3, 2),
        "cores": threads,
        "kind": "oracle",
        "sample": (f"the whole step on one input ({reps} repetition(s)), fp64 C oracle: lm_head + argmax row-split "
                   f"over {threads} threads, the combine on one thread (the oracle's combine has no row split)"),
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
        "one_thread": {"value": round(sp.step_bytes / per1 / 1e9, 3), "unit": "GB/s",
                       "ms_per_step": round(per1 * 1e3, 1), "drafts_per_s": round(sp.b / per1, 3), "cores": 1,
                       "sample": "the same step, one repetition"},
    }
    return base, ctx


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def steps_by_batch(args) -> dict:
    """The draft step (mtp_draft_step) at 154,880 x 4,096 in wider batches and
    the other precisions: BF16 b = 2, 4, 8; FP8 and NVFP4 b = 1 and 8. Each is
    timed as the main step is (resident rotated inputs, at least 0.3 s of
    warm-up steps, K steps between two events on the launch stream), with
    p10 / p50 / p90 over windows of back-to-back steps."""
    from dataclasses import replace

    import torch

    import synthetic_inputs as si

    out = {}
    for dt, b in (("bf16", 2), ("bf16", 4), ("bf16", 8), ("fp8", 1), ("fp8", 8), ("nvfp4", 1), ("nvfp4", 8)):
        wl = replace(si.WORKLOADS["step_154880x4096"], wdtype=dt, batch=b)
        sp = Stepper(wl, args.seed, with_combine=True)
        t0, i = time.perf_counter(), 0
        while i < args.warmup or time.perf_counter() - t0 < 0.3:
            for _ in range(20):
                sp.step(i)
                i += 1
            torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(sp.stream)
        for i in range(args.steps):
            sp.step(i)
        e.record(sp.stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(e) * 1e3 / args.steps
        w = windowed_us(sp.step, args.steps, sp.stream)
        out[f"{dt}_b{b}"] = {"us_per_step": round(us, 2), "drafts_per_s": round(b / us * 1e6, 1),
                             "step_bytes": sp.step_bytes, "GBps": round(sp.step_bytes / us / 1e3, 1),
                             "p10_us": round(w["p10"], 2), "p50_us": round(w["p50"], 2), "p90_us": round(w["p90"], 2),
                             "lm_kernel": lm_kernel(wl), "weight_copies": sp.ncopies}
        del sp
        torch.cuda.empty_cache()
    return {"step_by_batch": out}


def run_one(args, wl, want_cpu: bool, want_by_dtype: bool = False, want_steps: bool = False):
    import numpy as np
    import torch

    with_combine = wl.kind == "step"
    sp = Stepper(wl, args.seed, with_combine)
    r = time_steps(sp, args.steps, args.warmup)
    step_ms = r["gpu_ms_per_step"]
    lm_ms = r["lm_ms_mean"]
    achieved = sp.lm_bytes / (lm_ms * 1e-3) / 1e9
    value = sp.step_bytes / (step_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8e4m3-w/bf16-x/f32-acc", "nvfp4": "nvfp4-w/bf16-x/f32-acc"}[wl.wdtype],
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) activations; resident in HBM)",
        "config": {
            "workload": wl.name if (args.dtype is None and args.batch is None) else
            f"{wl.kind}_{wl.vocab}x{wl.hidden}_{wl.wdtype}_b{wl.batch}",
            "kind": "full draft step (mtp_draft_step: combine + lm_head + argmax)" if with_combine else
            "lm_head + argmax",
            "vocab": wl.vocab, "hidden": wl.hidden, "batch": wl.batch, "weights": wl.wdtype,
            "mtp_vocab_size": wl.mtp_vocab_size, "rotated_weight_copies": sp.ncopies,
            "parallelism": "1 GPU (full-vocab share)",
        },
        "drafts_per_s": round(wl.batch / (step_ms * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "step_bytes": sp.step_bytes,
        "wall_ms_per_step": round(r["wall_ms_per_step"], 5),
        "step_us_p10_p50_p90": [round(r["step_windows"][q], 2) for q in ("p10", "p50", "p90")],
        "lmhead_us_per_launch": round(lm_ms * 1e3, 2),
        "lmhead_us_p10_p50_p90": [round(r["lm_windows"][q], 2) for q in ("p10", "p50", "p90")],
        "percentiles": f"over windows of {BATCH} back-to-back calls (each window between two events)",
        "roofline": {
            "bound": "hbm",
            "kernel": f"{lm_kernel(wl)} (lm_head sweep + fused argmax)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "bytes_per_launch": sp.lm_bytes,
        },
    }
    tr = load_traffic(wl)
    if tr is not None:
        out["roofline"]["traffic"] = tr[0] + tr[1]
        out["roofline"]["traffic_read_write"] = [tr[0], tr[1]]
        out["roofline"]["traffic_over_algorithmic"] = round((tr[0] + tr[1]) / sp.lm_bytes, 4)
    out["roofline"]["traffic_source"] = ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated, "
                                         "for the current kernel sources" if tr is not None else
                                         "no counter record for the current kernel sources and this workload")
    if want_steps:
        out.update(steps_by_batch(args))
    if want_by_dtype:
        out.update(lmhead_by_dtype(args))
        # the read ceiling at the BF16 and NVFP4 heads' byte counts (154,880 x 4,096)
        out["stream_read_ceiling"] = stream_ceiling(args, {"bf16_weights": 154880 * 4096 * 2,
                                                           "nvfp4_weights": 154880 * (4096 // 2 + 4096 // 16)})
        out["stream_read_ceiling"]["kernel"] = ("mtp_stream_read: non-temporal 16-byte loads, contiguous units per "
                                                "wave, one block per CU, no compute; best of six launch shapes")
    if want_cpu:
        base, ctx = cpu_baseline(sp)
        out["cpu_baseline"] = base
        out["oracle_token_check"] = token_check(sp, ctx)
    return out


def token_check(sp: Stepper, ctx):
    """The GPU's copy-0 tokens (deterministic: copy 0 always sees the same input)
    against the oracle: equal where the tolerance tau = 1e-3 * sum |w x| decides
    the argmax, otherwise within tau[i1] + tau[g] of the oracle's winner i1."""
    import numpy as np

    import oracle

    xb, wdname, w, s, g, L = ctx
    gtok = sp.tok[0].cpu().numpy()
    ok, equal = True, 0
    for bi in range(sp.b):
        i1, gt = oracle.argmax(L[bi]), int(gtok[bi])
        if gt == i1:
            equal += 1
            continue
        rows = np.array([i1, gt])
        sub_s = None if s is None else np.ascontiguousarray(s[rows])
        _, tau = oracle.lmhead_logits(xb[bi:bi + 1], wdname, np.ascontiguousarray(w[rows]), sub_s, g, with_tau=True)
        ok = ok and (L[bi, i1] - L[bi, gt]) <= tau[0, 0] + tau[0, 1]
    return {"ok": bool(ok), "rows_equal": equal, "rows": sp.b}


def _loop_us(fn, k, stream):
    """Mean microseconds per call of k back-to-back calls between two events,
    after at least 0.3 s of untimed calls (an idle GPU runs its first launches
    slower)."""
    import torch

    t0, i = time.perf_counter(), 0
    while i < max(3, k // 10) or time.perf_counter() - t0 < 0.3:
        for _ in range(10):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(k):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / k


def _copies(nbytes: int) -> int:
    """Weight copies to rotate so a copy is re-read only after more than twice
    the Infinity Cache has streamed through."""
    return int(min(32, max(2, -(-2 * MALL_BYTES // max(nbytes, 1)) + 1)))


def next_report(args) -> None:
    """The rows past the draft step itself, each on its own line:
    - lm_head + argmax with the top-1 log-probability (and chain confidence),
      and with a grammar mask (density 1/2), against the plain sweep, at
      154,880 x 4,096, b = 1, per weight format;
    - chained drafts (combine with device-resident ids -> lm_head) against the
      same drafts with host ids, full step at 154,880 x 4,096 BF16;
    - the combine with the fc in FP8 / NVFP4 and the split e_proj / h_proj form,
      against the BF16 concat combine, at h = 4,096, b = 1.
    Calls go straight to the C entry points with prepared arguments, so host
    overhead stays below the kernels' time."""
    import numpy as np
    import torch

    import mtp_draft_head_02_amd as m
    import synthetic_inputs as si

    dev = "cuda:0"
    st = torch.cuda.current_stream()
    S = C.c_void_p(st.cuda_stream)
    L = m.lib
    K = args.steps
    vp = lambda t: None if t is None else C.c_void_p(t.data_ptr())

    def emit(d):
        print(json.dumps(d), flush=True)

    def timed(calls, nbytes):
        def fn(i):
            f, a = calls[i % len(calls)]
            r = f(*a)
            if r:
                raise RuntimeError(m.status_string(r))
        return _loop_us(fn, K, st)

    for dt in ("bf16", "fp8", "nvfp4"):
        wl = si.WORKLOADS[f"{dt}_154880x4096_b1"]
        wd = m.parse_wdtype(dt)
        base = lm_bytes(wd, wl.vocab, wl.hidden, 1)
        nc = _copies(base)
        heads = [m.quantize_head(si.lm_weight(wl, 50 + i, device=dev), dt) for i in range(nc)]
        x = si.lm_x(wl, 0, device=dev)
        ws = m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(wl.vocab, wl.hidden, 1, wd), dev)
        tok = torch.zeros(1, dtype=torch.int32, device=dev)
        lp = torch.zeros(1, dtype=torch.float32, device=dev)
        conf = torch.ones(1, dtype=torch.float32, device=dev)
        allowed = torch.zeros(1, dtype=torch.int32, device=dev)
        words = (wl.vocab + 31) // 32
        g = torch.Generator(device="cpu").manual_seed(1)
        mask = torch.randint(-2 ** 31, 2 ** 31 - 1, (1, words), generator=g, dtype=torch.int64).to(torch.int32).to(dev)
        wsb = ws.numel()
        common = lambda hd: (vp(x), 1, wl.hidden, wd, vp(hd.w), vp(hd.scale), vp(hd.gscale), wl.vocab, 0)
        runs = {
            "plain": ([(L.mtp_lmhead_argmax, common(hd) + (vp(tok), None, vp(ws), wsb, S)) for hd in heads], base),
            "logprob": ([(L.mtp_lmhead_argmax_logprob, common(hd) + (vp(tok), vp(lp), vp(conf), vp(ws), wsb, S))
                         for hd in heads], base + 8),
            "masked": ([(L.mtp_lmhead_argmax_masked, common(hd) + (vp(mask), words, vp(tok), vp(allowed), vp(ws), wsb, S))
                        for hd in heads], base + words * 4 + 4),
        }
        for name, (calls, nbytes) in runs.items():
            us = timed(calls, nbytes)
            emit({"row": "lm_head + argmax" if name == "plain" else f"lm_head + argmax, {name}",
                  "workload": wl.name, "us_per_call": round(us, 2), "bytes_per_call": nbytes,
                  "GBps": round(nbytes / us / 1e3, 1), "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                  "weight_copies": nc})
        del heads
        torch.cuda.empty_cache()

    # chained drafts: device-resident ids vs host ids (the same kernels)
    wl = si.WORKLOADS["step_154880x4096"]
    h = wl.hidden
    nbytes = lm_bytes(0, wl.vocab, h, 1) + combine_bytes(1, h)
    nc = _copies(nbytes)
    inps = [si.step_inputs(wl, 70 + i, device=dev) for i in range(nc)]
    heads = [m.quantize_head(si.lm_weight(wl, 70 + i, device=dev), "bf16") for i in range(nc)]
    cws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(1, h), dev)
    lws = m.zeroed_workspace(m.mtp_lmhead_argmax_workspace_bytes(wl.vocab, h, 1, 0), dev)
    toks = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(nc)]
    xs = [torch.empty((1, h), dtype=torch.bfloat16, device=dev) for _ in range(nc)]
    host_tok = [np.ascontiguousarray(inp["tokens"], dtype=np.int32) for inp in inps]
    eps, off = C.c_float(wl.eps), C.c_float(0.0)

    def cargs(c, tokp):
        inp = inps[c]
        return (vp(inp["embed"]), wl.vocab, tokp, vp(inp["hidden"]), vp(inp["gamma_e"]), vp(inp["gamma_h"]),
                vp(inp["fc"]), vp(inp["gamma_f"]), 1, h, eps, off, vp(xs[c]), vp(cws), cws.numel(), S)

    lm = [(vp(xs[c]), 1, h, 0, vp(heads[c].w), None, None, wl.vocab, 0, vp(toks[c]), None, vp(lws), lws.numel(), S)
          for c in range(nc)]
    chain = [cargs(c, vp(toks[(c - 1) % nc])) for c in range(nc)]
    hostc = [cargs(c, C.c_void_p(host_tok[c].ctypes.data)) for c in range(nc)]
    for name, comb, f in (("two launches, device-resident ids (chained)", chain, L.mtp_draft_combine_dev),
                          ("two launches, host ids", hostc, L.mtp_draft_combine)):
        def step(i, comb=comb, f=f):
            c = i % nc
            if f(*comb[c]) or L.mtp_lmhead_argmax(*lm[c]):
                raise RuntimeError("draft step failed")
        us = _loop_us(step, K, st)
        emit({"row": f"draft step, {name}", "workload": wl.name, "us_per_draft": round(us, 2),
              "drafts_per_s": round(1e6 / us, 1), "bytes_per_draft": nbytes, "GBps": round(nbytes / us / 1e3, 1),
              "weight_copies": nc})
    sws = m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(1, h), dev)

    def one_launch(c, tokp, on_dev):
        inp = inps[c]
        return (vp(inp["embed"]), wl.vocab, tokp, on_dev, vp(inp["hidden"]), vp(inp["gamma_e"]), vp(inp["gamma_h"]),
                vp(inp["fc"]), vp(inp["gamma_f"]), 1, h, eps, off, 0, vp(heads[c].w), None, None, wl.vocab, 0,
                vp(toks[c]), None, None, None, vp(sws), sws.numel(), S)

    for name, args_ in (("mtp_draft_step, device-resident ids (chained)",
                         [one_launch(c, vp(toks[(c - 1) % nc]), 1) for c in range(nc)]),
                        ("mtp_draft_step, host ids", [one_launch(c, C.c_void_p(host_tok[c].ctypes.data), 0)
                                                  for c in range(nc)])):
        def step1(i, args_=args_):
            if L.mtp_draft_step(*args_[i % nc]):
                raise RuntimeError("draft step failed")
        us = _loop_us(step1, K, st)
        emit({"row": f"draft step, {name}", "workload": wl.name, "us_per_draft": round(us, 2),
              "drafts_per_s": round(1e6 / us, 1), "bytes_per_draft": nbytes, "GBps": round(nbytes / us / 1e3, 1),
              "weight_copies": nc})
    # the chained drafts captured in a HIP graph, G per replay (launched on
    # the capture stream; the occupancy queries are cached by the calls above)
    G = 8
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Sc = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        for j in range(G):
            a_ = one_launch(j % nc, vp(toks[(j - 1) % nc]), 1)[:-1] + (Sc,)
            if L.mtp_draft_step(*a_):
                raise RuntimeError("draft step failed")
    torch.cuda.synchronize()
    us = _loop_us(lambda i: g.replay(), max(1, K // G), st) / G
    emit({"row": f"draft step, mtp_draft_step, device-resident ids, {G} chained per HIP graph replay",
          "workload": wl.name, "us_per_draft": round(us, 2), "drafts_per_s": round(1e6 / us, 1),
          "bytes_per_draft": nbytes, "GBps": round(nbytes / us / 1e3, 1), "weight_copies": nc})
    del g
    del inps, heads
    torch.cuda.empty_cache()

    # eager against HIP-graph chained drafts at 32,000 x 4,096 (a short step,
    # where the gaps between launches weigh more)
    wl = si.WORKLOADS["step_32000x4096"]
    h = wl.hidden
    nbytes = lm_bytes(0, wl.vocab, h, 1) + combine_bytes(1, h)
    nc = _copies(nbytes)
    inps = [si.step_inputs(wl, 75 + i, device=dev) for i in range(nc)]
    heads = [m.quantize_head(si.lm_weight(wl, 75 + i, device=dev), "bf16") for i in range(nc)]
    toks = [torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(nc)]
    sws = m.zeroed_workspace(m.mtp_draft_step_workspace_bytes(1, h), dev)

    def short(c, strm):
        inp = inps[c]
        return (vp(inp["embed"]), wl.vocab, vp(toks[(c - 1) % nc]), 1, vp(inp["hidden"]), vp(inp["gamma_e"]),
                vp(inp["gamma_h"]), vp(inp["fc"]), vp(inp["gamma_f"]), 1, h, eps, off, 0, vp(heads[c].w), None, None,
                wl.vocab, 0, vp(toks[c]), None, None, None, vp(sws), sws.numel(), strm)

    eager = [short(c, S) for c in range(nc)]

    def step2(i):
        if L.mtp_draft_step(*eager[i % nc]):
            raise RuntimeError("draft step failed")
    us = _loop_us(step2, K, st)
    emit({"row": "draft step, mtp_draft_step, device-resident ids (chained)", "workload": wl.name,
          "us_per_draft": round(us, 2), "drafts_per_s": round(1e6 / us, 1), "bytes_per_draft": nbytes,
          "GBps": round(nbytes / us / 1e3, 1), "weight_copies": nc})
    G = 8
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Sc = C.c_void_p(torch.cuda.current_stream().cuda_stream)
        for j in range(G):
            if L.mtp_draft_step(*short(j % nc, Sc)):
                raise RuntimeError("draft step failed")
    torch.cuda.synchronize()
    us = _loop_us(lambda i: g.replay(), max(1, K // G), st) / G
    emit({"row": f"draft step, mtp_draft_step, device-resident ids, {G} chained per HIP graph replay",
          "workload": wl.name, "us_per_draft": round(us, 2), "drafts_per_s": round(1e6 / us, 1),
          "bytes_per_draft": nbytes, "GBps": round(nbytes / us / 1e3, 1), "weight_copies": nc})
    del g, inps, heads
    torch.cuda.empty_cache()

    # combine variants at h = 4,096
    wl = si.WORKLOADS["step_32000x4096"]
    h = wl.hidden
    inp0 = si.step_inputs(wl, 80, device=dev)
    tk = np.ascontiguousarray(inp0["tokens"], dtype=np.int32)
    cws = m.zeroed_workspace(m.mtp_draft_combine_workspace_bytes(1, h), dev)
    x = torch.empty((1, h), dtype=torch.bfloat16, device=dev)
    small = 2 * h * 2 + 3 * h * 2 + h * 2  # embedding row, hidden, gammas, x out
    head_args = (vp(inp0["embed"]), wl.vocab, C.c_void_p(tk.ctypes.data), vp(inp0["hidden"]), vp(inp0["gamma_e"]),
                 vp(inp0["gamma_h"]))
    tail = lambda: (vp(inp0["gamma_f"]), 1, h, eps, off, vp(x), vp(cws), cws.numel(), S)
    variants = {"bf16 concat": ("bf16", 2 * h * h * 2), "fp8 fc": ("fp8", 2 * h * h + 4 * h),
                "nvfp4 fc": ("nvfp4", h * h + 2 * h * h // 16 + 4), "split (bf16)": ("split", 2 * h * h * 2)}
    for name, (kind, wbytes) in variants.items():
        nc = _copies(wbytes)
        if kind == "split":
            keep = [(si.normal_bf16(90 + i, si.TAG_LM, h, h, std=0.02, device=dev),
                     si.normal_bf16(190 + i, si.TAG_LM, h, h, std=0.02, device=dev)) for i in range(nc)]
            calls = [(L.mtp_draft_combine_split, head_args + (vp(e), vp(hp)) + tail()) for e, hp in keep]
        else:
            keep = [m.quantize_head(si.normal_bf16(90 + i, si.TAG_LM, h, 2 * h, std=0.02, device=dev), kind)
                    for i in range(nc)]
            calls = [(L.mtp_draft_combine_q, head_args + (q.wd, vp(q.w), vp(q.scale), vp(q.gscale)) + tail())
                     for q in keep]
        us = timed(calls, wbytes + small)
        nbytes = wbytes + small
        emit({"row": f"combine, {name}", "workload": f"fc {h} x {2 * h}, b = 1", "us_per_call": round(us, 2),
              "bytes_per_call": nbytes, "GBps": round(nbytes / us / 1e3, 1),
              "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4), "weight_copies": nc})
        del keep, calls
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the draft step's vocab shards are "
              "independent and this build runs the full-vocab share on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import synthetic_inputs as si

    def chosen_workload():
        w = si.WORKLOADS[args.workload]
        if args.dtype or args.batch:
            from dataclasses import replace

            w = replace(w, wdtype=args.dtype or w.wdtype, batch=args.batch or w.batch)
        return w

    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], chosen_workload())
        return
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.next_report:
        next_report(args)
        return
    if args.sweep_report:
        for name, wl in si.WORKLOADS.items():
            if wl.kind != "lmhead":
                continue
            print(json.dumps(run_one(args, wl, want_cpu=False)), flush=True)
            torch.cuda.empty_cache()
        return
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    wl = chosen_workload()
    by_dtype = not args.no_by_dtype and wl.kind == "step"
    default_step = by_dtype and wl.name == "step_154880x4096" and not args.dtype and not args.batch
    print(json.dumps(run_one(args, wl, want_cpu=not args.no_cpu_baseline, want_by_dtype=by_dtype,
                             want_steps=default_step)), flush=True)


if __name__ == "__main__":
    main()
