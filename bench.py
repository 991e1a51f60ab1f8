#!/usr/bin/env python3
"""Benchmark of the MTP draft step on one MI355X.

A step is one pass of the whole hot path for one batch of synthetic input:
mtp_draft_combine (embedding gather, two RMSNorms, concat, fc [h, 2h], final
RMSNorm) then mtp_lmhead_argmax (the draft lm_head sweep with the fused
argmax), the draft token left on the device. Default workload: vocab 154,880,
hidden 4,096, BF16 weights, b = 1 (the draft-head shape the pages time).

Prints ONE JSON line. `value` is the step's algorithmic HBM bytes divided by
the step time (GB/s); `drafts_per_s` is b / step time. `roofline` rates the
dominant kernel (the lm_head sweep) from HIP events around K back-to-back
launches of it on its own stream, after the timed steps. `cpu_baseline` times the oracle (test
infrastructure) on the host on the same input.

Inputs are resident in HBM before timing. Weights are rotated over enough
copies that a copy is re-read only after more traffic than the 256 MB Infinity
Cache holds.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--dtype bf16|fp8|nvfp4] [--batch B] [--no-cpu-baseline]
  python bench.py --sweep-report     # lm_head + argmax on every head workload (one JSON line each)
  python bench.py --pmc-summary FETCH.csv WRITE.csv [--workload/--dtype/--batch as profiled]

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
LM_KERNEL = "lmhead_argmax_kernel"
KERNEL_SOURCES = ("mtp_draft_head_02_amd/csrc/sweep.hip", "mtp_draft_head_02_amd/csrc/mtp_device.h",
                  "mtp_draft_head_02_amd/csrc/mtp_kernels.h")
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
    ap.add_argument("--sweep-report", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (the reference kernel for HBM byte counters)")
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

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        lm = [float(r["Counter_Value"]) for r in rows if LM_KERNEL in r["Kernel_Name"]]
        if len(copy) != 1 or not lm:
            raise SystemExit(f"{path}: need one copyBuffer dispatch and >=1 {LM_KERNEL} dispatch "
                             f"(got {len(copy)}, {len(lm)})")
        factor = COPY_BYTES / (copy[0] * 1024.0)
        mean_kib = sum(lm) / len(lm)
        return factor, mean_kib, len(lm)

    ff, fk, nf = read(fetch_csv, "FETCH_SIZE")
    wf, wk, nw = read(write_csv, "WRITE_SIZE")
    fb, wb = round(fk * 1024 * ff), round(wk * 1024 * wf)
    n_eff = min(wl.mtp_vocab_size, wl.vocab) if wl.mtp_vocab_size > 0 else wl.vocab
    import mtp_draft_head_02_amd as m

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
        self.tok = [torch.zeros(b, dtype=torch.int32, device=dev) for _ in range(self.ncopies)]
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        self._prepare()

    def _prepare(self):
        m, torch = self.m, self.torch
        vp = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
        s = C.c_void_p(self.stream.cuda_stream)
        self.lm_args, self.cb_args = [], []
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

    def step(self, i: int):
        k = i % self.ncopies
        if self.with_combine:
            st = self.m.lib.mtp_draft_combine(*self.cb_args[k])
            if st:
                raise RuntimeError(f"mtp_draft_combine failed: {self.m.status_string(st)}")
        self.step_lmhead(i)

    def step_lmhead(self, i: int):
        st = self.m.lib.mtp_lmhead_argmax(*self.lm_args[i % self.ncopies])
        if st:
            raise RuntimeError(f"mtp_lmhead_argmax failed: {self.m.status_string(st)}")


def time_steps(sp: Stepper, steps: int, warmup: int):
    """W untimed steps, then exactly K timed steps between two events on the
    launch stream (synchronized on both sides). Then, for the roofline, K
    back-to-back lm_head launches (the same rotated inputs) between two events on
    the same stream: the kernel's average launch duration, dispatch gap included.
    No events sit between the kernels of either loop: an event marker between
    two kernels adds a few microseconds of idle GPU."""
    torch = sp.torch
    for i in range(warmup):
        sp.step(i)
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
    return {"wall_ms_per_step": wall_ms, "gpu_ms_per_step": gpu_ms, "lm_ms_mean": lm_ms}


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
    base = {
        "value": round(sp.step_bytes / per / 1e9, 3),
        "unit": "GB/s",
        "drafts_per_s": round(sp.b / per, 3),
        "ms_per_step": round(per * 1e3, 2),
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole step on one input ({reps} repetition(s)), fp64 C oracle, {threads} threads",
    }
    return base, ctx


def run_one(args, wl, want_cpu: bool):
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
            "kind": "full draft step (combine + lm_head + argmax)" if with_combine else "lm_head + argmax",
            "vocab": wl.vocab, "hidden": wl.hidden, "batch": wl.batch, "weights": wl.wdtype,
            "mtp_vocab_size": wl.mtp_vocab_size, "rotated_weight_copies": sp.ncopies,
            "parallelism": "1 GPU (full-vocab share)",
        },
        "drafts_per_s": round(wl.batch / (step_ms * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "step_bytes": sp.step_bytes,
        "wall_ms_per_step": round(r["wall_ms_per_step"], 5),
        "lmhead_us_per_launch": round(lm_ms * 1e3, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": f"{LM_KERNEL} (lm_head sweep + fused argmax)",
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
    print(json.dumps(run_one(args, wl, want_cpu=not args.no_cpu_baseline)), flush=True)


if __name__ == "__main__":
    main()
