#!/usr/bin/env python3
"""Benchmark: Flex-Flash-Attention forward + backward TFLOP/s on one MI355X.

One step is one pass of the whole hot path over resident synthetic inputs:
block metadata of the slice table, forward (O, LSE) and backward (dQ, dK, dV).
FLOPs follow the MagiAttention blog deep-dive ("训练和 Benchmark 设置", FLOPs
equation): FLOPs_fwd = 4 * d * MaskArea * Hq, FLOPs_bwd = 2.5 * FLOPs_fwd,
MaskArea being the exact valid-pair count (computed on the device by the
metadata kernels); throughput = FLOPs / elapsed time (documentation page,
throughput formulas).

Default workload: 16384-token varlen-causal GQA (Hq 32, Hkv 8, d 128), lengths
U[256, 4096] trimmed to the total, seed 2.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import flexible_mask_attention_amd as ffa  # noqa: E402
from flexible_mask_attention_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
METRIC = "FFA fwd/bwd TFLOPs/s on valid mask area at 1 MI355X; % of bf16 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Case:
    """Resident inputs, outputs and scratch of one library call."""

    def __init__(self, call, seed, dev):
        self.c = call
        g = torch.Generator(device=dev).manual_seed(seed)
        shp = {"q": (call.Tq, call.Hq, call.d), "k": (call.Tk, call.Hkv, call.d),
               "v": (call.Tk, call.Hkv, call.d), "do": (call.Tq, call.Hq, call.d)}
        for n in ("q", "k", "v", "do"):
            setattr(self, n, torch.randn(*shp[n], generator=g, device=dev).to(torch.bfloat16))
        host = torch.tensor(call.slices, dtype=torch.int32).reshape(-1, 5)
        self.slices = host.to(dev)
        nbytes = ffa.meta_workspace_size(len(call.slices), call.Tq, call.Tk, call.d, host)
        self.meta_buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.meta = ffa.build_meta(self.slices, call.Tq, call.Tk, call.d, out=self.meta_buf)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(call.Hq, call.Tq, dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.ws = torch.empty(max(256, ffa.bwd_workspace_size(self.q, self.k)), dtype=torch.uint8, device=dev)

    def build_meta(self):
        c = self.c
        ffa._check(ffa.lib().ffa_build_block_meta(self.slices.data_ptr(), len(c.slices), c.Tq, c.Tk, c.d,
                                                  self.meta_buf.data_ptr(), self.meta_buf.numel(),
                                                  ffa._stream()), "ffa_build_block_meta")

    def fwd(self):
        ffa.fwd(self.q, self.k, self.v, self.meta, out=self.o, lse=self.lse)

    def bwd(self, phases=ffa.BWD_ALL):
        ffa.bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.meta, dq=self.dq, dk=self.dk,
                dv=self.dv, workspace=self.ws, phases=phases)

    def step(self):
        self.build_meta()
        self.fwd()
        self.bwd()


class GroupedCase:
    """All calls of a workload (same sequence lengths and head_dim) as one
    grouped launch: one tensor set with the calls' heads side by side, each
    call's kv heads with its own metadata (ffa_fwd_grouped / ffa_bwd_grouped)."""

    def __init__(self, calls, seed, dev):
        self.parts = [Case(c, seed + i, dev) for i, c in enumerate(calls)]
        c0 = calls[0]
        assert all((c.Tq, c.Tk, c.d) == (c0.Tq, c0.Tk, c0.d) for c in calls)
        for n in ("q", "k", "v", "do"):
            setattr(self, n, torch.cat([getattr(p, n) for p in self.parts], dim=1).contiguous())
        for p in self.parts:      # keep only the metadata of the parts
            for n in ("q", "k", "v", "do", "o", "lse", "dq", "dk", "dv", "ws"):
                setattr(p, n, None)
        self.metas = [p.meta for p in self.parts]
        self.kv_end, e = [], 0
        for c in calls:
            e += c.Hkv
            self.kv_end.append(e)
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[1], c0.Tq, dtype=torch.float32, device=dev)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.ws = torch.empty(max(256, ffa.bwd_workspace_size(self.q, self.k)), dtype=torch.uint8, device=dev)

    def build_meta(self):
        for p in self.parts:
            p.build_meta()

    def fwd(self):
        ffa.fwd_grouped(self.q, self.k, self.v, self.metas, self.kv_end, out=self.o, lse=self.lse)

    def bwd(self, phases=ffa.BWD_ALL):
        ffa.bwd_grouped(self.q, self.k, self.v, self.o, self.lse, self.do, self.metas, self.kv_end,
                        dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws, phases=phases)

    def step(self):
        self.build_meta()
        self.fwd()
        self.bwd()


PHASES = ["meta", "fwd", "bwd_dq", "bwd_dkdv"]


def phase_times(cases, min_reps, min_seconds=1.0):
    """Device time (ms) of each phase per step, from HIP events recorded on the
    stream the library launches on (torch's current stream), over at least
    ``min_reps`` repetitions and ``min_seconds`` of device time.  The backward
    runs as in a step: the dQ kernel with the row statistics folded in
    (PRE | DQ), then dK/dV.  Returns per phase the mean, median, first and
    third quartile and the number of samples."""
    samples = {n: [] for n in PHASES}
    total, reps = 0.0, 0
    while reps < min_reps or total < 1e3 * min_seconds:
        rep = {n: 0.0 for n in PHASES}
        for cs in cases:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record()
            cs.build_meta()
            ev[1].record()
            cs.fwd()
            ev[2].record()
            cs.bwd(ffa.BWD_PRE | ffa.BWD_DQ)
            ev[3].record()
            cs.bwd(ffa.BWD_DKDV)
            ev[4].record()
            torch.cuda.synchronize()
            for i, n in enumerate(PHASES):
                rep[n] += ev[i].elapsed_time(ev[i + 1])
        for n in PHASES:
            samples[n].append(rep[n])
        total += sum(rep.values())
        reps += 1
    out = {}
    for n in PHASES:
        x = sorted(samples[n])
        q = lambda f: x[min(len(x) - 1, int(round(f * (len(x) - 1))))]   # noqa: E731
        out[n] = {"mean": sum(x) / len(x), "median": q(0.5), "q1": q(0.25), "q3": q(0.75), "n": len(x)}
    return out


def gemm_ceiling(dev, n=8192, reps=20):
    """Dense bf16 GEMM throughput of the platform library (torch.matmul, which
    dispatches to hipBLASLt) at n^3, timed with HIP events: context for the
    kernels' fraction of the published peak, not a denominator."""
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b)
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    med = times[len(times) // 2]
    tf = 2.0 * n ** 3 / (med * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "shape": f"{n}^3 bf16",
            "library": "torch.matmul (hipBLASLt)", "stat": f"median of {reps}"}


def source_code_digest(csrc):
    """sha256 over the code of the HIP sources in directory ``csrc``: ``//``
    comments, trailing blanks and empty lines are dropped, so only a change
    of the code itself changes it (the sources use no other comment form)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            lines = [ln.split("//", 1)[0].rstrip() for ln in fh]
        code = "\n".join(ln for ln in lines if ln)
        h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()


def kernel_source_digest():
    """Digest of the library's HIP code; recorded hardware counters are only
    used while the kernels they were taken on are unchanged."""
    return source_code_digest(os.path.join(ROOT, "flexible_mask_attention_amd", "csrc"))


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from profiles/traffic.json: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch, rocprofv3 --pmc), each scaled by the
    ratio of known bytes to what the same counter reads for a plain device
    copy.  None when no record matches this kernel, workload and source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None or rec.get("workload") != workload:
        return None
    cal = rec["copy_calibration"]
    f_fetch = cal["bytes"] / (cal["FETCH_SIZE_KiB"] * 1024.0)
    f_write = cal["bytes"] / (cal["WRITE_SIZE_KiB"] * 1024.0)
    return int(round(k["FETCH_SIZE_KiB"] * 1024.0 * f_fetch + k["WRITE_SIZE_KiB"] * 1024.0 * f_write))


def profile_phase(cases, phase, reps):
    """Launch one phase `reps` times (for hardware-counter runs under
    rocprofv3 --pmc).  `copy` is the calibration kernel: a plain device copy
    of 1 GiB, whose true HBM traffic is 1 GiB read + 1 GiB written."""
    for cs in cases:
        cs.step()
    torch.cuda.synchronize()
    if phase == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(reps):
            dst.copy_(src)
    else:
        for _ in range(reps):
            for cs in cases:
                if phase == "meta":
                    cs.build_meta()
                elif phase == "fwd":
                    cs.fwd()
                elif phase == "bwd_dkdv":
                    cs.bwd(ffa.BWD_DKDV)
                elif phase == "bwd_dq":
                    cs.bwd(ffa.BWD_PRE | ffa.BWD_DQ)
                else:
                    raise SystemExit(f"unknown phase {phase}")
    torch.cuda.synchronize()
    log(f"profiled phase {phase}: {reps} launch(es) per call")


def host_threads():
    """Threads for the oracle leg: the cores this process may run on
    (affinity), capped by OMP_NUM_THREADS when the environment sets it (the
    host's share of cores per GPU)."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(env)) if env.isdigit() and int(env) > 0 else aff
    return n, aff


def cpu_baseline(call, seed, area, min_seconds=10.0, full_limit_tflop=3.0):
    """The fp64 oracle, untuned, timed on the host cores.  A workload whose
    whole forward + backward is at most ``full_limit_tflop`` TFLOP (the 256-token
    and 16K workloads) runs whole, all heads and the full mask, repeated until
    ``min_seconds`` have passed.  A larger one runs on a bounded sample: O, LSE
    and dQ (``forward_backward_rows``) of blocks of 256 consecutive query rows at
    seeded random offsets, all query heads, until ``min_seconds`` have passed; its
    FLOPs are the algorithmic ones of those rows (8 d per valid pair and head:
    Q K^T, P V, dO V^T, dS K).  Inputs are the CPU-seeded tensors of the same
    shapes."""
    from oracle import ffa_oracle as orc
    threads, aff = host_threads()
    torch.set_num_threads(threads)
    T = wl.make_tensors(call, seed)
    full = 4.0 * call.d * area * call.Hq * 3.5
    reps, t0 = 0, time.perf_counter()
    if full <= full_limit_tflop * 1e12:
        while True:
            orc.forward(T["q"], T["k"], T["v"], call.slices)
            orc.backward(T["q"], T["k"], T["v"], T["do"], call.slices)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds or reps >= 5:
                break
        f = full * reps
        sample = (f"whole workload (all {call.Hq} query heads, full mask), fwd + bwd, "
                  f"{reps} pass(es) in {dt:.1f} s")
    else:
        g = torch.Generator().manual_seed(seed)
        blocks = torch.randperm((call.Tq + 255) // 256, generator=g).tolist()
        done, pairs = 0, 0
        for b in blocks:
            rows = np.arange(256 * b, min(256 * b + 256, call.Tq))
            orc.forward_backward_rows(T["q"], T["k"], T["v"], T["do"], call.slices, rows)
            for sl in call.slices:
                lo, hi, ok = orc.row_intervals_vec(sl, rows)
                pairs += int(np.where(ok, hi - lo + 1, 0).sum())
            done += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
        f = 8.0 * call.d * pairs * call.Hq
        sample = (f"{done} block(s) of 256 consecutive query rows at seeded random offsets of {call.Tq}, "
                  f"all {call.Hq} query heads: O, LSE and dQ of those rows (oracle "
                  f"forward_backward_rows), {pairs} valid pairs per head, {dt:.1f} s")
    return {"value": round(f / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "affinity_cores": aff, "blas_threads": torch.get_num_threads(),
            "seconds": round(dt, 2), "sample": sample}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="1..5 (see workloads.py)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-ceiling", action="store_true")
    ap.add_argument("--min-time", type=float, default=1.0,
                    help="seconds of device time over which per-phase medians are taken")
    ap.add_argument("--profile-phase", default=None,
                    help="meta|fwd|bwd_dkdv|bwd_dq|copy: only launch that phase --reps times "
                         "(for hardware-counter runs); prints no JSON")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--grouped", action="store_true",
                    help="run a workload of several calls (the 128K video workload's two head "
                         "groups) as one grouped launch over one tensor set")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        log("bench.py measures one GPU only: this library has no multi-GPU path "
            "(each GPU would run its own share of the slices unchanged).")
        sys.exit(2)

    dev = torch.device("cuda:0")
    W = wl.workload(args.workload)
    if args.grouped:
        if len(W.calls) < 2:
            log("--grouped needs a workload of several calls (workload 4)")
            sys.exit(2)
        cases = [GroupedCase(W.calls, 100 * W.seed, dev)]
        parts = cases[0].parts
    else:
        cases = [Case(c, 100 * W.seed + i, dev) for i, c in enumerate(W.calls)]
        parts = cases
    torch.cuda.synchronize()
    areas = [p.meta.area() for p in parts]
    for p in parts:
        assert p.meta.status() == 0
    if args.profile_phase:
        profile_phase(cases, args.profile_phase, args.reps)
        return
    f_fwd = sum(4.0 * p.c.d * a * p.c.Hq for p, a in zip(parts, areas))
    f_bwd = 2.5 * f_fwd

    for _ in range(args.warmup):
        for cs in cases:
            cs.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for cs in cases:
            cs.step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps

    stats = phase_times(cases, max(20, args.steps // 2), args.min_time)
    ph = {n: stats[n]["median"] for n in PHASES}
    t_fwd = ph["fwd"] * 1e-3
    t_bwd = (ph["bwd_dkdv"] + ph["bwd_dq"]) * 1e-3
    # algorithmic FLOPs per kernel: fwd 4d per valid pair and head; of the
    # backward's 10d, dK/dV take 8d (Q K^T, dO V^T, P^T dO, dS^T Q), dQ 2d (dS K);
    # the dQ kernel also computes the row statistics -D and LSE log2 e
    alg = {"fwd": f_fwd, "bwd_dkdv": 0.8 * f_bwd, "bwd_dq": 0.2 * f_bwd}
    kernels = {}
    for n in ("fwd", "bwd_dkdv", "bwd_dq"):
        tf = alg[n] / (ph[n] * 1e-3) / 1e12
        st = stats[n]
        kernels[n] = {"ms": round(ph[n], 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "ms_mean": round(st["mean"], 4), "ms_iqr": [round(st["q1"], 4), round(st["q3"], 4)]}
    kernels["meta"] = {"ms": round(ph["meta"], 4),
                       "ms_iqr": [round(stats["meta"]["q1"], 4), round(stats["meta"]["q3"], 4)]}
    # roofline of the dominant kernel: algorithmic FLOPs per launch over its
    # average launch duration
    dom = max(("fwd", "bwd_dkdv", "bwd_dq"), key=lambda n: ph[n])
    achieved = round(alg[dom] / (stats[dom]["mean"] * 1e-3) / 1e12, 1)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": recorded_traffic(dom, W.name), "traffic_unit": "HBM bytes per launch"}

    value = (f_fwd + f_bwd) / step_s / 1e12
    c0 = W.calls[0]
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": W.name, "seqlen_q": c0.Tq, "seqlen_k": c0.Tk,
                   "num_heads_q": sum(c.Hq for c in W.calls), "num_heads_kv": sum(c.Hkv for c in W.calls),
                   "head_dim": c0.d, "num_slices": sum(len(c.slices) for c in W.calls),
                   "mask_area": sum(areas), "flops_fwd": f_fwd, "flops_bwd": f_bwd, "seed": W.seed,
                   "step": "block metadata + forward + backward",
                   "launch": "grouped (one launch for all head groups)" if args.grouped
                   else "one call per slice table"},
        "fwd_tflops": round(f_fwd / t_fwd / 1e12, 1),
        "fwd_pct_peak": round(100 * f_fwd / t_fwd / 1e12 / PEAK_BF16_TFLOPS, 2),
        "bwd_tflops": round(f_bwd / t_bwd / 1e12, 1),
        "bwd_pct_peak": round(100 * f_bwd / t_bwd / 1e12 / PEAK_BF16_TFLOPS, 2),
        "timing": {"stat": "median over HIP-event samples per phase, IQR alongside",
                   "samples": stats["fwd"]["n"],
                   "seconds": round(sum(stats[n]["mean"] for n in PHASES) * stats["fwd"]["n"] * 1e-3, 2)},
        "kernels": kernels,
        "roofline": roofline,
    }
    if not args.no_gemm_ceiling:
        out["gemm_ceiling"] = gemm_ceiling(dev)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(c0, W.seed, areas[0])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
