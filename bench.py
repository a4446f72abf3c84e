"""Benchmark of the attention hot path on one MI355X.

One step = forward (attn_fwd) + query-side backward with the preprocess folded in
(attn_bwd_dq_d: dQ and D) + key-side backward (attn_bwd_dkdv), the order attn_bwd
takes for bf16, over one batch of resident synthetic inputs: the whole path, fwd and bwd.  Default workload: B=4, H=16, N=4096,
d=128, causal, bf16 (the N = 4k case of the headline metric); the N = 16k case
(B=1, H=16) is measured in the same run and reported under "secondary", and the
same N = 16k shape with a local + global block mask under "block_sparse".

Prints ONE JSON line.  `value` is fwd+bwd TFLOP/s (4 N^2 d per head forward,
2.5x that backward, halved for the causal mask) from the wall clock around
the timed steps; per-kernel durations come from HIP events recorded on the
stream the kernels run on; `roofline` is for the dominant kernel.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

from exact_tiled_attention_12_amd import (attn_bwd_blocksparse, attn_bwd_dkdv, attn_bwd_dq_d,  # noqa: E402
                                          attn_fwd, attn_fwd_blocksparse, attn_fwd_fp8, prepare)
from exact_tiled_attention_12_amd.configs import CONFIGS  # noqa: E402
from exact_tiled_attention_12_amd.flops import attn_flops, blocksparse_flops  # noqa: E402
from exact_tiled_attention_12_amd.inputs import config_inputs, local_global_mask, make_fp8_inputs  # noqa: E402

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak at N=4k/16k, d=128"
PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5033.2           # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E, published
KERNEL_SOURCES = ["exact_tiled_attention_12_amd/csrc/attn_fwd.hip",
                  "exact_tiled_attention_12_amd/csrc/attn_bwd.hip",
                  "exact_tiled_attention_12_amd/csrc/attn_fwd_fp8.hip",
                  "exact_tiled_attention_12_amd/csrc/attn_common.h",
                  "exact_tiled_attention_12_amd/csrc/attn_tuning.h",
                  "exact_tiled_attention_12_amd/build.py"]          # (the compiler flags)


def source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def warm(run, steps, min_seconds):
    """Runs `run` at least `steps` times and until `min_seconds` of load have passed: the GPU's clocks
    take about 30 ms of load to settle, and a short workload's fixed step count covers less.  Returns
    the number of runs."""
    n, t0 = 0, time.perf_counter()
    while n < steps:
        run()
        n += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(5):
            run()
        n += 5
        torch.cuda.synchronize()
    return n


class Workload:
    def __init__(self, cfg, dev):
        self.cfg = cfg
        q, k, v, do = config_inputs(cfg)
        self.q, self.k, self.v = (t.to(dev) for t in (q, k, v))
        self.do = do.to(dev) if do is not None else None          # forward-only workloads have no dO
        B, H, N, d = q.shape
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.D = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.dq = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
        self.dk = torch.empty_like(self.dq)
        self.dv = torch.empty_like(self.dq)
        self.fl_fwd = attn_flops(B, H, N, d, cfg.causal, "fwd")
        self.fl_bwd = attn_flops(B, H, N, d, cfg.causal, "bwd")
        # each entry point's arguments checked and marshalled once (prepare): a step re-issues the same
        # C calls on the current stream, so that the host's per-call Python work does not leave the GPU
        # idle between short kernels (the d = 64 forward runs 41 us, about what those checks take)
        c = cfg
        self.launch = [prepare(attn_fwd, self.q, self.k, self.v, causal=c.causal, out=self.o, lse=self.lse)[0]]
        if c.backward:
            self.launch += [
                prepare(attn_bwd_dq_d, self.q, self.k, self.v, self.o, self.do, self.lse, D=self.D, causal=c.causal,
                        dq=self.dq)[0],
                prepare(attn_bwd_dkdv, self.q, self.k, self.v, self.do, self.lse, self.D, causal=c.causal,
                        dk=self.dk, dv=self.dv)[0]]

    KERNELS = ("attn_fwd", "attn_bwd_dq_d", "attn_bwd_dkdv")

    def step(self, ev=None):
        if ev is not None:
            ev[0].record()
        for i, launch in enumerate(self.launch):
            launch()
            if ev is not None:
                ev[i + 1].record()

    def measure(self, steps, warmup, min_warm_seconds=0.0):
        """Returns (wall seconds per step, {kernel: mean seconds per launch}), after `warmup` steps
        (and at least `min_warm_seconds` of them)."""
        self.warmup_done = warm(self.step, warmup, min_warm_seconds)
        # wall clock over exactly `steps` steps, synchronised on both sides
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        # per-kernel durations from events on the kernels' stream (a second pass)
        nk = len(self.KERNELS) if self.cfg.backward else 1
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
        for e in evs:
            self.step(e)
        torch.cuda.synchronize()
        per = {self.KERNELS[i]: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps * 1e-3 for i in range(nk)}
        return wall, per


class SparseWorkload:
    """Workload 4's shape (B=1 H=16 N=16384 d=128 causal) under a local + global block
    mask: each 128-query block keeps the key blocks within `window` blocks of its own
    and the first `n_global` ones.  One step = attn_fwd_blocksparse + attn_bwd_blocksparse."""

    def __init__(self, cfg, dev, window=8, n_global=1):
        self.cfg = cfg
        q, k, v, do = config_inputs(cfg)
        self.q, self.k, self.v, self.do = (t.to(dev) for t in (q, k, v, do))
        B, H, N, d = q.shape
        T = (N + 127) // 128
        self.mask_cpu = local_global_mask(T, window, n_global)
        self.mask = self.mask_cpu.to(dev)
        self.desc = (f"B={B} H={H} N={N} d={d} causal bf16, block mask: local {window} blocks + "
                     f"{n_global} global (128-row blocks), {int(self.mask_cpu.sum())} of {T * T} blocks kept")
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.ws = torch.empty(B * H * N * 4 + 256, dtype=torch.uint8, device=dev)
        self.dq = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
        self.dk = torch.empty_like(self.dq)
        self.dv = torch.empty_like(self.dq)
        self.fl_fwd = B * H * blocksparse_flops(self.mask_cpu, N, d, cfg.causal, "fwd")
        self.fl_bwd = 2.5 * self.fl_fwd
        self.fl_dense = attn_flops(B, H, N, d, cfg.causal, "fwd+bwd")

    def step(self, ev=None):
        c = self.cfg
        if ev is not None:
            ev[0].record()
        attn_fwd_blocksparse(self.q, self.k, self.v, self.mask, causal=c.causal, out=self.o, lse=self.lse)
        if ev is not None:
            ev[1].record()
        attn_bwd_blocksparse(self.q, self.k, self.v, self.o, self.do, self.lse, self.mask, causal=c.causal,
                             workspace=self.ws, dq=self.dq, dk=self.dk, dv=self.dv)
        if ev is not None:
            ev[2].record()

    def measure(self, steps, warmup):
        self.warmup_done = warm(self.step, warmup, 0.06)
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for e in evs:
            self.step(e)
        torch.cuda.synchronize()
        t_fwd = sum(e[0].elapsed_time(e[1]) for e in evs) / steps * 1e-3
        t_bwd = sum(e[1].elapsed_time(e[2]) for e in evs) / steps * 1e-3
        return wall, t_fwd, t_bwd


def fp8_forward(cfg, dev, steps, warmup):
    """attn_fwd_fp8 on a workload's shape (fp8 e4m3 Q, K, V with per-tensor factors, O in bf16):
    mean HIP-event time per launch over `steps` launches on the current stream."""
    (q8, k8, v8), (sq, sk, sv) = make_fp8_inputs(cfg.B, cfg.H, cfg.N, cfg.d, seed=cfg.seed)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q8.shape[:-1], dtype=torch.float32, device=dev)
    run = prepare(attn_fwd_fp8, q8, k8, v8, sq, sk, sv, causal=cfg.causal, out=o, lse=lse)[0]
    warm(run, warmup, 0.06)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps * 1e-3
    fl = attn_flops(cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal, "fwd")
    return {"workload": f"B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} causal={cfg.causal}, fp8 e4m3 Q/K/V "
                        f"(per-tensor factors), O bf16", "us": round(t * 1e6, 2),
            "tflops": round(fl / t / 1e12, 2), "frac_fp8_peak": round(fl / t / 1e12 / PEAK_FP8_TFLOPS, 4),
            "frac_bf16_peak": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}


def cpu_baseline(cfg, budget_s=12.0):
    """The fp64 oracle (as it stands) on whole heads of the same workload, fwd + bwd."""
    import oracle
    q, k, v, do = config_inputs(cfg)
    BH = cfg.B * cfg.H
    flat = lambda t: t.reshape(BH, cfg.N, cfg.d)
    done, t0 = 0, time.perf_counter()
    while done < BH:
        oracle.fwd(flat(q)[done], flat(k)[done], flat(v)[done], causal=cfg.causal)
        oracle.bwd(flat(q)[done], flat(k)[done], flat(v)[done], flat(do)[done], causal=cfg.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    fl = attn_flops(1, done, cfg.N, cfg.d, cfg.causal, "fwd+bwd")
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} of {BH} heads, naive fp64 forward + backward (explicit N x N S, P, dP, dS), "
                      f"N={cfg.N}, d={cfg.d}, causal={cfg.causal}; {dt:.1f} s wall"}


def workload_entry(idx, dev, steps, warmup):
    """One workload's line: per-kernel mean HIP-event time, TFLOP/s and fraction of the bf16 peak
    (algorithmic FLOPs: 4 N^2 d per head forward, the backward's 2.5x split as in main())."""
    cfg = CONFIGS[idx]
    w = Workload(cfg, dev)
    wall, per = w.measure(steps, warmup, 0.06)    # warm-up of at least 60 ms (30 steps of workload 2: ~1.5 ms)
    warmup = w.warmup_done
    kflops = {"attn_fwd": w.fl_fwd, "attn_bwd_dkdv": 2.0 * w.fl_fwd, "attn_bwd_dq_d": 0.5 * w.fl_fwd}
    ent = {"workload": f"{cfg.name} (seed {cfg.seed})", "steps": steps, "warmup": warmup,
           "ms_per_step": round(wall * 1e3, 4),
           "kernels": {n: {"us": round(t * 1e6, 2), "tflops": round(kflops[n] / t / 1e12, 2),
                           "frac_peak": round(kflops[n] / t / 1e12 / PEAK_BF16_TFLOPS, 4)} for n, t in per.items()},
           "fwd_tflops": round(w.fl_fwd / per["attn_fwd"] / 1e12, 2),
           "fwd_frac_peak": round(w.fl_fwd / per["attn_fwd"] / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if cfg.backward:
        tb = sum(t for n, t in per.items() if n != "attn_fwd")
        ent.update(bwd_us=round(tb * 1e6, 2), bwd_tflops=round(w.fl_bwd / tb / 1e12, 2),
                   bwd_frac_peak=round(w.fl_bwd / tb / 1e12 / PEAK_BF16_TFLOPS, 4),
                   value=round((w.fl_fwd + w.fl_bwd) / wall / 1e12, 2))
    else:
        ent.update(value=round(w.fl_fwd / wall / 1e12, 2))
    log(f"bench: workload {idx} step {wall * 1e3:.3f} ms; " +
        ", ".join(f"{n} {t * 1e6:.1f} us ({kflops[n] / t / 1e12:.0f} TFLOP/s)" for n, t in per.items()))
    del w
    torch.cuda.empty_cache()
    return ent


PROBE_MIXES = {0: "MFMA only (register operands)", 1: "MFMA fed from LDS (one ds_read_b128 per product)",
               2: "MFMA + softmax-like VALU (per product: exp of an FMA, a max, an add)",
               3: "MFMA fed from LDS + softmax-like VALU"}


def mfma_ceiling(dev, launches=20, iters=4096, mix=0):
    """What the matrix cores sustain now: libmfma_rate.so's bf16 MFMA loop (two waves per SIMD, four
    independent accumulator chains per wave; `mix` adds LDS operand reads and/or softmax-like VALU work)
    over every CU, after ~50 ms of the same load so that the clock has settled.  Returns its TFLOP/s
    (HIP events over `launches` launches), the shader clock from its s_memtime / s_memrealtime stamps
    (median over workgroups, MHz), and the FLOP per CU and clock those two imply (4096 when the
    products issue back to back), or None without the probe."""
    import ctypes
    import statistics
    from exact_tiled_attention_12_amd.build_probe import PROBE_PATH
    if not os.path.exists(PROBE_PATH):
        log("bench: no libmfma_rate.so (build it with __graft_entry__.build())")
        return None
    L = ctypes.CDLL(PROBE_PATH)
    L.mfma_rate_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.mfma_rate_probe.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wg = 2 * cus                                            # 256 threads each: 8 waves per CU
    out = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    stamps = torch.zeros(wg * 4, dtype=torch.int64, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream

    def run():
        if L.mfma_rate_probe(wg, iters, mix, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stamps.data_ptr()),
                             ctypes.c_void_p(st)) != 0:
            raise RuntimeError("mfma_rate_probe failed")

    for _ in range(100):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        run()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / launches
    flops = wg * 4 * iters * 4 * 32768.0
    tf = flops / t / 1e12
    s4 = stamps.cpu().view(wg, 4).tolist()
    mhz = statistics.median((t1 - t0) / ((r1 - r0) / 100e6) / 1e6 for t0, t1, r0, r1 in s4 if r1 > r0)
    return {"tflops": round(tf, 1), "us_per_launch": round(t * 1e6, 2), "shader_clock_mhz": round(mhz, 1),
            "flop_per_cu_per_clock": round(tf * 1e12 / (cus * mhz * 1e6), 1), "compute_units": cus,
            "mix": PROBE_MIXES[mix],
            "method": f"libmfma_rate.so: {wg} workgroups x 4 waves, {iters} x 4 independent "
                      "v_mfma_f32_32x32x16_bf16 per wave; HIP events over "
                      f"{launches} launches after 100 unmeasured ones; clock = s_memtime ticks per "
                      "s_memrealtime (100 MHz) tick"}


def trace_summary(path, skip):
    """Per-kernel launch statistics from a rocprofv3 kernel trace (CSV), over the launches after the
    first `skip` of each kernel (the warm-up: a fresh process's first launches run at lower clocks).
    Prints a markdown table; needs no GPU."""
    import csv
    import statistics
    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            durs.setdefault(name, []).append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))
    print(f"| kernel | launches (all) | launches kept | average (us) | median (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|---|---|")
    for name, ts in sorted(durs.items(), key=lambda kv: -sum(e - b for b, e in kv[1])):
        ts.sort()
        kept = [(e - b) / 1e3 for b, e in ts[skip:]]
        if not kept:
            continue
        print(f"| `{name}` | {len(ts)} | {len(kept)} | {statistics.mean(kept):.1f} | {statistics.median(kept):.1f} | "
              f"{min(kept):.1f} | {max(kept):.1f} |")


def clock_summary(prefix, skip):
    """Per-kernel GFX clock from a rocprofv3 run with --pmc GRBM_COUNT --kernel-trace (CSV output,
    files PREFIX_counter_collection.csv, PREFIX_kernel_trace.csv, PREFIX_agent_info.csv): GRBM_COUNT
    counts GFX clocks on every XCD of the dispatch, so clock = GRBM_COUNT / XCDs / duration.  Prints a
    markdown table over the dispatches after the first `skip` of each kernel; needs no GPU."""
    import csv
    import statistics
    xcc = 1
    with open(prefix + "_agent_info.csv", newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Agent_Type", "").upper().endswith("GPU") or int(row.get("Num_Xcc") or 0) > 0:
                xcc = max(xcc, int(row.get("Num_Xcc") or 1))
    with open(prefix + "_kernel_trace.csv", newline="") as f:
        span = {r["Dispatch_Id"]: (int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in csv.DictReader(f)}
    per = {}
    with open(prefix + "_counter_collection.csv", newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != "GRBM_COUNT" or r["Dispatch_Id"] not in span:
                continue
            b, e = span[r["Dispatch_Id"]]
            if e > b:
                per.setdefault(r["Kernel_Name"], []).append((b, (e - b) * 1e-9, float(r["Counter_Value"])))
    print(f"XCDs per dispatch: {xcc}")
    print("| kernel | dispatches kept | median duration (us) | median clock (MHz) |")
    print("|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(x[1] for x in kv[1])):
        v = sorted(v)[skip:]
        if not v:
            continue
        short = name
        if name.endswith(")"):                 # drop the parameter list (the last balanced parentheses)
            depth = 0
            for i in range(len(name) - 1, -1, -1):
                depth += {")": 1, "(": -1}.get(name[i], 0)
                if depth == 0:
                    short = name[:i]
                    break
        print(f"| `{short}` | {len(v)} | {statistics.median(x[1] for x in v) * 1e6:.1f} | "
              f"{statistics.median(x[2] / xcc / x[1] / 1e6 for x in v):.0f} |")


def load_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it matches these sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    ent = t.get("kernels", {}).get(kernel)
    if not ent or t.get("source_hash") != source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks take about 20 steps (~30 ms of this load) to settle: the first steps of a process
    # run 5-15% slower, so the default warmup covers them
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--no-secondary", action="store_true", help="skip the N=16k measurement")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sparse", action="store_true", help="skip the block-sparse measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 forward measurement")
    ap.add_argument("--fp8-only", action="store_true", help="only the fp8 forward (for profiling)")
    ap.add_argument("--sparse-only", action="store_true",
                    help="only the block-sparse measurement (prints its JSON object; for profiling)")
    ap.add_argument("--copy-only", action="store_true",
                    help="only run a plain 1 GiB device copy (rocprofv3 counter calibration)")
    ap.add_argument("--no-other", action="store_true", help="skip workloads 2 and 5")
    ap.add_argument("--no-clock", action="store_true", help="skip the measured matrix-core ceiling")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="print per-kernel statistics of a rocprofv3 kernel trace (no GPU needed) and exit")
    ap.add_argument("--probe-only", action="store_true",
                    help="only the matrix-core ceiling probe, then 10 steps of the workload (for clock counters)")
    ap.add_argument("--clock-summary", metavar="PREFIX",
                    help="print per-kernel clocks from a rocprofv3 GRBM_COUNT run (no GPU needed) and exit")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --trace-summary: leave out the first SKIP launches of each kernel")
    args = ap.parse_args()

    if args.trace_summary:
        trace_summary(args.trace_summary, args.skip)
        return
    if args.clock_summary:
        clock_summary(args.clock_summary, args.skip)
        return

    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for {args.gpus}); "
              "heads shard across GPUs with no exchange, but no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_only:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel(), "launches": 3}))
        return

    if args.probe_only:
        res = []
        for mix in PROBE_MIXES:
            res.append(mfma_ceiling(dev, launches=10, mix=mix))
            log(f"bench: probe mix {mix} ({PROBE_MIXES[mix]}): {res[-1]['tflops']} TFLOP/s at "
                f"{res[-1]['shader_clock_mhz']} MHz ({res[-1]['flop_per_cu_per_clock']} FLOP per CU and clock)")
        w = Workload(CONFIGS[args.config], dev)
        for _ in range(10):
            w.step()
        torch.cuda.synchronize()
        print(json.dumps({"mfma_probe": res}), flush=True)
        return

    if args.fp8_only:
        for ci in (3, 4):
            r = fp8_forward(CONFIGS[ci], dev, args.steps, args.warmup)
            log(f"bench: fp8 forward {r['workload']}: {r['us']} us, {r['tflops']} TFLOP/s")
            print(json.dumps(r), flush=True)
        return

    if args.sparse_only:
        ws = SparseWorkload(CONFIGS[4], dev)
        log(f"bench: block-sparse, {ws.desc}")
        wall_s, tf_s, tb_s = ws.measure(args.steps, args.warmup)
        log(f"bench: block-sparse step {wall_s * 1e3:.3f} ms; fwd {tf_s * 1e6:.1f} us, bwd {tb_s * 1e6:.1f} us")
        print(json.dumps({"block_sparse_ms_per_step": round(wall_s * 1e3, 4), "fwd_us": round(tf_s * 1e6, 2),
                          "bwd_us": round(tb_s * 1e6, 2)}), flush=True)
        return

    cfg = CONFIGS[args.config]
    log(f"bench: workload {cfg.index} ({cfg.name}), warmup {args.warmup}, steps {args.steps}")
    w = Workload(cfg, dev)
    wall, per = w.measure(args.steps, args.warmup)
    flops = w.fl_fwd + (w.fl_bwd if cfg.backward else 0.0)
    value = flops / wall / 1e12
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    # algorithmic FLOPs per launch: forward 4 N^2 d per head; the backward's 2.5x
    # split as the key side's 4 products (2.0x) and the query side's 3 (1.5x)
    # minus the recomputed S and dP both sides share (counted once, on the key side)
    kflops = {"attn_fwd": w.fl_fwd, "attn_bwd_dkdv": 2.0 * w.fl_fwd, "attn_bwd_dq_d": 0.5 * w.fl_fwd}
    kern = {}
    for name, t in per.items():
        ent = {"us": round(t * 1e6, 2)}
        if name in kflops:
            tf = kflops[name] / t / 1e12
            ent.update(tflops=round(tf, 2), frac_peak=round(tf / PEAK_BF16_TFLOPS, 4))
        kern[name] = ent
    t_bwd = sum(t for n, t in per.items() if n != "attn_fwd")
    if cfg.backward:
        kern["bwd_total_tflops"] = round(w.fl_bwd / t_bwd / 1e12, 2)
        kern["bwd_frac_peak"] = round(w.fl_bwd / t_bwd / 1e12 / PEAK_BF16_TFLOPS, 4)
    kern["fwd_frac_peak"] = round(w.fl_fwd / per["attn_fwd"] / 1e12 / PEAK_BF16_TFLOPS, 4)
    log("bench: step %.3f ms; " % (wall * 1e3) + ", ".join(f"{n} {t * 1e6:.1f} us" for n, t in per.items()) +
        f"; fwd {w.fl_fwd / per['attn_fwd'] / 1e12:.1f} TFLOP/s" +
        (f", bwd {w.fl_bwd / t_bwd / 1e12:.1f} TFLOP/s" if cfg.backward else ""))

    # dominant kernel = the largest share of the step
    dom = max((n for n in per if n in kflops), key=lambda n: per[n])
    achieved = kflops[dom] / per[dom] / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "algorithmic_flop_per_launch": kflops[dom], "avg_launch_us": round(per[dom] * 1e6, 2),
                "traffic": load_traffic(dom)}

    ceiling = None
    if not args.no_clock:
        # the published peak assumes 2.4 GHz on every CU; the chip holds a lower clock under matrix-core
        # load, so the rate a pure MFMA loop sustains now is a second, measured ceiling
        # (mix 0); and what a dependency-free loop with the attention loop's work per product (an LDS operand
        # read, an exponential and three other VALU instructions) sustains (mix 3)
        ceiling = mfma_ceiling(dev)
        mixed = mfma_ceiling(dev, mix=3) if ceiling else None
        if ceiling and mixed:
            for c_ in (ceiling, mixed):
                c_["frac_of_ceiling"] = {n: round(kflops[n] / per[n] / 1e12 / c_["tflops"], 4) for n in per
                                         if n in kflops}
            ceiling["with_attention_mix"] = mixed
            roofline["measured_mfma_ceiling"] = ceiling["tflops"]
            roofline["frac_of_measured_ceiling"] = round(achieved / ceiling["tflops"], 4)
            roofline["measured_mixed_ceiling"] = mixed["tflops"]
            roofline["frac_of_mixed_ceiling"] = round(achieved / mixed["tflops"], 4)
            log(f"bench: MFMA ceiling {ceiling['tflops']} TFLOP/s at {ceiling['shader_clock_mhz']} MHz "
                f"({ceiling['flop_per_cu_per_clock']} FLOP per CU and clock); with the attention loop's mix "
                f"{mixed['tflops']} TFLOP/s at {mixed['shader_clock_mhz']} MHz")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"attention {'fwd+bwd' if cfg.backward else 'fwd'}, B={B} H={H} N={N} d={d} "
                               f"causal={cfg.causal} bf16 (Q,K,V,dO ~ N(0,1), seed {cfg.seed})",
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": d, "causal": cfg.causal,
                   "parallelism": "single GPU"},
        "kernels": kern,
        "roofline": roofline,
        "mfma_ceiling": ceiling,
        "source_hash": source_hash(),
    }

    if cfg.index == 3 and not args.no_secondary:
        cfg4 = CONFIGS[4]
        w = None
        torch.cuda.empty_cache()
        log("bench: secondary workload 4 (N=16384)")
        w4 = Workload(cfg4, dev)
        steps4 = max(3, args.steps // 2)
        wall4, per4 = w4.measure(steps4, max(2, args.warmup // 2), 0.06)
        tb4 = sum(t for n, t in per4.items() if n != "attn_fwd")
        out["secondary"] = {
            "workload": "B=1 H=16 N=16384 d=128 causal bf16 (Q,K x0.5)", "steps": steps4,
            "ms_per_step": round(wall4 * 1e3, 4),
            "value": round((w4.fl_fwd + w4.fl_bwd) / wall4 / 1e12, 2),
            "fwd_tflops": round(w4.fl_fwd / per4["attn_fwd"] / 1e12, 2),
            "fwd_frac_peak": round(w4.fl_fwd / per4["attn_fwd"] / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_tflops": round(w4.fl_bwd / tb4 / 1e12, 2),
            "bwd_frac_peak": round(w4.fl_bwd / tb4 / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels_us": {n: round(t * 1e6, 2) for n, t in per4.items()},
        }
        log(f"bench: N=16384 step {wall4 * 1e3:.3f} ms; " + ", ".join(f"{n} {t * 1e6:.1f} us" for n, t in per4.items()))

    if cfg.index == 3 and not args.no_other:
        # the other two bf16 workloads: 2 (d = 64, non-causal, forward) and 5 (d = 80, causal, fwd + bwd)
        w = None
        torch.cuda.empty_cache()
        out["other_workloads"] = {f"workload_{i}": workload_entry(i, dev, args.steps, args.warmup) for i in (2, 5)}

    if cfg.index == 3 and not args.no_sparse:
        torch.cuda.empty_cache()
        ws = SparseWorkload(CONFIGS[4], dev)
        log(f"bench: block-sparse, {ws.desc}")
        steps_s = max(3, args.steps // 2)
        wall_s, tf_s, tb_s = ws.measure(steps_s, max(2, args.warmup // 2))
        out["block_sparse"] = {
            "workload": ws.desc, "steps": steps_s, "ms_per_step": round(wall_s * 1e3, 4),
            "value": round((ws.fl_fwd + ws.fl_bwd) / wall_s / 1e12, 2), "unit": "TFLOP/s (kept pairs)",
            "fwd_us": round(tf_s * 1e6, 2), "bwd_us": round(tb_s * 1e6, 2),
            "fwd_tflops": round(ws.fl_fwd / tf_s / 1e12, 2),
            "bwd_tflops": round(ws.fl_bwd / tb_s / 1e12, 2),
            "kept_fraction_of_causal_flops": round((ws.fl_fwd + ws.fl_bwd) / ws.fl_dense, 4),
        }
        log(f"bench: block-sparse step {wall_s * 1e3:.3f} ms; fwd {tf_s * 1e6:.1f} us, bwd {tb_s * 1e6:.1f} us")

    if cfg.index == 3 and not args.no_fp8:
        torch.cuda.empty_cache()
        out["fp8_forward"] = [fp8_forward(CONFIGS[ci], dev, max(5, args.steps), max(2, args.warmup // 2))
                              for ci in (3, 4)]
        log("bench: fp8 forward " + "; ".join(f"{r['workload'].split(',')[0]}: {r['us']} us, {r['tflops']} TFLOP/s"
                                               for r in out["fp8_forward"]))

    if not args.no_cpu:
        log("bench: CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
