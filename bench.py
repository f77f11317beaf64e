"""Benchmark of one layer's FlexPrefill causal prefill on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
fp_prefill_plan (pattern determination + cumulative-attention selection)
followed by fp_prefill_attend (block-sparse attention).  Inputs are resident
in HBM before the timed region.  Default workload: the Llama-3.1-8B-shaped
layer (32 query / 8 key-value heads, head dim 128, bf16) at N = 131072,
block 128, gamma 0.95, tau 0.1, minimum budget 1024 tokens.

Prints ONE JSON line: sparse ms per layer (the metric), its parts, the dense
causal baseline with the same tile kernel, effective TFLOP/s over computed
blocks, the attention kernel's roofline (time from HIP events recorded by
the library around that kernel), and the CPU oracle timed on a bounded
sample (cpu_baseline).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--seed S]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill ms/layer + effective TFLOP/s & speedup vs dense @128k, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0
ATTN_SOURCES = ("attn_kernels.hip",)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attention_counters_llama8b_128k.md")


class PowerSampler:
    """Socket power and graphics clock of the GPU, read from the kernel GPU driver's
    metrics table (amdsmi, read-only) every 10 ms while a callable runs
    back to back for a few seconds.  The table lags the load by a few hundred
    milliseconds, so the first 40 % of the samples are dropped and a window
    much shorter than a second reads stale values.  The chip holds its socket
    power at the cap under these kernels, and the clock it settles at explains
    the attention kernel's fraction of the 2.4 GHz matrix peak.  Returns None
    where amdsmi is not available."""

    def __init__(self):
        self.ok = False
        try:
            import threading
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            cap = amdsmi.amdsmi_get_power_cap_info(self._h).get("power_cap")
            self.cap_w = round(cap / 1e6, 1) if isinstance(cap, (int, float)) else None
            self._threading = threading
            self.ok = True
        except Exception:
            pass

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        pw, clk = m.get("current_socket_power"), m.get("current_gfxclk")
        ok = lambda v: isinstance(v, (int, float)) and 0 < v < 65535
        return (pw if ok(pw) else None), (clk if ok(clk) else None)

    def measure(self, fn, seconds: float, sync_every: int = 4):
        if not self.ok:
            return None
        import torch
        stop, samples = [False], []

        def run():
            while not stop[0]:
                try:
                    samples.append(self._read())
                except Exception:
                    pass
                time.sleep(0.01)
        t = self._threading.Thread(target=run, daemon=True)
        t.start()
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            fn()
            n += 1
            if n % sync_every == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        stop[0] = True
        t.join()
        s = samples[int(len(samples) * 0.4):]
        pw = sorted(x for x, _ in s if x is not None)
        clk = sorted(y for _, y in s if y is not None)
        if not pw or not clk:
            return None
        return {"source": "amdsmi gpu metrics", "window_s": round(elapsed, 2), "calls": n, "samples": len(s),
                "socket_power_w_median": pw[len(pw) // 2], "gfxclk_mhz_median": clk[len(clk) // 2],
                "power_cap_w": self.cap_w}


def kernel_source_hash() -> str:
    """Hash of the attention kernel source without its // comments and blank
    lines (a comment edit does not change the kernel the counters measured)."""
    h = hashlib.sha256()
    for s in ATTN_SOURCES:
        with open(os.path.join(ROOT, "sparse_long_context_last_amd", "csrc", s), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def attention_kernel_name(cfg, token: bool) -> str:
    """The template instance of the sparse attention kernel the library runs
    for this workload (bf16: query-block pairs at block 64)."""
    g = "true" if token else "false"
    if cfg.dtype == "bf16":
        return f"fp::k_attn_bf16<{cfg.block}, true, {g}, {'true' if cfg.block == 64 else 'false'}, {cfg.d}>"
    return f"fp::k_attn_f32<{cfg.block}, true, {g}, {cfg.d}>"


def read_traffic(workload: str, default_settings: bool):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current attention kernel source and this workload
    (planned with the default settings)."""
    if not default_settings or not os.path.exists(COUNTERS_FILE):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(COUNTERS_FILE).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, sample_rows: int, budget_s: float, max_budget: int = 0,
                 qa_selection: str = "flattened", vs_granularity: str = "block"):
    """The oracle as it stands on the host cores, on a bounded sample of the
    layer, extrapolated by the oracle's own cost model.

    Selection: one query head of every planted type is planned in full; a
    head's planning cost is taken as that of the head of its type.
    Attention: the oracle computes a query-block row r from its full causal
    prefix (a dense [block, (r + 1) block] score matrix, masked afterwards),
    so a row costs in proportion to r + 1 "prefix blocks" whatever the
    selection; sampled rows of those heads give seconds per prefix block,
    scaled to the layer's Hq nb (nb + 1) / 2 prefix blocks."""
    import numpy as np
    import oracle as O
    from synth import LayerGen
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits, threadpool_info
        threadpool_limits(cores)
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas = None
    gen = LayerGen(cfg)
    types = [t for t in ("V", "S", "QA", "N") if t in gen.types]
    heads = {t: gen.types.index(t) for t in types}
    count = {t: gen.types.count(t) for t in types}
    plan_s, plans, inputs = {}, {}, {}
    for t in types:
        h = heads[t]
        q, k, v = gen.q_head(0, h), gen.k_head(0, h // cfg.group), gen.v_head(0, h // cfg.group)
        t0 = time.perf_counter()
        plans[t] = O.plan_head(q, k, cfg.block, cfg.gamma, cfg.tau, cfg.min_budget, max_budget, qa_selection,
                               vs_granularity)
        plan_s[t] = time.perf_counter() - t0
        inputs[t] = (q, k, v)
    rng = np.random.default_rng(7)
    per_head = max(1, sample_rows // len(types))
    work = []
    for t in types:
        rows = {cfg.nb - 1} | set(rng.choice(cfg.nb, size=min(cfg.nb, per_head - 1), replace=False).tolist())
        work += [(t, int(r)) for r in sorted(rows)]
    order = rng.permutation(len(work))
    t0 = time.perf_counter()
    prefix_done, rows_done = 0, 0
    for i in order:
        t, r = work[i]
        q, k, v = inputs[t]
        O.attend_rows(q, k, v, plans[t].mask, cfg.block, [r], plans[t].cols)
        prefix_done += r + 1
        rows_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t_attn = time.perf_counter() - t0
    prefix_total = cfg.B * cfg.Hq * cfg.nb * (cfg.nb + 1) // 2
    sel_s = cfg.B * sum(plan_s[t] * count[t] for t in types)
    attn_s = t_attn * prefix_total / max(prefix_done, 1)
    return {"value": round((sel_s + attn_s) * 1e3, 1), "unit": "ms/layer", "cores": cores, "kind": "oracle",
            "sample": ("selection: one head per planted type planned in full ("
                       + ", ".join(f"{t} {plan_s[t]:.2f} s x {count[t]} heads" for t in types)
                       + f" = {sel_s:.1f} s per layer); float64 attention: {rows_done} query-block rows of those "
                       f"heads covering {prefix_done} causal prefix blocks in {t_attn:.1f} s, scaled to the "
                       f"layer's {prefix_total} prefix blocks = {attn_s:.0f} s (the oracle builds each row's "
                       f"full causal prefix); host cores {cores}, BLAS threads {blas}")}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llama8b_128k")
    ap.add_argument("--seed", type=int, default=None,
                    help="seed of the synthetic inputs (default: the configuration's own)")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=24)
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--max-budget", type=int, default=0,
                    help="cap every query-block row at this many keys (0: uncapped)")
    ap.add_argument("--qa-selection", default="flattened", choices=["flattened", "querywise"],
                    help="how query-aware heads select blocks from the estimated map")
    ap.add_argument("--vs-granularity", default="block", choices=["block", "token"],
                    help="vertical-slash columns as whole blocks or token by token")
    ap.add_argument("--varlen", default="",
                    help="comma-separated sequence lengths: time a packed [T, H, d] batch of sequences of "
                         "these lengths (the --config head shape) instead of the batched layer")
    ap.add_argument("--power-s", type=float, default=2.5,
                    help="seconds of extra steps (and dense calls) over which socket power and clock are sampled "
                         "after the timed region (0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 (heads shard across "
                                   "GPUs with no exchange, each GPU running the layer on its share of heads)",
                          "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import sparse_long_context_last_amd as F
    from synth import BY_NAME, LayerGen
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        return 1
    cfg = BY_NAME[args.config]
    if args.seed is not None:
        cfg = cfg.with_(seed=args.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    lens = [int(x) for x in args.varlen.split(",") if x.strip()] if args.varlen else None
    if lens:
        # packed batch: each sequence generated with its own seed at the config's head shape
        if min(lens) < 1:
            print(json.dumps({"error": "--varlen lengths must be positive"}))
            return 2
        parts = []
        for b, n in enumerate(lens):
            n_gen = -(-n // 128) * 128
            qs_, ks_, vs_ = LayerGen(cfg.with_(B=1, N=n_gen, seed=cfg.seed + 7 * b)).torch_layer(dev)
            parts.append([t[0, :, :n].transpose(0, 1) for t in (qs_, ks_, vs_)])
            del qs_, ks_, vs_
        q, k, v = (torch.cat([pt[i] for pt in parts]).contiguous() for i in range(3))
        del parts
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        workload = f"{cfg.name}_varlen_{len(lens)}seq_{int(cu[-1])}tok"
    else:
        q, k, v = LayerGen(cfg).torch_layer(dev)
        workload = cfg.name
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    print(f"[bench] inputs {workload} generated in {gen_s:.1f}s", file=sys.stderr, flush=True)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def make_plan():
        kw = dict(block=cfg.block, gamma=cfg.gamma, tau=cfg.tau, min_budget=cfg.min_budget,
                  max_budget=args.max_budget, qa_selection=args.qa_selection,
                  vs_granularity=args.vs_granularity)
        return F.plan_varlen(q, k, cu, **kw) if lens else F.plan(q, k, **kw)

    def step():
        P = make_plan()
        F.attend(P, q, k, v, out=out)
        return P

    for _ in range(args.warmup):
        P = step()
    torch.cuda.synchronize()
    # timed steps: whole hot path; the library's events time the attention kernel
    F.profile_enable(True)
    F.profile_read(reset=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    plans = []
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        P = make_plan()
        ev[i][1].record(stream)
        F.attend(P, q, k, v, out=out)
        ev[i][2].record(stream)
        plans.append(P)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    plan_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev]))
    attend_ms = float(np.median([b.elapsed_time(c) for _, b, c in ev]))
    step_ms = float(np.mean([a.elapsed_time(c) for a, _, c in ev]))
    kern_ms, kern_n, _, _ = F.profile_read(reset=True)
    F.profile_enable(False)
    # socket power and clock over a few seconds of the same steps, after the timed ones
    power = PowerSampler()
    power_steps = power.measure(step, args.power_s) if args.power_s > 0 else None
    info = plans[-1].info()
    colptrs = ([c for c in plans[-1].debug_seqs("colptr") if c is not None]
               if args.vs_granularity == "token" else None)
    pattern, djs, _, _ = plans[-1].copy_out()
    del plans

    flop_per_block = 4.0 * cfg.block * cfg.block * cfg.d
    sparse_flop = info.total_blocks * flop_per_block
    gathered_tiles = 0
    if args.vs_granularity == "token":
        # gathered-column tiles: ceil(columns before the row's end / 64) per row,
        # each 64 keys x block queries x 4 d FLOP
        gathered_tiles = sum(int(((c.astype(np.int64)[:, 1:] + 63) // 64).sum()) for c in colptrs)
        sparse_flop += gathered_tiles * 4.0 * 64 * cfg.block * cfg.d
    dense_flop = info.dense_blocks * flop_per_block
    kern_avg_ms = kern_ms / max(kern_n, 1)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = sparse_flop / (kern_avg_ms * 1e-3) / 1e12

    dense_ms = None
    power_dense = None
    if not args.no_dense:
        F.profile_enable(True)
        F.profile_read(reset=True)
        outd = torch.empty_like(q)
        def dense():
            if lens:
                F.dense_attend_varlen(q, k, v, cu, block=cfg.block, out=outd)
            else:
                F.dense_attend(q, k, v, block=cfg.block, out=outd)
        dense()      # warm-up
        torch.cuda.synchronize()
        F.profile_read(reset=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.dense_reps):
            dense()
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / args.dense_reps
        _, _, dk_ms, dk_n = F.profile_read(reset=True)
        F.profile_enable(False)
        if args.power_s > 0:
            power_dense = power.measure(dense, args.power_s, sync_every=1)
        dense_kernel_ms = dk_ms / max(dk_n, 1)
        del outd

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, device=dev, dtype=torch.float32)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    traffic = read_traffic(workload, args.max_budget == 0 and args.qa_selection == "flattened"
                           and args.vs_granularity == "block")
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "kernel": attention_kernel_name(cfg, args.vs_granularity == "token"),
            "algorithmic_flop_per_launch": sparse_flop, "avg_kernel_ms": round(kern_avg_ms, 4),
            "launches": kern_n}
    cpu = None
    if not args.no_cpu_baseline and not lens:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, args.cpu_rows, args.cpu_budget_s, args.max_budget,
                           args.qa_selection, args.vs_granularity)

    rec = {
        "metric": METRIC,
        "value": round(step_ms, 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded planted head types; no datasets or weights)",
        "config": {"workload": workload, "B": len(lens) if lens else cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "N": None if lens else cfg.N, "seqlens": lens,
                   "d": cfg.d, "block": cfg.block, "gamma": cfg.gamma, "tau": cfg.tau,
                   "min_budget": cfg.min_budget, "max_budget": args.max_budget,
                   "qa_selection": args.qa_selection, "vs_granularity": args.vs_granularity,
                   "seed": cfg.seed, "parallelism": "single GPU"},
        "plan_ms": round(plan_ms, 3),
        "attend_ms": round(attend_ms, 3),
        "attention_kernel_ms": round(kern_avg_ms, 3),
        "wall_ms_per_step": round(wall_ms, 3),
        "dense_ms": round(dense_ms, 3) if dense_ms is not None else None,
        "dense_kernel_ms": round(dense_kernel_ms, 3) if dense_ms is not None else None,
        "speedup_vs_dense": round(dense_ms / step_ms, 3) if dense_ms is not None else None,
        "computed_blocks": info.total_blocks,
        "gathered_column_tiles": gathered_tiles,
        "dense_blocks": info.dense_blocks,
        "density": round(info.total_blocks / max(info.dense_blocks, 1), 5),
        "query_aware_heads": info.query_aware_heads,
        "eff_tflops_attention_kernel": round(achieved, 1),
        "eff_tflops_layer": round(sparse_flop / (step_ms * 1e-3) / 1e12, 1),
        "mfma_frac_attention_kernel": round(achieved / peak, 4),
        "dense_eff_tflops": round(dense_flop / (dense_kernel_ms * 1e-3) / 1e12, 1) if dense_ms else None,
        "roofline": roof,
        "power_sparse_steps": power_steps,
        "power_dense": power_dense,
        "cpu_baseline": cpu,
        "input_generation_s": round(gen_s, 1),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
