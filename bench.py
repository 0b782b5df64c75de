"""Benchmark: masked attention forward + backward on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input:
tile classification, forward kernel, backward pre-pass, backward kernel and
dQ finalize (plus mask localization for the context-parallel rank share).
Inputs are resident in HBM before the timed region starts.

Metric: TFLOP/s counted over UNMASKED pairs only (forward 4*d*NNZ, backward
10*d*NNZ, NNZ = exact number of open (query, key) pairs summed over batch and
heads) and that figure as a fraction of the bf16 dense MFMA peak.

Prints ONE JSON line. Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--seed S] [--no-cpu-baseline] [--no-sweep]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

METRIC = "masked attn fwd/bwd TFLOP/s on unmasked FLOPs, % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
HEADLINE = "c4_doc_causal_128k"


def nnz_of(vectors, seq_q, batch, heads):
    """Exact open-pair count from the bound vectors, O(Sk) per (b, h)."""
    total = 0
    for b in range(batch):
        for h in range(heads):
            pick = lambda x: x[b if x.shape[0] > 1 else 0, h if x.shape[1] > 1 else 0].astype(np.int64)
            lts, lte, uts, ute = (pick(x) for x in vectors)
            a0, a1 = np.clip(lts, 0, seq_q), np.clip(lte, 0, seq_q)
            b0, b1 = np.clip(uts, 0, seq_q), np.clip(ute, 0, seq_q)
            a1, b1 = np.maximum(a1, a0), np.maximum(b1, b0)
            inter = np.maximum(0, np.minimum(a1, b1) - np.maximum(a0, b0))
            total += int((seq_q - ((a1 - a0) + (b1 - b0) - inter)).sum())
    return total


SOURCES = {"fwd": "fwd.hip", "bwd": "bwd.hip", "bwd_dq": "bwd.hip", "bwd_dq_ds": "bwd_ds.hip",
           "fwd_fp8": "fwd_fp8.hip"}


def _profile_record(tag: str, kernel: str, workload: str):
    """Value of a machine-readable line `<tag>: kernel=K workload=W
    source=F sha256=H <key>=V` in the summaries under profiles/, kept only
    while F's sha256 prefix still equals H (the kernel has not changed since
    the profile was taken); else None."""
    import glob
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    src = SOURCES.get(kernel)
    if src is None:
        return None
    with open(os.path.join(root, "masked_tiled_attention_amd", "csrc", src), "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    pat = re.compile(tag + r": kernel=(\S+) workload=(\S+) source=(\S+) sha256=(\S+) \w+=([0-9.]+)")
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                m = pat.match(line.strip())
                if m and m[1] == kernel and m[2] == workload and m[3] == src and m[4] == digest:
                    return float(m[5])
    return None


def profiled_kernel_us(kernel: str, workload: str):
    """rocprofv3 average duration (us) of `kernel` over the timed steps of a
    bench.py run on `workload`, from the kernel-stats summaries under
    profiles/ (None when none matches the kernel's current source)."""
    return _profile_record("kernel_avg", kernel, workload)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summaries under profiles/, or None when none was
    taken on the kernel's current source."""
    v = _profile_record("traffic", kernel, workload)
    return None if v is None else int(v)


class Runner:
    """Device-resident inputs, outputs and workspaces of one workload."""

    def __init__(self, fm, w, torch, store_ds=True):
        self.fm, self.w, self.t = fm, w, torch
        dev = "cuda"
        self.q, self.k, self.v = (x.to(dev) for x in (w.q, w.k, w.v))
        self.do = w.do.to(dev) if w.backward else None
        if w.global_vectors is not None:
            self.gmask = fm.Mask.from_vectors(w.global_vectors, dev)
            self.mask = fm.fm_mask_localize(self.gmask, w.seq_q_global, w.chunk_start, w.chunk_len)
            torch.cuda.synchronize()
            self.vectors = tuple(x.cpu().numpy() for x in (self.mask.lts, self.mask.lte,
                                                           self.mask.uts, self.mask.ute))
            # the rank's mask-pruned K/V transfer set over the backward's key tiles
            self.transfer_bk = fm.fm_kernel_tile(w.head_dim, True)[1]
            need, count = fm.fm_kv_transfer_set(self.mask, w.seq_q, self.transfer_bk)
            self.kv_tiles = (int(count.sum()), int(need.numel()))
            # chunk -> rank planning for the whole context-parallel layout:
            # open pairs per chunk (device), then the host plan vs dual-chunk
            nck = 16   # 8 ranks, two chunks each
            cl = w.seq_q_global // nck
            starts, lens = [i * cl for i in range(nck)], [cl] * nck
            fm.fm_chunk_work(self.gmask, w.seq_q_global, starts, lens)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            cw = fm.fm_chunk_work(self.gmask, w.seq_q_global, starts, lens)
            t1.record()
            torch.cuda.synchronize()
            work = cw.sum(dim=0).cpu().tolist()
            ranks = nck // 2
            plan, mx = fm.fm_cp_plan(work, ranks)
            dual = [0] * ranks
            for c in range(nck):
                dual[min(c, nck - 1 - c)] += work[c]
            self.cp_plan = {"chunks": nck, "ranks": ranks, "chunk_work_ms": round(t0.elapsed_time(t1), 4),
                            "mean_load": sum(work) // ranks, "dual_chunk_max_load": max(dual),
                            "planned_max_load": mx}
            # finer chunks (8 per rank): the snake order vs the plan
            nf = 64
            clf = w.seq_q_global // nf
            wf = fm.fm_chunk_work(self.gmask, w.seq_q_global, [i * clf for i in range(nf)], [clf] * nf)
            wf = wf.sum(dim=0).cpu().tolist()
            _, mxf = fm.fm_cp_plan(wf, ranks)
            snake = [0] * ranks
            for c in range(nf):
                k, p_ = divmod(c, ranks)
                snake[p_ if k % 2 == 0 else ranks - 1 - p_] += wf[c]
            self.cp_plan["chunks_64"] = {"snake_max_load": max(snake), "planned_max_load": mxf}
        else:
            self.gmask = None
            self.mask = fm.Mask.from_vectors(w.vectors, dev)
            self.vectors = w.vectors
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device=dev)
        ws_f = fm.fm_workspace_size(self.q, self.k, self.v, self.mask, False, w.scale)
        self.ws_f = torch.empty(ws_f, dtype=torch.uint8, device=dev)
        if w.backward:
            # with the stored-dS workspace (sized from the classified mask) dQ is
            # formed from the dS tiles the dK/dV kernel writes; else recomputed
            ws_b = (fm.fm_bwd_workspace_size_ds(self.q, self.k, self.v, self.mask, w.scale) if store_ds
                    else fm.fm_workspace_size(self.q, self.k, self.v, self.mask, True, w.scale))
            self.ws_b = torch.empty(ws_b, dtype=torch.uint8, device=dev)
            self.ws_b_bytes = ws_b
            self.dq, self.dk, self.dv = (torch.empty_like(x) for x in (self.q, self.k, self.v))
        self.nnz = nnz_of(self.vectors, w.seq_q, w.batch, w.heads)

    def step(self):
        fm, w = self.fm, self.w
        if self.gmask is not None:
            self.mask = fm.fm_mask_localize(self.gmask, w.seq_q_global, w.chunk_start, w.chunk_len)
            fm.fm_kv_transfer_set(self.mask, w.seq_q, self.transfer_bk)
        fm.fm_attn_fwd(self.q, self.k, self.v, self.mask, w.scale, o=self.o, lse=self.lse,
                       workspace=self.ws_f)
        if w.backward:
            fm.fm_attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, self.mask, w.scale,
                           dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws_b)

    def dq_path(self):
        """True when the last backward formed dQ from stored dS tiles."""
        return self.fm.fm_bwd_dq_path(self.q, self.k, self.v, self.mask, self.ws_b, self.w.scale)

    def flops(self):
        d = self.w.head_dim
        return 4 * d * self.nnz, (10 * d * self.nnz if self.w.backward else 0)


class Fp8Runner:
    """The FP8 forward (E4M3 codes of the workload's shape, descales 1/64)
    on device-resident inputs."""

    def __init__(self, fm, w, torch, seed):
        from synth import tensors as ST
        dev = "cuda"
        self.fm, self.w = fm, w
        shp_q = (w.batch, w.seq_q, w.heads, w.head_dim)
        shp_k = (w.batch, w.seq_k, w.heads, w.head_dim)
        self.q = ST.fp8_codes("q", shp_q, seed).to(dev)
        self.k = ST.fp8_codes("k", shp_k, seed).to(dev)
        self.v = ST.fp8_codes("v", shp_k, seed).to(dev)
        self.ds = (1 / 64, 1 / 64, 1 / 64)
        self.mask = fm.Mask.from_vectors(w.vectors, dev)
        self.o = torch.empty(shp_q, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.batch, w.heads, w.seq_q), dtype=torch.float32, device=dev)
        n = fm.fm_workspace_size_fp8(self.q, self.k, self.v, self.mask, w.scale)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.nnz = nnz_of(w.vectors, w.seq_q, w.batch, w.heads)

    def step(self):
        self.fm.fm_attn_fwd_fp8(self.q, self.k, self.v, self.ds, self.mask, self.w.scale, o=self.o, lse=self.lse,
                                workspace=self.ws)


def time_steps(r, steps, warmup, torch, min_ms=0.0):
    """Wall time of whole steps on the launch stream, with nothing recorded
    inside a step: `warmup` untimed steps, then `steps` timed ones (more, when
    min_ms is set, until the timed region lasts about min_ms), one HIP event
    at each step boundary. Returns {"steps", "mean", "median", "min"} in ms
    per step."""
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    n = steps
    if min_ms > 0:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(2):
            r.step()
        e1.record()
        torch.cuda.synchronize()
        est = max(e0.elapsed_time(e1) / 2, 1e-3)
        n = max(steps, int(math.ceil(min_ms / est)))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        r.step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
    return {"steps": n, "mean": ev[0].elapsed_time(ev[n]) / n, "median": statistics.median(per), "min": min(per)}


def stage_times(r, steps, torch):
    """Per-stage kernel times from a separate, instrumented pass: the library
    records a HIP event pair around each of its launches, on the launch
    stream. Returns {stage: (ms per step, ms per launch, launches per step)}."""
    fm = r.fm
    torch.cuda.synchronize()
    fm.fm_profile_begin(64 * steps + 64)
    for _ in range(steps):
        r.step()
    raw = fm.fm_profile_end()
    return {s: (v[0] / steps, v[0] / v[1] if v[1] else 0.0, v[1] / steps) for s, v in raw.items()}


def cpu_baseline(w, vectors, budget_rows=None):
    """The oracle (float64 numpy, as it stands) on a bounded sample of the
    same workload: forward + backward of a contiguous block of query rows of
    head 0 against all keys (the block as a sub-problem: its rows are a
    single chunk, the vectors localized to it by the oracle)."""
    from oracle import attention as OA
    from oracle import masks as OM
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    d = w.head_dim
    rows = budget_rows or max(128, min(w.seq_q, int(7e10 / (w.seq_k * d))))
    r0 = max(0, (w.seq_q - rows) // 2)
    loc = OM.localize(tuple(x[:1, :1] for x in vectors), [r0], [rows])
    q = w.q[:1, r0:r0 + rows, :1].double().numpy()
    k = w.k[:1, :, :1].double().numpy()
    v = w.v[:1, :, :1].double().numpy()
    nnz = OA.nnz_closed_form(loc, rows)
    t0 = time.perf_counter()
    OA.forward(q, k, v, loc, w.scale, block=256)
    flops = 4 * d * nnz
    if w.backward:
        do = w.do[:1, r0:r0 + rows, :1].double().numpy()
        OA.backward(q, k, v, do, loc, w.scale, block=256)
        flops += 10 * d * nnz
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{w.name}: query rows [{r0}, {r0 + rows}) of batch 0 head 0 against all "
                      f"{w.seq_k} keys, fwd{'+bwd' if w.backward else ''}, nnz {nnz}, "
                      f"{dt:.1f} s, float64 numpy"}


def _tflops(flops, ms):
    return round(flops / (ms * 1e-3) / 1e12, 2) if ms > 0 else None


def _timing(t):
    return {"steps": t["steps"], "mean_ms": round(t["mean"], 4), "median_ms": round(t["median"], 4),
            "min_ms": round(t["min"], 4)}


# Executed matrix flops per open pair of each attention kernel: forward 4d
# (QK^T, PV), dK/dV kernel 8d (QK^T, dO V^T, P^T dO, dS^T Q), recompute dQ
# kernel 6d (QK^T, dO V^T, dS K), dQ from stored dS 2d (dS K).
KERNEL_FLOPS_PER_PAIR = {"fwd": 4, "bwd": 8, "bwd_dq": 6, "bwd_dq_ds": 2}
BWD_STAGES = ("bwd_pre", "bwd_plan", "bwd", "bwd_dq", "bwd_dq_ds")


def split_ms(st, backward):
    """(forward ms, backward ms) per step from stage times. The summary, class
    map and launch-order passes run as one launch each in the forward and in
    the backward (which does both of its tilings in each); their small cost is
    split evenly."""
    per = lambda s: st[s][0]
    shared = per("classify_summary") + per("classify_map") + per("order")
    fwd_ms = per("fwd") + (shared / 2 if backward else shared)
    bwd_ms = sum(per(s) for s in BWD_STAGES) + shared / 2 if backward else 0.0
    return fwd_ms, bwd_ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-store-ds", action="store_true",
                    help="minimum backward workspace: dQ recomputes S and dP instead of reading stored dS")
    ap.add_argument("--no-recompute", action="store_true",
                    help="skip timing the minimum-workspace (recompute dQ) backward beside the headline")
    ap.add_argument("--fp8-forward", action="store_true",
                    help="time only the FP8 forward (E4M3 codes of the workload's shape) and print its line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels shard over (batch, head) with no exchange, but no multi-GPU path is built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import masked_tiled_attention_amd as fm
    from synth import configs as SC

    fm.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy: {nbytes} bytes read, {nbytes} bytes written")
        del src, dst

    # sweep lines: at least 5 warm-up steps, then at least 20 timed steps or
    # 200 ms, whichever is longer; stage times from a separate 5-step pass
    SW_WARM, SW_STEPS, SW_MIN_MS, ST_STEPS = 5, 20, 200.0, 5

    if args.fp8_forward:
        w = SC.build(args.workload, args.seed, tensors=False)
        r = Fp8Runner(fm, w, torch, args.seed)
        t = time_steps(r, args.steps, args.warmup, torch)
        st = stage_times(r, ST_STEPS, torch)
        flops = 4 * w.head_dim * r.nnz
        kms = st["fwd"][1]
        achieved = flops / (kms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "fp8_forward_throughput", "value": _tflops(flops, t["mean"]), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["mean"], 4),
            "timing": _timing(t), "higher_is_better": True, "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_q": w.seq_q, "seq_k": w.seq_k,
                       "head_dim": w.head_dim, "nnz": r.nnz, "passes": "fwd"},
            "stages_ms_per_step": {s_: round(v[0], 4) for s_, v in st.items() if v[2]},
            "roofline": {"bound": "mfma", "kernel": "fwd_fp8", "kernel_ms": round(kms, 4), "achieved": round(achieved, 2),
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                         "traffic": measured_traffic("fwd_fp8", w.name)}}), flush=True)
        return

    log(f"[bench] building {args.workload} seed {args.seed}")
    w = SC.build(args.workload, args.seed)
    store_ds = not args.no_store_ds
    r = Runner(fm, w, torch, store_ds)
    t = time_steps(r, args.steps, args.warmup, torch)
    ms = t["mean"]
    st = stage_times(r, max(5, min(args.steps, 20)), torch)
    f_fwd, f_bwd = r.flops()
    fwd_ms, bwd_ms = split_ms(st, w.backward)
    total_tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    log(f"[bench] {w.name}: {ms:.3f} ms/step (median {t['median']:.3f}, min {t['min']:.3f}), "
        f"{total_tflops:.1f} TFLOP/s")

    # dominant kernel: the one with the largest time per step
    d = w.head_dim
    kern = max((k for k in KERNEL_FLOPS_PER_PAIR if st[k][2]), key=lambda s_: st[s_][0])
    kflops = KERNEL_FLOPS_PER_PAIR[kern] * d * r.nnz
    kms = st[kern][1]
    achieved = kflops / (kms * 1e-3) / 1e12
    prof_us = profiled_kernel_us(kern, w.name)
    roof = {"bound": "mfma", "kernel": kern, "kernel_ms": round(kms, 4), "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(kern, w.name),
            "flop_per_launch": kflops,
            "kernel_ms_rocprof": None if prof_us is None else round(prof_us / 1e3, 4),
            "frac_rocprof": None if prof_us is None else round(kflops / (prof_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    out = {
        "metric": METRIC,
        "value": round(total_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": t["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_q": w.seq_q,
                   "seq_k": w.seq_k, "head_dim": w.head_dim, "seed": args.seed,
                   "passes": "fwd+bwd" if w.backward else "fwd", "nnz": r.nnz,
                   "dq_from": ("stored dS" if store_ds else "recompute") if w.backward else None,
                   "density": round(r.nnz / (w.batch * w.heads * w.seq_q * w.seq_k), 5)},
        "timing": _timing(t),
        "pct_of_bf16_peak": round(100 * total_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": _tflops(f_fwd, fwd_ms)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": _tflops(f_bwd, bwd_ms),
                "workspace_bytes": r.ws_b_bytes if w.backward else None},
        "stages_ms_per_step": {s_: round(v[0], 4) for s_, v in st.items() if v[2]},
        "roofline": roof,
    }
    if w.backward:
        log(f"[bench] dQ path of the timed backward: {'stored dS' if r.dq_path() else 'recompute'}")
        out["config"]["dq_from"] = "stored dS" if r.dq_path() else "recompute"
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, r.vectors)
    del r
    torch.cuda.empty_cache()
    if w.backward and store_ds and not args.no_recompute:
        # the same step with the minimum workspace: dQ recomputes S and dP, and
        # no intermediate matrix is kept in HBM
        log(f"[bench] {w.name} with the minimum backward workspace (recompute dQ)")
        rr = Runner(fm, w, torch, store_ds=False)
        tr = time_steps(rr, args.steps, args.warmup, torch)
        sr = stage_times(rr, 5, torch)
        _, bwd_r = split_ms(sr, True)
        out["bwd_recompute"] = {
            "ms": round(bwd_r, 4), "tflops": _tflops(f_bwd, bwd_r), "workspace_bytes": rr.ws_b_bytes,
            "dq_kernel_ms": round(sr["bwd_dq"][1], 4),
            "dq_kernel_tflops": _tflops(6 * d * rr.nnz, sr["bwd_dq"][1]),
            "step": {"tflops": _tflops(f_fwd + f_bwd, tr["mean"]), **_timing(tr)},
            "dq_from": "stored dS" if rr.dq_path() else "recompute"}
        del rr
        torch.cuda.empty_cache()
    if not args.no_sweep:
        sweep = []
        # the other workloads, then grouped-query attention on the prefix-LM
        # workload (8 query heads on 2 K/V heads)
        jobs = [(name, None) for name in SC.NAMES if name != args.workload] + [("c3b_prefix_lm_32k", 2)]
        for name, kv_heads in jobs:
            log(f"[bench] sweep {name}" + (f" with {kv_heads} K/V heads" if kv_heads else ""))
            wx = SC.build(name, args.seed)
            if kv_heads:
                wx.k = wx.k[:, :, :kv_heads].contiguous()
                wx.v = wx.v[:, :, :kv_heads].contiguous()
            rx = Runner(fm, wx, torch, store_ds)
            tx = time_steps(rx, SW_STEPS, SW_WARM, torch, SW_MIN_MS)
            sx = stage_times(rx, ST_STEPS, torch)
            a, b = rx.flops()
            item = {"workload": name + (f" ({wx.heads} query heads on {kv_heads} K/V heads)" if kv_heads else ""),
                    "nnz": rx.nnz, "ms_per_step": round(tx["mean"], 4), "timing": _timing(tx),
                    "tflops": _tflops(a + b, tx["mean"]),
                    "fwd_kernel_tflops": _tflops(a, sx["fwd"][0])}
            if wx.backward:
                item["dkdv_kernel_tflops"] = _tflops(8 * wx.head_dim * rx.nnz, sx["bwd"][0])
                if rx.dq_path():
                    item["dq_ds_kernel_tflops"] = _tflops(2 * wx.head_dim * rx.nnz, sx["bwd_dq_ds"][0])
                    item["dq_ds_gbs"] = round(2 * rx.nnz / (sx["bwd_dq_ds"][0] * 1e-3) / 1e9, 1)
                else:
                    item["dq_kernel_tflops"] = _tflops(6 * wx.head_dim * rx.nnz, sx["bwd_dq"][0])
                _, bwd_x = split_ms(sx, True)
                item["bwd_tflops"] = _tflops(b, bwd_x)
            if wx.global_vectors is not None:
                item["localize_ms"] = round(sx["localize"][0], 4)
                item["transfer_set_ms"] = round(sx["transfer"][0], 4)
                item["kv_tiles_needed"] = f"{rx.kv_tiles[0]} of {rx.kv_tiles[1]} ({rx.transfer_bk}-key tiles)"
                item["cp_plan"] = rx.cp_plan
            sweep.append(item)
            del rx
            torch.cuda.empty_cache()
        out["workloads"] = sweep
        # the headline workload's spread over mask seeds: the document lengths
        # (and with them the density) change with the seed
        spread = [{"seed": args.seed, "nnz": out["config"]["nnz"], "density": out["config"]["density"],
                   "ms_per_step": out["ms_per_step"], "tflops": out["value"]}]
        for sd in (x for x in range(4) if x != args.seed):
            log(f"[bench] seed spread {w.name} seed {sd}")
            wx = SC.build(w.name, sd)
            rx = Runner(fm, wx, torch, store_ds)
            tx = time_steps(rx, SW_STEPS, SW_WARM, torch, SW_MIN_MS)
            a, b = rx.flops()
            spread.append({"seed": sd, "nnz": rx.nnz,
                           "density": round(rx.nnz / (wx.batch * wx.heads * wx.seq_q * wx.seq_k), 5),
                           "ms_per_step": round(tx["mean"], 4), "timing": _timing(tx),
                           "tflops": _tflops(a + b, tx["mean"])})
            del rx
            torch.cuda.empty_cache()
        out["seed_spread"] = spread
        # the FP8 forward (E4M3 inputs) on the long workloads, beside the bf16
        # forward kernel of the same workload
        fp8 = []
        bf16_fwd = {it["workload"]: it.get("fwd_kernel_tflops") for it in sweep}
        bf16_fwd[w.name] = _tflops(f_fwd, st["fwd"][0])
        for name in ("c3b_prefix_lm_32k", "c4_causal_128k", "c4_doc_causal_128k"):
            log(f"[bench] fp8 forward {name}")
            wx = SC.build(name, args.seed, tensors=False)
            rx = Fp8Runner(fm, wx, torch, args.seed)
            tx = time_steps(rx, SW_STEPS, SW_WARM, torch, SW_MIN_MS)
            sx = stage_times(rx, ST_STEPS, torch)
            kt = 4 * wx.head_dim * rx.nnz / (sx["fwd"][0] * 1e-3) / 1e12
            fp8.append({"workload": name, "nnz": rx.nnz, "ms_per_call": round(tx["mean"], 4), "timing": _timing(tx),
                        "fwd_kernel_ms": round(sx["fwd"][0], 4), "v_transpose_ms": round(sx["v_transpose"][0], 4),
                        "fwd_kernel_tflops": round(kt, 2), "frac_of_fp8_peak": round(kt / PEAK_FP8_TFLOPS, 4),
                        "bf16_fwd_kernel_tflops": bf16_fwd.get(name)})
            del rx
            torch.cuda.empty_cache()
        out["fp8_forward"] = fp8
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
