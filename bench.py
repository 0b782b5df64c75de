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
import os
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


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the rocprofv3
    FETCH_SIZE / WRITE_SIZE summaries under profiles/, or None when none was
    taken on the kernel's current source (sha256 prefix recorded with it)."""
    import glob
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    src = {"fwd": "fwd.hip", "bwd": "bwd.hip", "bwd_dq": "bwd.hip", "bwd_dq_ds": "bwd_ds.hip",
           "fwd_fp8": "fwd_fp8.hip"}.get(kernel)
    if src is None:
        return None
    with open(os.path.join(root, "masked_tiled_attention_amd", "csrc", src), "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()[:16]
    pat = re.compile(r"traffic: kernel=(\S+) workload=(\S+) source=(\S+) sha256=(\S+) bytes=(\d+)")
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                m = pat.match(line.strip())
                if m and m[1] == kernel and m[2] == workload and m[3] == src and m[4] == digest:
                    return int(m[5])
    return None


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


def time_steps(r, steps, warmup, torch, profile=True):
    fm = r.fm
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if profile:
        fm.fm_profile_begin(64 * steps + 64)
    start.record()
    for _ in range(steps):
        r.step()
    stop.record()
    torch.cuda.synchronize()
    stages = fm.fm_profile_end() if profile else {}
    ms = start.elapsed_time(stop) / steps
    return ms, stages


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-store-ds", action="store_true",
                    help="minimum backward workspace: dQ recomputes S and dP instead of reading stored dS")
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

    if args.fp8_forward:
        w = SC.build(args.workload, args.seed, tensors=False)
        r = Fp8Runner(fm, w, torch, args.seed)
        ms, stages = time_steps(r, args.steps, args.warmup, torch)
        per = lambda s: stages[s][0] / max(1, args.steps)
        flops = 4 * w.head_dim * r.nnz
        kms = stages["fwd"][0] / max(1, stages["fwd"][1])
        achieved = flops / (kms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "fp8_forward_throughput", "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
            "higher_is_better": True, "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_q": w.seq_q, "seq_k": w.seq_k,
                       "head_dim": w.head_dim, "nnz": r.nnz, "passes": "fwd"},
            "stages_ms_per_step": {s_: round(v[0] / max(1, args.steps), 4) for s_, v in stages.items() if v[1]},
            "roofline": {"bound": "mfma", "kernel": "fwd_fp8", "kernel_ms": round(kms, 4), "achieved": round(achieved, 2),
                         "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                         "traffic": measured_traffic("fwd_fp8", w.name)}}), flush=True)
        return

    log(f"[bench] building {args.workload} seed {args.seed}")
    w = SC.build(args.workload, args.seed)
    store_ds = not args.no_store_ds
    r = Runner(fm, w, torch, store_ds)
    ms, stages = time_steps(r, args.steps, args.warmup, torch)
    f_fwd, f_bwd = r.flops()
    per = lambda s: stages[s][0] / max(1, args.steps)
    # classification runs once in the forward and twice in the backward (one
    # per backward kernel tiling); its small cost is split in that ratio
    cls_ms = per("classify_summary") + per("classify_map")
    fwd_ms = per("fwd") + (cls_ms / 3 if w.backward else cls_ms)
    bwd_ms = (per("bwd_pre") + per("bwd_plan") + per("bwd") + per("bwd_dq") + per("bwd_dq_ds") + 2 * cls_ms / 3
              if w.backward else 0.0)
    total_tflops = (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
    log(f"[bench] {w.name}: {ms:.3f} ms/step, {total_tflops:.1f} TFLOP/s")

    # dominant kernel: the one with the largest time per step. Executed matrix
    # flops per open pair: forward 4d (QK^T, PV), dK/dV kernel 8d (QK^T, dO V^T,
    # P^T dO, dS^T Q), dQ kernel 6d (QK^T, dO V^T, dS K) or, from stored dS, 2d.
    d = w.head_dim
    kernel_flops = {"fwd": 4 * d * r.nnz, "bwd": 8 * d * r.nnz, "bwd_dq": 6 * d * r.nnz,
                    "bwd_dq_ds": 2 * d * r.nnz}
    kern = max((k for k in kernel_flops if stages[k][1]), key=lambda s: stages[s][0])
    kflops = kernel_flops[kern]
    kms = stages[kern][0] / max(1, stages[kern][1])
    achieved = kflops / (kms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(total_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
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
        "pct_of_bf16_peak": round(100 * total_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(f_fwd / (fwd_ms * 1e-3) / 1e12, 2) if fwd_ms else None},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 2) if bwd_ms else None},
        "stages_ms_per_step": {s: round(v[0] / max(1, args.steps), 4) for s, v in stages.items() if v[1]},
        "roofline": {"bound": "mfma", "kernel": kern, "kernel_ms": round(kms, 4),
                     "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(kern, w.name)},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w, r.vectors)
    if not args.no_sweep:
        sweep = []
        del r
        torch.cuda.empty_cache()
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
            msx, st = time_steps(rx, 5, 2, torch)
            a, b = rx.flops()
            pf = lambda s: st[s][0] / 5
            item = {"workload": name + (f" ({wx.heads} query heads on {kv_heads} K/V heads)" if kv_heads else ""),
                    "nnz": rx.nnz, "ms_per_step": round(msx, 4),
                    "tflops": round((a + b) / (msx * 1e-3) / 1e12, 2),
                    "fwd_kernel_tflops": round(a / (pf("fwd") * 1e-3) / 1e12, 2)}
            if wx.backward:
                item["dkdv_kernel_tflops"] = round(8 * wx.head_dim * rx.nnz / (pf("bwd") * 1e-3) / 1e12, 2)
                if st["bwd_dq_ds"][1] and pf("bwd_dq_ds") > pf("bwd_dq"):
                    item["dq_ds_kernel_tflops"] = round(2 * wx.head_dim * rx.nnz / (pf("bwd_dq_ds") * 1e-3) / 1e12, 2)
                    item["dq_ds_gbs"] = round(2 * rx.nnz / (pf("bwd_dq_ds") * 1e-3) / 1e9, 1)
                else:
                    item["dq_kernel_tflops"] = round(6 * wx.head_dim * rx.nnz / (pf("bwd_dq") * 1e-3) / 1e12, 2)
                bwd_x = sum(pf(s_) for s_ in ("bwd_pre", "bwd_plan", "bwd", "bwd_dq", "bwd_dq_ds"))
                item["bwd_tflops"] = round(b / (bwd_x * 1e-3) / 1e12, 2)
            if wx.global_vectors is not None:
                item["localize_ms"] = round(pf("localize"), 4)
                item["transfer_set_ms"] = round(pf("transfer"), 4)
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
            msx, _ = time_steps(rx, 5, 2, torch)
            a, b = rx.flops()
            spread.append({"seed": sd, "nnz": rx.nnz,
                           "density": round(rx.nnz / (wx.batch * wx.heads * wx.seq_q * wx.seq_k), 5),
                           "ms_per_step": round(msx, 4), "tflops": round((a + b) / (msx * 1e-3) / 1e12, 2)})
            del rx
            torch.cuda.empty_cache()
        out["seed_spread"] = spread
        # the FP8 forward (E4M3 inputs) on the long workloads, beside the bf16
        # forward kernel of the same workload
        fp8 = []
        bf16_fwd = {it["workload"]: it.get("fwd_kernel_tflops") for it in sweep}
        bf16_fwd[w.name] = round(f_fwd / (per("fwd") * 1e-3) / 1e12, 2)
        for name in ("c3b_prefix_lm_32k", "c4_causal_128k", "c4_doc_causal_128k"):
            log(f"[bench] fp8 forward {name}")
            wx = SC.build(name, args.seed, tensors=False)
            rx = Fp8Runner(fm, wx, torch, args.seed)
            msx, st = time_steps(rx, 5, 2, torch)
            pf = lambda s: st[s][0] / 5
            kt = 4 * wx.head_dim * rx.nnz / (pf("fwd") * 1e-3) / 1e12
            fp8.append({"workload": name, "nnz": rx.nnz, "ms_per_call": round(msx, 4),
                        "fwd_kernel_ms": round(pf("fwd"), 4), "v_transpose_ms": round(pf("v_transpose"), 4),
                        "fwd_kernel_tflops": round(kt, 2), "frac_of_fp8_peak": round(kt / PEAK_FP8_TFLOPS, 4),
                        "bf16_fwd_kernel_tflops": bf16_fwd.get(name)})
            del rx
            torch.cuda.empty_cache()
        out["fp8_forward"] = fp8
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
