"""Benchmark one DSA layer on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload s1m] [--secondary s128k]

A step is one pass of the layer's hot path over one batch of synthetic input
already resident in HBM: indexer + fused top-k and sparse attention forward
(one pipelined call that overlaps the two over query chunks on two streams),
and the backward for workloads that train (s128k, zigzag4).  Prints one JSON
line: tokens/s of the primary workload over the timed steps, the roofline of
its dominant kernel (per-launch durations from HIP events on the launch stream,
in a pass of the separate entry points after the timed steps), the CPU oracle
timed on a bounded sample of the same workload, and the secondary workload's
tokens/s, with the autograd integration's modes (plain, lean, offload) timed on it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_context_sparse_topk_amd as D  # noqa: E402
from long_context_sparse_topk_amd import training as TR  # noqa: E402
import synthetic as syn  # noqa: E402

HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
BF16_PEAK = 2.5e15         # flop/s, dense bf16 MFMA
FP8_PEAK = 5.0e15          # flop/s, dense fp8 MFMA
# VALU issue: 256 CUs x 4 SIMDs, one wave64 VALU instruction (16 lanes a cycle, 4 cycles)
# per SIMD every 4 cycles at 2.4 GHz; MFMA instructions take an issue slot too
VALU_ISSUE_PEAK = 256 * 4 * 2.4e9 / 4    # wave64 VALU instructions/s
# the indexer's minimal VALU stream per 64 (query, pool) pairs: the epilogue (4 clamps, 3 adds,
# 1 compare per pair, one pair a lane) and the MFMA that score them (16x16x32 bf16: 2 per 64
# pairs; 32x32x64 fp8: 1 per 256 pairs)
INDEX_EPILOGUE_PER64 = 8
INDEX_MFMA_PER64 = {"bf16": 2.0, "fp8": 0.25}
SCALE = 1.0 / np.sqrt(128.0)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
_CSRC = "long_context_sparse_topk_amd/csrc/"
KERNEL_SOURCES = {
    "attn_fwd_kernel": [_CSRC + "attn_fwd.hip"],
    "indexer_topk_kernel": [_CSRC + "indexer.hip", _CSRC + "indexer_common.hpp"],
    "indexer32_fp8_kernel": [_CSRC + "indexer_mfma32.hip", _CSRC + "indexer_common.hpp"],
    "sparse_attn_bwd": [_CSRC + "attn_bwd.hip"],   # dq + inverse lists + dk/dv
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work per launch (per-unit figures: see the design notes)


def positions(wl) -> np.ndarray:
    qp = wl.q_positions()
    return np.arange(wl.sq, dtype=np.int64) if qp is None else qp.astype(np.int64)


def work(wl):
    pos = positions(wl)
    nc = (pos + 1) // 4
    part = (pos + 1) % 4
    nkeys = 4 * np.minimum(nc, wl.topk) + part
    H, k = wl.heads, wl.topk
    keys = int(nkeys.sum())
    # (query row, pool) entries of the key sets: selected pools + own incomplete pool
    entries = int((np.minimum(nc, wl.topk) + (part > 0)).sum())
    n_pools = (wl.sk + 3) // 4
    per_q_fwd = 2 * H * 128 * 2 + 4 * H + 4 * k
    # dq pass: q, o, dout read, dq written, lse, idx, the per-(row, head) record
    per_q_dq = 4 * H * 128 * 2 + 4 * H + 4 * k + 16 * H
    # dk/dv pass per entry: q and dout rows, the record, the list entry written and read
    per_entry_kv = 2 * H * 128 * 2 + 16 * H + 8
    return {
        "index_flop": 512 * int(nc.sum()),          # 4 heads x 64 dims x 2 per (query, pool)
        "index_pairs": int(nc.sum()),
        "keys": keys,
        "entries": entries,
        "fwd_bytes": 512 * keys + per_q_fwd * wl.sq,
        # K, V rows gathered per key (dq pass); inverse lists (idx read twice);
        # dk/dv pass entries; per pool K, V read and dK, dV written
        "bwd_bytes": 512 * keys + per_q_dq * wl.sq + 8 * k * wl.sq + per_entry_kv * entries
                     + 4 * 1024 * n_pools,
    }


# ---------------------------------------------------------------------------


class Layer:
    """Inputs, outputs and workspaces of one workload, all resident on the GPU."""

    def __init__(self, wl, device):
        self.wl = wl
        parts = ("index", "attn", "bwd") if wl.backward else ("index", "attn")
        log(f"{wl.name}: generating inputs")
        h = syn.make_inputs(wl, parts=parts)
        self.host = h
        dev = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device)
        self.t = {n: dev(h[n]) for n in parts_names(parts)}
        self.q_pos = None if h["q_pos"] is None else torch.from_numpy(h["q_pos"]).to(device)
        Sq, Sk, H, k = wl.sq, wl.sk, wl.heads, wl.topk
        self.idx = torch.empty((Sq, k), dtype=torch.int32, device=device)
        self.ws_idx = torch.empty(D.index_topk_ws_bytes(Sq, Sk, k, q_chunk=wl.q_chunk), dtype=torch.uint8,
                                  device=device)
        self.out = torch.empty((Sq, H, 128), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((Sq, H), dtype=torch.float32, device=device)
        if wl.backward:
            self.dq = torch.empty_like(self.out)
            self.dk = torch.empty((Sk, 128), dtype=torch.bfloat16, device=device)
            self.dv = torch.empty_like(self.dk)
            self.ws_bwd = torch.empty(D.sparse_attn_bwd_ws_bytes(Sq, Sk, H, k), dtype=torch.uint8,
                                      device=device)
        torch.cuda.synchronize()

    def step(self, ev=None):
        """One step: indexer + top-k and forward pipelined over query chunks (one call), then
        the backward for training workloads.  ev: events around the two parts."""
        t, wl = self.t, self.wl
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        D.index_attn_fwd(t["q_idx"], t["k_idx"], t["w_idx"], t["q"], t["k"], t["v"], topk=wl.topk,
                         q_chunk=wl.q_chunk, q_pos=self.q_pos, scale=SCALE, idx=self.idx, out=self.out,
                         lse=self.lse, ws=self.ws_idx)
        rec(1)
        if wl.backward:
            self.backward()
            rec(2)

    def backward(self):
        t, wl = self.t, self.wl
        D.sparse_attn_bwd(t["q"], t["k"], t["v"], self.out, t["dout"], self.lse, self.idx,
                          q_pos=self.q_pos, scale=SCALE, ws=self.ws_bwd, dq=self.dq, dk=self.dk,
                          dv=self.dv)

    def step_fp8(self):
        """The pipelined call with the fp8 indexer (dsa_index_attn_fwd_fp8)."""
        t, wl = self.t, self.wl
        D.index_attn_fwd(t["q_idx"], t["k_idx"], t["w_idx"], t["q"], t["k"], t["v"], topk=wl.topk,
                         q_chunk=wl.q_chunk, q_pos=self.q_pos, scale=SCALE, idx=self.idx, out=self.out,
                         lse=self.lse, ws=self.ws_idx, fp8=True)

    def index_fp8(self, ev):
        """The fp8 indexer (dsa_index_topk_fp8) as a separate call, with events around it."""
        t, wl = self.t, self.wl
        ev[0].record()
        D.index_topk(t["q_idx"], t["k_idx"], t["w_idx"], topk=wl.topk, q_chunk=wl.q_chunk,
                     q_pos=self.q_pos, out=self.idx, ws=self.ws_idx, fp8=True)
        ev[1].record()

    def index_rows(self, fp8=False):
        """One more (untimed) separate indexer call and its row statistics: rows whose first
        sampled threshold failed (scored again with the wider margin) and rows the exact
        pass scored."""
        t, wl = self.t, self.wl
        D.index_topk(t["q_idx"], t["k_idx"], t["w_idx"], topk=wl.topk, q_chunk=wl.q_chunk,
                     q_pos=self.q_pos, out=self.idx, ws=self.ws_idx, fp8=fp8)
        retried, exact = D.index_topk_stats(self.ws_idx, Sq=wl.sq, Sk=wl.sk, topk=wl.topk)
        return {"retried": retried, "exact_pass": exact, "of": wl.sq}

    def kernels(self, ev):
        """The same work as separate entry-point calls, one after the other on the current
        stream (the stream every kernel of these calls is launched on), with events around
        each: the per-launch durations of the kernels in isolation."""
        t, wl = self.t, self.wl
        ev[0].record()
        D.index_topk(t["q_idx"], t["k_idx"], t["w_idx"], topk=wl.topk, q_chunk=wl.q_chunk,
                     q_pos=self.q_pos, out=self.idx, ws=self.ws_idx)
        ev[1].record()
        D.sparse_attn_fwd(t["q"], t["k"], t["v"], self.idx, q_pos=self.q_pos, scale=SCALE,
                          out=self.out, lse=self.lse)
        ev[2].record()
        if wl.backward:
            self.backward()
            ev[3].record()


def parts_names(parts):
    names = []
    if "index" in parts:
        names += ["q_idx", "k_idx", "w_idx"]
    if "attn" in parts:
        names += ["q", "k", "v"]
    if "bwd" in parts:
        names += ["dout"]
    return names


def run(layer: Layer, steps: int, warmup: int):
    """Time `steps` pipelined steps (wall clock between synchronisations), then the same
    number of passes of the separate calls for per-kernel durations."""
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    bw = layer.wl.backward
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(3 if bw else 2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        layer.step(sev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_parts = {"index_fwd_pipelined": [e[0].elapsed_time(e[1]) / 1e3 for e in sev]}
    if bw:
        step_parts["bwd"] = [e[1].elapsed_time(e[2]) / 1e3 for e in sev]

    layer.kernels([torch.cuda.Event(enable_timing=True) for _ in range(4)])   # warm the pass
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(4 if bw else 3)] for _ in range(steps)]
    for s in range(steps):
        layer.kernels(kev[s])
    torch.cuda.synchronize()
    per = {"index": [e[0].elapsed_time(e[1]) / 1e3 for e in kev],
           "fwd": [e[1].elapsed_time(e[2]) / 1e3 for e in kev]}
    if bw:
        per["bwd"] = [e[2].elapsed_time(e[3]) / 1e3 for e in kev]
    # the step's pipelined call with the fp8 indexer instead (same ids on these inputs)
    layer.step_fp8()
    ev8 = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ts8 = []
    for _ in range(steps):
        ev8[0].record()
        layer.step_fp8()
        ev8[1].record()
        torch.cuda.synchronize()
        ts8.append(ev8[0].elapsed_time(ev8[1]) / 1e3)
    step_parts["index_fwd_pipelined_fp8_indexer"] = ts8
    # the fp8 indexer variant, timed the same way (its ids equal the bf16 path's on these inputs)
    layer.index_fp8([torch.cuda.Event(enable_timing=True) for _ in range(2)])
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for s in range(steps):
        layer.index_fp8(fev[s])
    torch.cuda.synchronize()
    per["index_fp8"] = [e[0].elapsed_time(e[1]) / 1e3 for e in fev]
    avg = {k: float(np.mean(v)) for k, v in per.items()}
    avg_step = {k: float(np.mean(v)) for k, v in step_parts.items()}
    return wall, avg, avg_step


def training_modes(layer: Layer, steps: int, warmup: int):
    """The autograd integration on the same inputs, per mode: ms per step (forward and
    backward, wall clock between synchronisations) and the bytes the layer keeps between
    its forward and its backward beyond its own inputs (device) or in pinned host memory."""
    t, wl = layer.t, layer.wl
    q, k, v = (t[n].detach().requires_grad_(True) for n in ("q", "k", "v"))
    res = {}
    for mode in TR.MODES:
        def step():
            out, _ = TR.sparse_attention(t["q_idx"], t["k_idx"], t["w_idx"], q, k, v, topk=wl.topk,
                                         q_pos=layer.q_pos, scale=SCALE, q_chunk=wl.q_chunk, mode=mode)
            kept = (out.grad_fn.saved_device_bytes, out.grad_fn.saved_host_bytes)
            torch.autograd.grad(out, (q, k, v), t["dout"])
            return kept
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            kept = step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        res[mode] = {"ms_per_step": round(ms, 3), "kept_device_bytes": int(kept[0]),
                     "kept_host_bytes": int(kept[1])}
    return res


def separate_sum(avg: dict) -> float:
    """Seconds of one step run as separate calls (the bf16 indexer, forward and backward; the fp8
    indexer variant is timed beside them, not part of the step)."""
    return sum(v for k, v in avg.items() if k != "index_fp8")


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in list(files) + [_CSRC + "dsa_device.hpp", _CSRC + "dsa_kernels.hpp"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel][workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(layer: Layer, budget_rows: int):
    """The oracle as it stands on a random sample of query rows of the same
    workload (indexer + top-k, forward, and backward dq for training
    workloads); tokens/s = rows / seconds."""
    from oracle import dsa_oracle as O
    wl, h = layer.wl, layer.host
    rng = np.random.default_rng(2024)
    rows = np.sort(rng.choice(wl.sq, size=min(budget_rows, wl.sq), replace=False))
    workers = min(16, os.cpu_count() or 1)
    qp = h["q_pos"]
    t0 = time.perf_counter()
    sel = O.index_topk(h["q_idx"], h["k_idx"], h["w_idx"], qp, wl.topk, rows=rows, workers=workers)
    full = np.zeros((wl.sq, wl.topk), np.int32)
    full[rows] = sel
    O.sparse_attn_fwd(h["q"], h["k"], h["v"], full, qp, SCALE, rows=rows, workers=workers)
    if wl.backward:
        O.sparse_attn_bwd(h["q"], h["k"], h["v"], h["dout"], full, qp, SCALE, rows=rows,
                          key_rows=np.empty(0, np.int64), workers=workers)
    dt = time.perf_counter() - t0
    what = "index+top-k, fwd" + (", bwd (dq)" if wl.backward else "")
    return {"value": rows.shape[0] / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{rows.shape[0]} random query rows of {wl.name} ({what}); "
                      f"{dt:.2f} s wall on {workers} worker processes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="s1m", choices=sorted(syn.WORKLOADS))
    ap.add_argument("--secondary", default="s128k", help="second workload timed in the same run ('' = none)")
    ap.add_argument("--others", default="s4k,s32k,zigzag4",
                    help="further workloads timed in the same run, comma-separated ('' = none)")
    ap.add_argument("--cpu-rows", type=int, default=8192, help="oracle sample size (rows; about 10 s of host work at S = 1M)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for HBM counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the layer's sharding is a design note, not code). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        sys.exit(2)
    D.lib()
    device = torch.device("cuda:0")

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=device)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    wl = syn.WORKLOADS[args.workload]
    layer = Layer(wl, device)
    log(f"{wl.name}: warmup {args.warmup}, timed {args.steps}")
    wall, avg, avg_step = run(layer, args.steps, args.warmup)
    w = work(wl)
    step_s = wall / args.steps
    value = wl.sq / step_s

    # dominant kernel of the step and its roofline
    kern = {
        "indexer_topk_kernel": {"s": avg["index"], "bound": "mfma", "achieved": w["index_flop"] / avg["index"] / 1e12,
                                "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s"},
        "attn_fwd_kernel": {"s": avg["fwd"], "bound": "hbm", "achieved": w["fwd_bytes"] / avg["fwd"] / 1e9,
                            "peak": HBM_PEAK / 1e9, "unit": "GB/s"},
    }
    if wl.backward:
        kern["sparse_attn_bwd"] = {"s": avg["bwd"], "bound": "hbm",
                                   "achieved": w["bwd_bytes"] / avg["bwd"] / 1e9,
                                   "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    dom = max(kern, key=lambda n: kern[n]["s"])
    dk = kern[dom]
    traffic = measured_traffic(dom, wl.name)
    roofline = {"kernel": dom, "bound": dk["bound"], "achieved": round(dk["achieved"], 2), "peak": dk["peak"],
                "unit": dk["unit"], "frac": round(dk["achieved"] / dk["peak"], 4),
                "traffic": traffic, "ms_per_launch": round(dk["s"] * 1e3, 3),
                # inside the pipelined step the kernels share the CUs, so the launch durations come
                # from the pass of separate calls right after the timed steps
                "launches": "separate calls after the timed steps"}
    if traffic is not None and dk["bound"] == "hbm":
        # the measured bytes beyond L2 (the 256 MB MALL serves part of them) per second, against
        # the HBM peak: the algorithmic rate above counts every gathered row, cached or not
        roofline["traffic_frac"] = round(traffic / dk["s"] / HBM_PEAK, 4)
    kernels = {n: {"ms": round(v["s"] * 1e3, 3), "achieved": round(v["achieved"], 2), "unit": v["unit"],
                   "frac": round(v["achieved"] / v["peak"], 4)} for n, v in kern.items()}
    # the indexer beside the dominant kernel (bf16 MFMA-bound), and the fp8 variant (opt-in,
    # dsa_index_topk_fp8) against the fp8 peak and, for comparison, the bf16 one
    ki = kern["indexer_topk_kernel"]
    def valu_view(kind, seconds):
        # the same launch against the VALU issue rate: the minimal VALU stream of the scoring
        # (epilogue + MFMA issue) per second, against VALU_ISSUE_PEAK
        instr = w["index_pairs"] / 64.0 * (INDEX_EPILOGUE_PER64 + INDEX_MFMA_PER64[kind])
        return {"bound": "alu", "achieved": round(instr / seconds / 1e9, 2), "peak": VALU_ISSUE_PEAK / 1e9,
                "unit": "G wave64 VALU instr/s", "frac": round(instr / seconds / VALU_ISSUE_PEAK, 4)}

    roofline["indexer"] = {"kernel": "indexer_topk_kernel", "bound": "mfma", "achieved": round(ki["achieved"], 2),
                           "peak": ki["peak"], "unit": "TFLOP/s", "frac": round(ki["achieved"] / ki["peak"], 4),
                           "traffic": measured_traffic("indexer_topk_kernel", wl.name),
                           "ms_per_launch": round(ki["s"] * 1e3, 3),
                           "valu": valu_view("bf16", avg["index"]),
                           "rows": layer.index_rows()}
    f8 = w["index_flop"] / avg["index_fp8"] / 1e12
    kernels["indexer32_fp8_kernel"] = {"ms": round(avg["index_fp8"] * 1e3, 3), "achieved": round(f8, 2),
                                       "unit": "TFLOP/s", "frac": round(f8 * 1e12 / FP8_PEAK, 4),
                                       "frac_of_bf16_peak": round(f8 * 1e12 / BF16_PEAK, 4),
                                       "traffic": measured_traffic("indexer32_fp8_kernel", wl.name),
                                       "valu": valu_view("fp8", avg["index_fp8"]),
                                       "rows": layer.index_rows(fp8=True)}

    secondary = None
    if args.secondary and args.secondary != wl.name:
        sw = syn.WORKLOADS[args.secondary]
        # device memory of the secondary workload alone: its inputs, outputs and workspaces
        base_mem = torch.cuda.memory_allocated(device)
        torch.cuda.reset_peak_memory_stats(device)
        sl = Layer(sw, device)
        swall, savg, sstep = run(sl, args.steps, args.warmup)
        peak_mem = torch.cuda.max_memory_allocated(device) - base_mem
        sws = work(sw)
        secondary = {"workload": sw.name, "tokens_per_s": round(sw.sq * args.steps / swall, 1),
                     "ms_per_step": round(swall / args.steps * 1e3, 3),
                     "pass": "index+fwd+bwd" if sw.backward else "index+fwd",
                     "ms": {k: round(v * 1e3, 3) for k, v in savg.items()},
                     "step_ms": {k: round(v * 1e3, 3) for k, v in sstep.items()},
                     "separate_calls_ms_per_step": round(separate_sum(savg) * 1e3, 3),
                     "index_mfma_frac": round(sws["index_flop"] / savg["index"] / BF16_PEAK, 4),
                     "index_fp8_mfma_frac": round(sws["index_flop"] / savg["index_fp8"] / FP8_PEAK, 4),
                     "fwd_gather_GBps": round(sws["fwd_bytes"] / savg["fwd"] / 1e9, 1)}
        if sw.backward:
            secondary["bwd_GBps"] = round(sws["bwd_bytes"] / savg["bwd"] / 1e9, 1)
        secondary["peak_mem_bytes"] = int(peak_mem)
        secondary["index_ws_bytes"] = int(sl.ws_idx.numel())
        if sw.backward:
            secondary["bwd_ws_bytes"] = int(sl.ws_bwd.numel())
            log(f"{sw.name}: training modes (autograd)")
            secondary["training"] = training_modes(sl, args.steps, args.warmup)
        del sl

    # the remaining workloads: throughput, the indexer's fraction of the MFMA peak and the
    # attention kernels' algorithmic bytes per second
    others = []
    for name in [n for n in args.others.split(",") if n and n not in (wl.name, args.secondary)]:
        ow = syn.WORKLOADS[name]
        ol = Layer(ow, device)
        owall, oavg, ostep = run(ol, args.steps, args.warmup)
        ows = work(ow)
        rec = {"workload": ow.name, "tokens_per_s": round(ow.sq * args.steps / owall, 1),
               "ms_per_step": round(owall / args.steps * 1e3, 3),
               "pass": "index+fwd+bwd" if ow.backward else "index+fwd",
               "ms": {k: round(v * 1e3, 3) for k, v in oavg.items()},
               "index_mfma_frac": round(ows["index_flop"] / oavg["index"] / BF16_PEAK, 4),
               "index_fp8_mfma_frac": round(ows["index_flop"] / oavg["index_fp8"] / FP8_PEAK, 4),
               # algorithmic bytes per second; K and V of these workloads (8 to 64 MiB) stay in
               # the L2 and the 256 MB MALL, so this is a cache-bandwidth rate, not a fraction
               # of the HBM roofline (it can exceed the HBM peak)
               "fwd_gather_GBps": round(ows["fwd_bytes"] / oavg["fwd"] / 1e9, 1),
               "gather_bound": "cache-resident K/V (no HBM roofline)"}
        if ow.backward:
            rec["bwd_GBps"] = round(ows["bwd_bytes"] / oavg["bwd"] / 1e9, 1)
        others.append(rec)
        del ol

    cpu = None
    if not args.no_cpu_baseline:
        log("oracle CPU baseline")
        cpu = cpu_baseline(layer, args.cpu_rows)
        cpu["value"] = round(cpu["value"], 2)

    line = {
        "metric": "DSA layer tokens/s (indexer + top-k + sparse attention fwd, +bwd when training)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "seq_len": wl.seq, "queries": wl.sq, "heads": wl.heads,
                   "head_dim": 128, "indexer": "4x64", "pool": 4, "topk": wl.topk, "q_chunk": wl.q_chunk,
                   "pass": "index+fwd+bwd" if wl.backward else "index+fwd", "parallelism": "single-gpu"},
        "roofline": roofline,
        "kernels": kernels,
        # the step's parts as timed (indexer and forward pipelined in one call), and the same
        # work as separate calls one after the other (the per-kernel durations above)
        "step_ms": {k: round(v * 1e3, 3) for k, v in avg_step.items()},
        "separate_calls_ms_per_step": round(separate_sum(avg) * 1e3, 3),
        "index_mfma_frac": round(w["index_flop"] / avg["index"] / BF16_PEAK, 4),
        "fwd_gather_GBps": round(w["fwd_bytes"] / avg["fwd"] / 1e9, 1),
        # the same step with the fp8 indexer (dsa_index_attn_fwd_fp8; its ids equal the bf16
        # indexer's on these integer inputs), timed with events around each call
        "fp8_indexer_step": {"ms_per_step": round((avg_step["index_fwd_pipelined_fp8_indexer"]
                                                   + avg_step.get("bwd", 0.0)) * 1e3, 3),
                             "tokens_per_s": round(wl.sq / (avg_step["index_fwd_pipelined_fp8_indexer"]
                                                            + avg_step.get("bwd", 0.0)), 1)},
        "cpu_baseline": cpu,
        "secondary": secondary,
        "others": others,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
