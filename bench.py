#!/usr/bin/env python3
"""Benchmark of the fused attention training op on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
forward (O, LSE) -> preprocess (Delta) -> backward (dQ, dK, dV), back to back on
one stream, through the C ABI. Inputs are resident in HBM before timing starts.

The headline line is the DiT self-attention workload (B=1, Hq=16, Hkv=8,
S=1542, D=128, bf16, pad mask): mask-adjusted fwd+bwd TFLOP/s (14 * D * N FLOPs
per step, N = unmasked score pairs). Other workloads are reported under "extra".

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload dit_sa]
                    [--extra lm_causal,dit_ca,long_window,dit_sa_len,dit_sa_band,lm_sinks,lm_alibi,lm_softcap,long_window_q8,long_window_f16]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

METRIC = "attention fwd+bwd TFLOP/s (mask-adjusted) and % of MI355X bf16 MFMA peak"


# the other workloads timed by default, beside the headline one
DEFAULT_EXTRA = ("lm_causal", "dit_ca", "long_window", "dit_sa_len", "dit_sa_band", "lm_sinks", "lm_alibi",
                 "lm_softcap", "long_window_q8", "long_window_f16")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dit_sa")
    ap.add_argument("--extra", default=",".join(DEFAULT_EXTRA),
                    help="other workloads to time, comma separated ('none' for none); long_window is the "
                         "64-chunk walk over a 32768-long window")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--splits", default="table",
                    help="backward split: 'table' (the workload's measured setting), 'tune' (time a few settings "
                         "once at setup, untimed), 'model' (the library's cost model), KVxQ (e.g. 2x1) or KVxQxTILES "
                         "(q-way split of the first TILES 128-row query tiles only, e.g. 2x2x6)")
    ap.add_argument("--kv-walk", type=int, default=0,
                    help="bf16 backward dK/dV walk: 0 the library's choice, 1 one wave per 32 keys, 2 split by role")
    ap.add_argument("--dq-launch", type=int, default=-1,
                    help="bf16 backward dQ: -1 the workload table's setting, 0 the library's choice, 1 / 2 the dQ "
                         "walk in the dK/dV launch / its own, 3 dQ from stored dS")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference kernel that "
                         "scales the HBM byte counters) and exit")
    return ap.parse_args()


class Workload:
    """Device buffers and the three calls of one step for a seeded case."""

    def __init__(self, key: str, splits: str = "table", kv_walk: int = 0, dq_launch: int = -1):
        import torch

        from flash_attention_train_amd import accounting, binding, configs
        self.key = key
        self.kv_walk = kv_walk
        self.dq_launch = configs.WORKLOADS[key].bwd_dq_launch if dq_launch < 0 else dq_launch
        self.case = c = configs.make(key)
        self.pairs = accounting.case_pairs(c)
        self.fwd_flops = accounting.fwd_flops(self.pairs, c.D)
        self.bwd_flops = accounting.bwd_flops(self.pairs, c.D)
        self.pre_bytes = accounting.preprocess_bytes(c.B, c.Hq, c.Sq, c.D, c.dtype)
        self.step_bytes = accounting.step_bytes(c)
        dev = "cuda"

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.q, self.k, self.v, self.do = up(c.q), up(c.k), up(c.v), up(c.do)
        self.mask = None if c.mask is None else torch.from_numpy(c.mask).to(dev)
        # a structured mask (key / query lengths as device arrays, a window): given to every call
        st = c.meta.get("structure")
        self.sk = {}
        if st is not None:
            for n in ("key_len", "q_len"):
                self.sk[n] = None if st[n] is None else torch.tensor(st[n], dtype=torch.int32, device=dev)
            self.sk["window"] = tuple(st["window"])
        # attention sinks (per-head logits): given to the forward; the step adds their gradient
        self.sinks = None if c.meta.get("sinks") is None else torch.from_numpy(c.meta["sinks"]).to(dev)
        self.dsink = None if self.sinks is None else torch.zeros_like(self.sinks)
        # ALiBi slopes (per head), given to the forward and the backward
        self.alibi = None if c.meta.get("alibi") is None else torch.from_numpy(c.meta["alibi"]).to(dev)
        # a logit softcap, given to the forward and the backward (0 = none)
        self.softcap = float(c.meta.get("softcap", 0.0))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(c.B, c.Hq, c.Sq, dtype=torch.float32, device=dev)
        self.delta = torch.empty_like(self.lse)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.k)
        self.dv = torch.empty_like(self.v)
        self.B = binding
        self.tiles = None
        if self.mask is not None:
            self.tiles = binding.mask_tile_map(self.mask, self.q, self.k)  # sized once, refilled every step
        # forward workspace: the split-key walk's partial rows when the grid is short
        self.fws_bytes = binding.fwd_workspace_bytes(self.q, self.k, scale=c.scale, causal=c.causal,
                                                     q_offset=c.q_offset, mask=self.mask, softcap=self.softcap,
                                                     **self.sk)
        self.fws = torch.empty(max(self.fws_bytes, 256), dtype=torch.uint8, device=dev)
        # the split the library chose: its workspace holds splits * B * Hq * Sq * (2 D + 8) bytes,
        # rounded up to 256
        self.fwd_split = self.fws_bytes // (c.B * c.Hq * c.Sq * (2 * c.D + 8)) if self.fws_bytes else 1
        # backward split: the library's cost model, or (tune) the fastest of a few
        # settings timed once here on this workload, outside every timed region
        self.kv_split = self.q_split = self.q_split_tiles = 0
        self.splits_from = "library cost model"
        if splits == "table" and configs.WORKLOADS[key].bwd_splits:
            self.kv_split, self.q_split, self.q_split_tiles = configs.WORKLOADS[key].bwd_splits
            self.splits_from = "workload table"
        elif "x" in splits:  # KVxQ or KVxQxTILES
            v = [int(x) for x in splits.split("x")]
            self.kv_split, self.q_split = v[0], v[1]
            self.q_split_tiles = v[2] if len(v) > 2 else 0
            self.splits_from = "given"
        elif splits == "tune":
            self.splits_from = "tuned once at setup"
            self.fwd()
            self.pre()
            self.kv_split, self.q_split = binding.tune_bwd_splits(
                self.q, self.k, self.v, self.do, self.lse, self.delta, mask=self.mask, scale=c.scale,
                causal=c.causal, q_offset=c.q_offset, mask_tiles=self.tiles, **self.sk)
        nws = binding.bwd_workspace_bytes(self.q, self.k, scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                                          mask=self.mask, kv_split=self.kv_split, q_split=self.q_split,
                                          q_split_tiles=self.q_split_tiles, softcap=self.softcap,
                                          dq_launch=self.dq_launch, **self.sk)
        self.ws_bytes = nws
        self.ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)

    def classify(self):
        """The mask tile map (dead / open / mixed 64 x 64 blocks), part of every step
        that has a dense mask."""
        if self.mask is not None:
            self.B.mask_tile_map(self.mask, self.q, self.k, out=self.tiles)

    def fwd(self):
        c = self.case
        self.B.fwd(self.q, self.k, self.v, mask=self.mask, scale=c.scale, causal=c.causal, q_offset=c.q_offset,
                   out=self.o, lse=self.lse, mask_tiles=self.tiles, workspace=self.fws, sinks=self.sinks,
                   alibi=self.alibi, softcap=self.softcap, **self.sk)

    def pre(self):
        self.B.bwd_preprocess(self.o, self.do, delta=self.delta)

    def bwd(self):
        c = self.case
        self.B.bwd(self.q, self.k, self.v, self.do, self.lse, self.delta, mask=self.mask, scale=c.scale,
                   causal=c.causal, q_offset=c.q_offset, dq=self.dq, dk=self.dk, dv=self.dv, workspace=self.ws,
                   kv_split=self.kv_split, q_split=self.q_split, q_split_tiles=self.q_split_tiles,
                   mask_tiles=self.tiles, alibi=self.alibi, softcap=self.softcap, kv_walk=self.kv_walk,
                   dq_launch=self.dq_launch, **self.sk)
        if self.sinks is not None:  # the sinks' gradient, added into their accumulator
            self.B.bwd_sinks(self.lse, self.delta, self.sinks, dsink=self.dsink)

    def step(self):
        self.classify()
        self.fwd()
        self.pre()
        self.bwd()


def time_graph(w: Workload, steps: int, warmup: int) -> dict:
    """Captures one whole step (mask map, forward, preprocess, backward: the same launches
    as the eager step) in a HIP graph and times `steps` replays between synchronizes
    (`ms`: wall clock over all of them), each replay also bracketed by HIP events on the
    replay stream (`median_ms`, `min_ms`). The graph removes the host's per-launch cost,
    which a training loop that captures its attention layer does not pay either."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w.step()  # one eager step on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        w.step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    return {"ms": ms, "median_ms": float(np.median(per)), "min_ms": float(per.min())}


def time_workload(w: Workload, steps: int, warmup: int, graph: bool = True) -> dict:
    """Times `steps` whole eager steps (wall clock around synchronizes) and, inside the
    same timed region, each call with HIP events on the stream it is launched on; then
    (graph=True) the same step replayed from a captured graph."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        w.step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        w.classify()
        w.fwd()
        e[1].record(stream)
        w.pre()
        e[2].record(stream)
        w.bwd()
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    pre_ms = np.array([e[1].elapsed_time(e[2]) for e in ev])
    bwd_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])
    eager_ms = wall * 1e3 / steps
    g = time_graph(w, steps, warmup) if graph else {"ms": eager_ms, "median_ms": eager_ms, "min_ms": eager_ms}
    step_ms = g["ms"]
    total_flops = w.fwd_flops + w.bwd_flops
    return {
        "ms_per_step": step_ms,
        "step_ms_median": g["median_ms"], "step_ms_min": g["min_ms"],
        "tflops_at_median": total_flops / (g["median_ms"] * 1e-3) / 1e12,
        "timing": "hip graph replay of the whole step" if graph else "eager launches",
        "eager_ms_per_step": eager_ms,
        "eager_tflops": total_flops / (eager_ms * 1e-3) / 1e12,
        "tflops": total_flops / (step_ms * 1e-3) / 1e12,
        "fwd_ms_mean": float(fwd_ms.mean()), "pre_ms_mean": float(pre_ms.mean()), "bwd_ms_mean": float(bwd_ms.mean()),
        "fwd_ms_median": float(np.median(fwd_ms)), "bwd_ms_median": float(np.median(bwd_ms)),
        "fwd_tflops": w.fwd_flops / (fwd_ms.mean() * 1e-3) / 1e12,
        "bwd_tflops": w.bwd_flops / (bwd_ms.mean() * 1e-3) / 1e12,
        "fwdbwd_event_tflops": total_flops / ((fwd_ms + pre_ms + bwd_ms).mean() * 1e-3) / 1e12,
        "pre_gbs": w.pre_bytes / (pre_ms.mean() * 1e-3) / 1e9,
        "pre_hbm_frac": w.pre_bytes / (pre_ms.mean() * 1e-3) / 1e9 / 8000.0,
        "step_bytes": w.step_bytes,
        "step_hbm_frac": w.step_bytes / (step_ms * 1e-3) / 8e12,
        "pairs": w.pairs,
        "fwd_split": w.fwd_split,
        "bwd_splits": [w.kv_split, w.q_split, w.q_split_tiles],
        "bwd_splits_from": w.splits_from,
        "bwd_dq_launch": w.dq_launch,
        "gflop_per_step": total_flops / 1e9,
    }


def time_long_window(steps: int, warmup: int, key: str = "long_window") -> dict:
    """The long-window exact walk at full size: 64 query chunks of 512 rows over a
    32768-long cached K/V window, each chunk forward -> preprocess -> chunked backward
    (dK/dV added into fp32 window accumulators, zeroed at the start of the walk). The
    whole walk (192 launches) is captured in one HIP graph and replayed; FLOPs are the
    walk's exact causal pairs, which equal the one-shot causal run's. With
    key = "long_window_q8" (or "long_window_f16") the window is stored as q8_0 (fp16) and
    read in place: the kernels convert each K / V tile to bf16 as they load it, and no
    bf16 copy of the window exists."""
    import torch

    from flash_attention_train_amd import accounting, binding, configs
    W, C = configs.LONG_WINDOW, configs.LONG_CHUNK
    c = configs.make(key)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")

    q, do = up(c.q), up(c.do)
    q8, f16 = c.meta.get("q8"), c.meta.get("f16")
    sc = {}  # the q8_0 scale planes
    if q8 is not None:  # the window as stored: int8 quants and their fp16 scales
        k, sc["k_scale"] = (torch.from_numpy(a).to("cuda") for a in q8["k"])
        v, sc["v_scale"] = (torch.from_numpy(a).to("cuda") for a in q8["v"])
    elif f16 is not None:
        k, v = (torch.from_numpy(f16[n]).to("cuda") for n in ("k", "v"))
    else:
        k, v = up(c.k), up(c.v)
    dk_acc = torch.zeros((1, c.Hkv, W, c.D), dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    O, dQ = torch.empty_like(q), torch.empty_like(q)
    LSE = torch.empty((1, c.Hq, W), dtype=torch.float32, device="cuda")
    Delta = torch.empty_like(LSE)
    plan = configs.chunk_plan(W, C)

    def window(sk):  # the K / V rows (and q8_0 scales) the chunk sees
        return k[:, :, :sk], v[:, :, :sk], {n: x[:, :, :sk] for n, x in sc.items()}

    need = max(binding.bwd_workspace_bytes(q[:, :, p0:p0 + n], window(sk)[0], scale=c.scale, causal=True,
                                           q_offset=p0, **window(sk)[2]) for p0, n, sk in plan)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    fneed = max(binding.fwd_workspace_bytes(q[:, :, p0:p0 + n], window(sk)[0], scale=c.scale, causal=True,
                                            q_offset=p0, **window(sk)[2]) for p0, n, sk in plan)
    fws = torch.empty(max(fneed, 256), dtype=torch.uint8, device="cuda")

    def walk():
        dk_acc.zero_()
        dv_acc.zero_()
        for p0, n, sk in plan:
            qc, doc = q[:, :, p0:p0 + n], do[:, :, p0:p0 + n]
            kc, vc, skw = window(sk)
            binding.fwd(qc, kc, vc, scale=c.scale, causal=True, q_offset=p0, out=O[:, :, p0:p0 + n],
                        lse=LSE[:, :, p0:p0 + n], workspace=fws, **skw)
            binding.bwd_preprocess(O[:, :, p0:p0 + n], doc, delta=Delta[:, :, p0:p0 + n])
            binding.bwd_chunked(qc, kc, vc, doc, LSE[:, :, p0:p0 + n], Delta[:, :, p0:p0 + n], dk_acc, dv_acc,
                                scale=c.scale, causal=True, q_offset=p0, dq=dQ[:, :, p0:p0 + n], workspace=ws,
                                **skw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        walk()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        walk()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    pairs = accounting.chunked_pairs(c.Hq, W, C)
    flops = accounting.fwd_flops(pairs, c.D) + accounting.bwd_flops(pairs, c.D)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"ms_per_walk": ms, "tflops": tflops, "pct_of_peak": 100.0 * tflops / accounting.MI355X_BF16_DENSE_TFLOPS,
            "chunks": len(plan), "pairs": pairs, "gflop_per_walk": flops / 1e9,
            "timing": "hip graph replay of the whole 64-chunk walk"}


KERNEL_SOURCES = ("flash_attention_train_amd/csrc/fa_bwd_bf16.hip", "flash_attention_train_amd/csrc/fa_device.h",
                  "flash_attention_train_amd/csrc/fa_kernels.h", "flash_attention_train_amd/csrc/fa_tile.h")


def source_digest(paths=KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, splits, dq_launch: int = 0):
    """HBM bytes per backward call from the committed counter summary, or None when
    there is none for this workload, split and dQ formation, or the kernel source changed since."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic_bwd.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("source_sha256") != source_digest() or entry.get("bwd_splits") != list(splits) or \
            entry.get("bwd_dq_launch", 0) != dq_launch:
        return None
    return entry.get("hbm_bytes_per_launch")


def copy_calibration(mib: int):
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": mib << 20, "launches": 5}), flush=True)


def cpu_baseline(key: str, min_seconds: float = 10.0, max_reps: int = 8) -> dict:
    """The oracle as it stands (fp64 C, all host cores) on whole steps of the workload
    (fwd + bwd), repeated until about `min_seconds` of CPU work: mask-adjusted FLOPs
    per second."""
    import oracle
    from flash_attention_train_amd import accounting, configs
    c = configs.make(key)
    threads = oracle.default_threads()
    m = None if c.mask is None else c.mask.astype(np.float64)
    args = (c.f64("q"), c.f64("k"), c.f64("v"), c.f64("do"), m)
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        oracle.backward(*args, scale=c.scale, causal=c.causal, q_offset=c.q_offset, threads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    # the forward alone (O and LSE), timed the same way over a shorter budget
    freps, fdt = 0, 0.0
    while freps < max_reps and (freps == 0 or fdt < min_seconds / 3):
        t0 = time.perf_counter()
        oracle.forward(*args[:3], args[4], scale=c.scale, causal=c.causal, q_offset=c.q_offset, threads=threads)
        fdt += time.perf_counter() - t0
        freps += 1
    n = accounting.case_pairs(c)
    flops = reps * (accounting.fwd_flops(n, c.D) + accounting.bwd_flops(n, c.D))
    cpu = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} whole fwd+bwd step(s) of the {key} workload (all heads), float64, {dt:.1f} s; "
                      f"forward alone: {freps} call(s), {fdt:.1f} s",
            "seconds": dt, "fwd_value": freps * accounting.fwd_flops(n, c.D) / fdt / 1e12,
            "fwd_seconds": fdt, "cpu": cpu}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the op and its measurement are single-device "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch

    from flash_attention_train_amd import accounting, binding, configs
    binding.lib()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    log(f"[bench] device {torch.cuda.get_device_name(0)}; workload {args.workload}")
    w = Workload(args.workload, args.splits, args.kv_walk, args.dq_launch)
    r = time_workload(w, args.steps, args.warmup, graph=not args.eager)
    log(f"[bench] {args.workload}: {r['ms_per_step']:.3f} ms/step, {r['tflops']:.1f} TFLOP/s")

    extra = {}
    for key in [k for k in args.extra.split(",") if k and k not in (args.workload, "none")]:
        if key in ("long_window", "long_window_q8", "long_window_f16"):
            extra[key] = time_long_window(max(2, args.steps // 8), 1, key)
            log(f"[bench] {key}: {extra[key]['ms_per_walk']:.2f} ms/walk, {extra[key]['tflops']:.1f} TFLOP/s")
            torch.cuda.empty_cache()
            continue
        we = Workload(key, args.splits if "x" not in args.splits else "table", args.kv_walk, args.dq_launch)
        re_ = time_workload(we, max(5, args.steps // 2), args.warmup, graph=not args.eager)
        re_["pct_of_peak"] = 100.0 * re_["tflops"] / accounting.MI355X_BF16_DENSE_TFLOPS
        # near the ridge (few keys per row): the step against the HBM roofline as well
        re_["hbm_roofline"] = {"bytes_per_step": we.step_bytes, "achieved_gbs": we.step_bytes / (re_["ms_per_step"] * 1e-3) / 1e9,
                               "peak_gbs": accounting.MI355X_HBM_GBS,
                               "frac": we.step_bytes / (re_["ms_per_step"] * 1e-3) / 1e9 / accounting.MI355X_HBM_GBS}
        extra[key] = re_
        log(f"[bench] {key}: {re_['ms_per_step']:.3f} ms/step, {re_['tflops']:.1f} TFLOP/s")
        del we
        torch.cuda.empty_cache()

    peak = accounting.MI355X_BF16_DENSE_TFLOPS
    # the backward call is one kernel launch when it needs no workspace; split walks add
    # the reduce passes over their fp32 slices, timed with it (the same events)
    single = w.ws_bytes == 0
    achieved = r["bwd_tflops"]
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs shaped like the workload; no datasets or weights)",
        "config": {"workload": configs.WORKLOADS[args.workload].title, "global_batch": w.case.B,
                   "seq_len": w.case.Sq, "unmasked_pairs": w.pairs, "gflop_per_step": round(r["gflop_per_step"], 3)},
        "pct_of_peak": round(100.0 * r["tflops"] / peak, 2),
        "roofline": {"kernel": "bwd_bf16_kernel (fa_train_bwd)" if single else
                     "fa_train_bwd (its dK/dV walk, dQ walk or pass, and reduce passes)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(args.workload, [w.kv_split, w.q_split, w.q_split_tiles], w.dq_launch),
                     "flop_per_launch": w.bwd_flops, "launch_ms": round(r["bwd_ms_mean"], 5)},
        "breakdown": {k: round(v, 4) if isinstance(v, float) else v for k, v in r.items()},
        "extra": extra,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the host cores ...")
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
