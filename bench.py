#!/usr/bin/env python3
"""Throughput of the absorbed-MLA sparse decode step on one MI355X.

One step = one mla_decode_attn call over the whole batch (selection
compaction + query rotation + W_UK absorption, split-KV attention over the
selected 576-wide cache rows, merge + W_UV up-projection), one query token per
sequence.  Inputs are synthetic (seeded, shaped like the pages' workloads) and
resident in HBM before the timed region; R copies of every input are cycled
so that consecutive steps never find their data in the 256 MB Infinity Cache.
The timed steps are replayed from a HIP graph; HIP events recorded by the
library around each of its kernels give the per-kernel durations.

Prints one JSON line.  Default workload: the ragged batch (B=128, L_b ~
U{1024..16384}, top-k = min(2048, L_b)), the largest of the five.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode attn tokens/s and achieved HBM TB/s (% peak) at B,L,top-k"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES_BF16 = 576 * 2          # one selected cache row: 512 latent + 64 rotary features
DESCR = {
    "tiny": "B=1, H=16, L=65, all positions selected, fp32",
    "page": "B=1, H=128, L=1001 (P=1000 cached + 1), all positions selected, bf16",
    "batched": "B=32, H=128, L=4096, top-k 2048 random incl. newest, bf16",
    "long": "B=64, H=128, L=16384, top-k 2048 random incl. newest, bf16",
    "ragged": "B=128, H=128, L_b~U{1024..16384}, top-k=min(2048,L_b) (half random, half recent), "
              "bf16 caches/queries, fp32 W_UK/W_UV",
}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("mla_attn.hip", "mla_device.hpp"):
        with open(os.path.join(ROOT, "decode_attention_absorbed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current attention kernel source."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(workload)
    if not e or d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


class Hip:
    """The few HIP runtime calls the bench needs for events."""

    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.L.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.L.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on the first sequences of the same workload
    (all heads), until about budget_s seconds of work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    cfg = oracle.RopeConfig(**w.rope)
    n, t0 = 0, time.perf_counter()
    while n < w.B:
        oracle.decode_attention(w.q_nope, w.q_pe, w.w_uk, w.w_uv, w.kv_cache, w.pe_cache, w.topk_indices,
                                w.cache_lens, cfg, form="restricted", batch=[n])
        n += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} of {w.B} sequences of the {w.name} workload, all {w.H} heads, "
                      f"fp64 non-absorbed definition over the selected rows ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ragged", choices=list(DESCR))
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--replicas", type=int, default=0, help="input copies cycled (0 = enough for 1.5 GB)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": src.numel() * 4}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU mode); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    from decode_attention_absorbed_amd import mla

    torch.cuda.set_device(0)
    w = W.workload(args.workload)
    act = torch.bfloat16 if w.dtype_act == "bf16" else torch.float32
    wt = torch.bfloat16 if w.dtype_w == "bf16" else torch.float32
    rows = w.selected_rows()
    kv_bytes = rows * 576 * (2 if w.dtype_act == "bf16" else 4)
    w_bytes = 2 * w.H * 128 * 512 * (2 if w.dtype_w == "bf16" else 4)
    touched = kv_bytes + w_bytes + w.B * w.H * 192 * 2
    R = args.replicas or max(2, math.ceil(1.5e9 / touched))

    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    base = dict(q_nope=dev(w.q_nope, act), q_pe=dev(w.q_pe, act), w_uk=dev(w.w_uk, wt), w_uv=dev(w.w_uv, wt),
                kv_cache=dev(w.kv_cache, act), pe_cache=dev(w.pe_cache, act),
                topk_indices=torch.from_numpy(w.topk_indices).cuda(),
                cache_lens=torch.from_numpy(w.cache_lens).cuda())
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    table = mla.rope_freqs(w.rope)
    scale = mla.softmax_scale(192, w.rope)
    out = torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    nws = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(base["kv_cache"]), mla._dtype_code(base["w_uk"]))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    splits = mla.num_splits(w.B, w.H, w.K, mla._dtype_code(base["kv_cache"]))

    hip = Hip()
    K = args.steps
    events = [[hip.event() for _ in range(2 * mla.MLA_NUM_KERNELS)] for _ in range(K)]
    ev_arrays = [(ctypes.c_void_p * len(e))(*[x.value for x in e]) for e in events]

    def params(i, with_events):
        r = reps[i % R]
        p = mla.build_params(r["q_nope"], r["q_pe"], r["w_uk"], r["w_uv"], r["kv_cache"], r["pe_cache"],
                             r["topk_indices"], r["cache_lens"], table, scale, out, lse, ws)
        if with_events:
            p.profile_events = ctypes.cast(ev_arrays[i], ctypes.c_void_p)
        return p

    plain = [params(i, False) for i in range(R)]
    timed = [params(i, True) for i in range(K)]

    for i in range(args.warmup):
        mla.decode_attn(plain[i % R])
    torch.cuda.synchronize()

    # Per-kernel durations: K eager steps with HIP events recorded by the
    # library around each of its kernels on the launch stream.
    for i in range(K):
        mla.decode_attn(timed[i])
    torch.cuda.synchronize()
    eager_ms = None
    graph = None
    if not args.no_graph:
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(K):
                mla.decode_attn(plain[i % R])
        graph.replay()                      # upload + one untimed pass
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            mla.decode_attn(plain[i % R])
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - t0) * 1e3 / K

    # Timed region: K steps (graph replay, or eager launches with --no-graph).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(K):
            mla.decode_attn(timed[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    per_kernel = {}
    for k, name in enumerate(mla.KERNEL_NAMES):
        per_kernel[name] = float(np.mean([hip.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in events]))
    ms_step = elapsed * 1e3 / K
    t_attn_s = per_kernel["attention"] * 1e-3
    achieved = rows * ROW_BYTES_BF16 / t_attn_s / 1e9 if w.dtype_act == "bf16" else kv_bytes / t_attn_s / 1e9
    flops = 2.0 * w.H * (576 + 512) * rows + 4.0 * w.B * w.H * 128 * 512
    tr = measured_traffic(args.workload)
    line = {
        "metric": METRIC,
        "value": w.B * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype_act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {DESCR[args.workload]}", "B": w.B, "H": w.H,
                   "L_max": w.L_max, "top_k": w.K, "selected_rows": rows, "num_splits": splits,
                   "input_replicas": R, "hip_graph": graph is not None},
        "eager_ms_per_step": eager_ms,
        "hbm_tb_s_step": kv_bytes / (ms_step * 1e-3) / 1e12,
        "hbm_pct_peak_step": kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "mfma_tflops_step": flops / (ms_step * 1e-3) / 1e12,
        "kernel_ms": per_kernel,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": tr,
                     "kernel": "attention", "algorithmic_bytes": rows * ROW_BYTES_BF16,
                     "mfma_tflops": 2.0 * w.H * (576 + 512) * rows / t_attn_s / 1e12},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
