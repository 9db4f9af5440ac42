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
SETTLE_STEPS = 250                # untimed steps (~30 ms) before the per-kernel event loop
PREROLL_S = 0.03                  # untimed graph replays right before the timed region
DESCR = {
    "tiny": "B=1, H=16, L=65, all positions selected, fp32",
    "page": "B=1, H=128, L=1001 (P=1000 cached + 1), all positions selected, bf16",
    "batched": "B=32, H=128, L=4096, top-k 2048 random incl. newest, bf16",
    "long": "B=64, H=128, L=16384, top-k 2048 random incl. newest, bf16",
    "ragged": "B=128, H=128, L_b~U{1024..16384}, top-k=min(2048,L_b) (half random, half recent), "
              "bf16 caches/queries, fp32 W_UK/W_UV",
    "ragged_h16": "the ragged batch at a 16-head shard: B=128, H=16, L_b~U{1024..16384}, "
                  "top-k=min(2048,L_b) (half random, half recent), bf16 caches/queries, fp32 W_UK/W_UV",
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


def op_traffic(name, sources):
    """HBM bytes per launch of an adjacent kernel from the committed counter
    summary, if it was taken on the current source of that kernel."""
    path = os.path.join(ROOT, "profiles", "ops_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        e = json.load(f).get(name)
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(ROOT, "decode_attention_absorbed_amd", "csrc", src), "rb") as fh:
            h.update(fh.read())
    if not e or e.get("source_hash") != h.hexdigest()[:16]:
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


def _host_info():
    """CPU model and the BLAS library numpy runs on (for the baseline record)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, blas


def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on the first sequences of the same workload
    (all heads), until about budget_s seconds of work.  Its thread pool is
    set to every core this process may run on (sched_getaffinity).  Returns
    the baseline record and the oracle's outputs for the sequences it did."""
    import numpy as np
    import oracle
    import contextlib
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limiter = contextlib.nullcontext()
    model, blas = _host_info()
    cfg = oracle.RopeConfig(**w.rope)
    outs, lses = [], []
    with limiter:
        n, t0 = 0, time.perf_counter()
        while n < w.B:
            o, l = oracle.decode_attention(w.q_nope, w.q_pe, w.w_uk, w.w_uv, w.kv_cache, w.pe_cache,
                                           w.topk_indices, w.cache_lens, cfg, form="restricted", batch=[n])
            outs.append(o[0])
            lses.append(l[0])
            n += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
    rec = {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"first {n} of {w.B} sequences of the {w.name} workload, all {w.H} heads, "
                     f"fp64 non-absorbed definition over the selected rows ({dt:.1f} s)",
           "cpu_model": model, "blas": blas}
    return rec, np.array(outs), np.array(lses)


def parity_record(out, lse, ref, ref_lse):
    """Per-row relative L2 error of the step's output against the oracle
    (rows = (sequence, head) output vectors) and the largest |dLSE|."""
    import numpy as np
    n = ref.shape[0]
    got = np.asarray(out[:n], dtype=np.float64)
    err = np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
    dl = np.abs(np.asarray(lse[:n], dtype=np.float64) - ref_lse)
    return {"max_rel_l2": float(err.max()), "p99_rel_l2": float(np.percentile(err, 99)),
            "median_rel_l2": float(np.median(err)), "max_dlse": float(dl.max()),
            "rows": int(err.size), "sequences": int(n), "tol": 1e-2}


def stream_copy_gbs(nbytes=1 << 30, reps=10):
    """Measured device-to-device copy rate (GB/s, bytes read + written),
    the achievable ceiling beside the 8 TB/s peak."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    rate = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return rate


def _timed_launches(fn, K, warmup):
    """Average duration (ms) of fn() over K launches, from HIP events on the
    launching stream (torch's current stream), after warmup launches."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / K
    return sum(a.elapsed_time(b) for a, b in ev) / K, wall


def bench_op(args):
    """One JSON line for one of the adjacent entry points (not the decode
    step): top-k selection, rotary apply, or the decode step with the fused
    append switched on."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    from decode_attention_absorbed_amd import mla

    torch.cuda.set_device(0)
    K, warm = args.steps, args.warmup
    rng = np.random.default_rng(2024)
    line = {"n_gpus": 1, "steps": K, "warmup": warm, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "data": "synthetic"}
    if args.op == "topk":
        # the long-context indexer output: 64 sequences x 16384 scores, k = 2048
        B, L, k = 64, 16384, 2048
        scores_np = rng.standard_normal((B, L)).astype(np.float32)
        reps = [torch.from_numpy(scores_np).cuda() for _ in range(8)]
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        outs = torch.empty((B, k), dtype=torch.int32, device="cuda")
        it = [0]

        def fn():
            mla.topk(reps[it[0] % 8], lens, k, out=outs)
            it[0] += 1
        ms, wall = _timed_launches(fn, K, warm)
        nbytes = B * L * 4 + B * k * 4
        t0, n = time.perf_counter(), 0
        while n < B and time.perf_counter() - t0 < args.cpu_budget:
            oracle.topk_select(scores_np[n].astype(np.float64), L, k)
            n += 1
        cpu = {"value": n / (time.perf_counter() - t0), "unit": "sequences/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} of {B} score rows"}
        line.update(metric="top-k selection sequences/s", value=B / (ms * 1e-3), unit="sequences/s",
                    ms_per_step=ms, wall_ms_per_launch=wall, dtype="f32",
                    config={"workload": f"top-k: B={B} rows of L={L} fp32 scores, k={k}"},
                    roofline={"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "traffic": op_traffic("topk", ["mla_topk.hip", "mla_device.hpp"]),
                              "kernel": "topk_reg_kernel<16>", "algorithmic_bytes": nbytes},
                    cpu_baseline=cpu)
    elif args.op == "rope":
        # a prefill chunk of 16384 tokens at positions 0..16383, 64 heads of
        # 64 rotary features each (the indexer's query shape), bf16
        T, Hh = 16384, 64
        N = T * Hh
        table = mla.rope_freqs(W.ROPE_YARN)
        xs = [torch.from_numpy(rng.standard_normal((T, Hh, 64)).astype(np.float32)).cuda().to(torch.bfloat16)
              for _ in range(2)]
        pos = torch.arange(T, dtype=torch.int32, device="cuda")
        ys = [torch.empty_like(x) for x in xs]
        it = [0]

        def fn():
            i = it[0] % 2
            mla.rope_apply(xs[i], pos, table, args.rope_layout == "interleaved", out=ys[i])
            it[0] += 1
        ms, wall = _timed_launches(fn, K, warm)
        # read + write every vector; the table row (256 B) and position of each token once
        nbytes = N * 64 * 2 * 2 + T * (256 + 4)
        xc = xs[0].reshape(N, 64)[:4096].float().cpu().numpy().astype(np.float64)
        pc = np.repeat(np.arange(T), Hh)[:4096]
        f = oracle.rope_rotate if args.rope_layout == "interleaved" else oracle.rope_rotate_halves
        cfg = oracle.RopeConfig(**W.ROPE_YARN)
        t0, n = time.perf_counter(), 0
        while n < 4096 and time.perf_counter() - t0 < args.cpu_budget:
            f(xc[n], int(pc[n]), cfg)
            n += 1
        cpu = {"value": n / (time.perf_counter() - t0), "unit": "vectors/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n} vectors"}
        line.update(metric="rotary apply vectors/s", value=N / (ms * 1e-3), unit="vectors/s", ms_per_step=ms,
                    wall_ms_per_launch=wall, dtype="bf16",
                    config={"workload": f"rope: {T} tokens x {Hh} heads of 64 bf16 features at positions "
                                        f"0..{T - 1}, {args.rope_layout} layout"},
                    roofline={"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                              "traffic": op_traffic("rope_" + args.rope_layout, ["mla_rope.hip", "mla_device.hpp"]),
                              "kernel": "rope_apply_kernel<bf16>", "algorithmic_bytes": nbytes},
                    cpu_baseline=cpu)
    else:
        # the decode step on the ragged batch, with and without the fused append
        w = W.workload("ragged")
        dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
        act, wt = torch.bfloat16, torch.float32
        t = dict(q_nope=dev(w.q_nope, act), q_pe=dev(w.q_pe, act), w_uk=dev(w.w_uk, wt), w_uv=dev(w.w_uv, wt),
                 kv=dev(w.kv_cache, act), pe=dev(w.pe_cache, act))
        idx = torch.from_numpy(w.topk_indices).cuda()
        lens = torch.from_numpy(w.cache_lens).cuda()
        kv_new, pe_new = (dev(a, act) for a in W.new_rows(w.B, "bf16", 2025))
        table = mla.rope_freqs(w.rope)
        scale = mla.softmax_scale(192, w.rope)
        out = torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
        ws = torch.empty(mla.workspace_size(w.B, w.H, w.K, 1, 0), dtype=torch.uint8, device="cuda")
        ps = {name: mla.build_params(t["q_nope"], t["q_pe"], t["w_uk"], t["w_uv"], t["kv"], t["pe"], idx, lens,
                                     table, scale, out, lse, ws, **extra)
              for name, extra in (("off", {}), ("on", dict(kv_new=kv_new, pe_new=pe_new)))}
        # the two modes alternate in rounds so that neither runs colder
        res = {"off": [], "on": []}
        for _ in range(4):
            for name, p in ps.items():
                res[name].append(_timed_launches(lambda: mla.decode_attn(p), max(K // 4, 1), warm)[0])
        res = {k: float(np.mean(v)) for k, v in res.items()}
        line.update(metric="MLA decode step with fused cache append, tokens/s", value=w.B / (res["on"] * 1e-3),
                    unit="tokens/s", ms_per_step=res["on"], ms_per_step_without_append=res["off"], dtype="bf16",
                    config={"workload": "ragged decode step (B=128, H=128, L_b~U{1024..16384}, top-k 2048) "
                                        "plus the append of one row per sequence",
                            "inputs_resident": "one copy (L2 / Infinity Cache may hold part of it)"})
    print(json.dumps(line), flush=True)


def bench_ab(args):
    """Same-process comparison of builds of the library (--ab LIB [LIB ...]):
    each build runs the workload's step on the same inputs, with its own
    workspace and outputs; its output on the first replica is compared with
    the first build's, then rounds of eager steps alternate the builds'
    order, and HIP events recorded by each build around its kernels give
    their mean durations.  Listing one build twice gives the A/A spread.
    Prints one JSON line."""
    import numpy as np
    import torch
    import workloads as W
    from decode_attention_absorbed_amd import mla

    torch.cuda.set_device(0)
    w = W.workload(args.workload)
    act = torch.bfloat16 if w.dtype_act == "bf16" else torch.float32
    wt = torch.bfloat16 if w.dtype_w == "bf16" else torch.float32
    R = 4
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    base = dict(q_nope=dev(w.q_nope, act), q_pe=dev(w.q_pe, act), w_uk=dev(w.w_uk, wt), w_uv=dev(w.w_uv, wt),
                kv_cache=dev(w.kv_cache, act), pe_cache=dev(w.pe_cache, act),
                topk_indices=torch.from_numpy(w.topk_indices).cuda(),
                cache_lens=torch.from_numpy(w.cache_lens).cuda())
    reps = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(R - 1)]
    table = mla.rope_freqs(w.rope)
    scale = mla.softmax_scale(192, w.rope)
    hip = Hip()
    N = 30                                            # event-timed steps per build per round
    nk = mla.MLA_NUM_KERNELS
    events = [[hip.event() for _ in range(2 * nk)] for _ in range(N)]
    ev_arrays = [(ctypes.c_void_p * len(e))(*[x.value for x in e]) for e in events]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    builds = []
    for path in args.ab:
        L = ctypes.CDLL(os.path.abspath(path))
        L.mla_decode_attn.argtypes = [ctypes.POINTER(mla.DecodeParams), ctypes.c_void_p]
        L.mla_decode_attn.restype = ctypes.c_int
        L.mla_decode_workspace_size.argtypes = [ctypes.c_int] * 7
        L.mla_decode_workspace_size.restype = ctypes.c_size_t
        n = L.mla_decode_workspace_size(w.B, w.H, w.K, mla._dtype_code(base["kv_cache"]),
                                        mla._dtype_code(base["w_uk"]), 0, 0)
        # the buffers live in the build's record for the whole run: params hold raw pointers
        b = dict(path=path, L=L, ws=torch.empty(n, dtype=torch.uint8, device="cuda"),
                 out=torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda"),
                 lse=torch.empty((w.B, w.H), dtype=torch.float32, device="cuda"), times=[])
        b["ps"] = [mla.build_params(r["q_nope"], r["q_pe"], r["w_uk"], r["w_uv"], r["kv_cache"], r["pe_cache"],
                                    r["topk_indices"], r["cache_lens"], table, scale, b["out"], b["lse"], b["ws"])
                   for r in reps]
        builds.append(b)

    def run(b, p):
        rc = b["L"].mla_decode_attn(ctypes.byref(p), stream)
        if rc != 0:
            raise RuntimeError(f"{b['path']}: mla_decode_attn returned {rc}")

    ref = None
    for b in builds:
        for i in range(SETTLE_STEPS):
            run(b, b["ps"][i % R])
        run(b, b["ps"][0])
        torch.cuda.synchronize()
        o = b["out"].clone()
        ref = o if ref is None else ref
        b["max_abs_diff_vs_first"] = float((o - ref).abs().max())
    for rnd in range(args.ab_rounds):
        for b in (builds if rnd % 2 == 0 else builds[::-1]):
            for i in range(50):
                run(b, b["ps"][i % R])
            for i in range(N):
                p = b["ps"][i % R]
                p.profile_events = ctypes.cast(ev_arrays[i], ctypes.c_void_p)
                run(b, p)
                p.profile_events = None
            torch.cuda.synchronize()
            t = np.array([[hip.elapsed_ms(e[2 * k], e[2 * k + 1]) for k in range(nk)] for e in events]) * 1e3
            b["times"].append(t.mean(axis=0))
    res = []
    for b in builds:
        t = np.array(b["times"])
        rec = {"lib": b["path"], "max_abs_diff_vs_first": b["max_abs_diff_vs_first"]}
        for k, name in enumerate(mla.KERNEL_NAMES):
            rec[f"{name}_us"] = round(float(t[:, k].mean()), 2)
            rec[f"{name}_us_min_round"] = round(float(t[:, k].min()), 2)
        res.append(rec)
    print(json.dumps({"mode": "ab", "workload": args.workload, "rounds": args.ab_rounds,
                      "steps_per_round": N, "builds": res}), flush=True)


def measure_decode(wname, K, warmup, no_graph=False, replicas=0):
    """Time the decode step on the named workload: K eager steps with HIP
    events around each kernel (per-kernel durations), then K steps in a
    timed region (one HIP-graph replay, or eager launches with no_graph).
    Returns (line, w, out0, lse0): the JSON fields of the measurement, the
    workload, and the step's outputs on replica 0 (the workload's own values,
    taken before any timing) for the parity record."""
    import numpy as np
    import torch
    import workloads as W
    from decode_attention_absorbed_amd import mla

    torch.cuda.set_device(0)
    w = W.workload(wname)
    act = torch.bfloat16 if w.dtype_act == "bf16" else torch.float32
    wt = torch.bfloat16 if w.dtype_w == "bf16" else torch.float32
    rows = w.selected_rows()
    kv_bytes = rows * 576 * (2 if w.dtype_act == "bf16" else 4)
    w_bytes = 2 * w.H * 128 * 512 * (2 if w.dtype_w == "bf16" else 4)
    touched = kv_bytes + w_bytes + w.B * w.H * 192 * 2
    R = replicas or max(2, math.ceil(1.5e9 / touched))

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

    for i in range(warmup):
        mla.decode_attn(plain[i % R])
    torch.cuda.synchronize()
    # Parity snapshot: one step on replica 0 (the workload's own values),
    # compared with the oracle's outputs from the cpu_baseline leg below.
    mla.decode_attn(plain[0])
    torch.cuda.synchronize()
    out0, lse0 = out.cpu().numpy(), lse.cpu().numpy()

    # Per-kernel durations: K eager steps with HIP events recorded by the
    # library around each of its kernels on the launch stream.  They follow
    # ~30 ms of untimed steps: after an idle stretch (the host copies above)
    # the first tens of steps run slower while the clock rises, and the
    # kernel averages are meant to describe the steady state.
    for i in range(SETTLE_STEPS):
        mla.decode_attn(plain[i % R])
    for i in range(K):
        mla.decode_attn(timed[i])
    torch.cuda.synchronize()
    eager_ms = None
    graph = None
    if not no_graph:
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(K):
                mla.decode_attn(plain[i % R])
        graph.replay()                      # upload + one untimed pass
        for i in range(SETTLE_STEPS):       # warm again after the capture's idle stretch
            mla.decode_attn(plain[i % R])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            mla.decode_attn(plain[i % R])
        torch.cuda.synchronize()
        eager_ms = (time.perf_counter() - t0) * 1e3 / K

    # Untimed pre-roll of ~30 ms right before the timed region, for the same
    # reason: the graph capture above leaves the GPU idle, and a short timed
    # region (20 steps are ~3 ms) would otherwise include the clock ramp.
    if graph is not None:
        for _ in range(max(1, math.ceil(PREROLL_S / max(K * 130e-6, 1e-6)))):
            graph.replay()
    else:
        for i in range(max(K, math.ceil(PREROLL_S / 130e-6))):
            mla.decode_attn(plain[i % R])

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

    per_kernel, spread = {}, {}
    for k, name in enumerate(mla.KERNEL_NAMES):
        d = np.array([hip.elapsed_ms(e[2 * k], e[2 * k + 1]) for e in events])
        per_kernel[name] = float(d.mean())
        spread[name] = {q: float(np.percentile(d, v)) for q, v in (("p10", 10), ("p50", 50), ("p90", 90))}
    copy_gbs = stream_copy_gbs()
    ms_step = elapsed * 1e3 / K
    t_attn_s = per_kernel["attention"] * 1e-3
    achieved = rows * ROW_BYTES_BF16 / t_attn_s / 1e9 if w.dtype_act == "bf16" else kv_bytes / t_attn_s / 1e9
    attn_flops = 2.0 * w.H * (576 + 512) * rows
    flops = attn_flops + 4.0 * w.B * w.H * 128 * 512
    core_s = (per_kernel["attention"] + per_kernel["merge"]) * 1e-3
    tr = measured_traffic(wname)
    line = {
        "metric": METRIC,
        "value": w.B * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype_act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wname}: {DESCR[wname]}", "B": w.B, "H": w.H,
                   "L_max": w.L_max, "top_k": w.K, "selected_rows": rows, "num_splits": splits,
                   "input_replicas": R, "hip_graph": graph is not None},
        "eager_ms_per_step": eager_ms,
        "hbm_tb_s_step": kv_bytes / (ms_step * 1e-3) / 1e12,
        "hbm_pct_peak_step": kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "mfma_tflops_step": flops / (ms_step * 1e-3) / 1e12,
        # the three fractions of 8 TB/s on KV bytes: attention kernel alone,
        # attention core (attention + merge kernels), whole step (graph replay)
        "attention_frac": kv_bytes / t_attn_s / 1e9 / HBM_PEAK_GBS,
        "attention_core_frac": kv_bytes / core_s / 1e9 / HBM_PEAK_GBS,
        "end_to_end_frac": kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        # MFMA work (QK^T, PV and both absorptions) over the same times, against 2.5 PF bf16
        "mfma_pct": {"attention": attn_flops / t_attn_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "attention_core": flops / core_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "end_to_end": flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS},
        "kernel_ms": per_kernel,
        "kernel_ms_spread": spread,
        "stream_copy_gb_s": copy_gbs,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": tr,
                     "kernel": "attention", "algorithmic_bytes": rows * ROW_BYTES_BF16,
                     "frac_of_copy": achieved / copy_gbs,
                     # all the HBM bytes the counters give per launch (rows, Q~ per split,
                     # partials) over the same time: how close the kernel runs to the copy rate
                     "traffic_gb_s": tr / t_attn_s / 1e9 if tr else None,
                     "traffic_frac_of_copy": tr / t_attn_s / 1e9 / copy_gbs if tr else None,
                     "mfma_tflops": 2.0 * w.H * (576 + 512) * rows / t_attn_s / 1e12},
    }
    return line, w, out0, lse0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="ragged", choices=list(DESCR))
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=40.0,
                    help="seconds of oracle work at most (the ragged batch takes ~10 s on 16 cores)")
    ap.add_argument("--replicas", type=int, default=0, help="input copies cycled (0 = enough for 1.5 GB)")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the primary one into other_workloads "
                         "(default: long,batched with the ragged workload, none otherwise)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)")
    ap.add_argument("--op", default="decode", choices=["decode", "topk", "rope", "append"],
                    help="decode: the decode step (default); others time an adjacent entry point")
    ap.add_argument("--rope-layout", default="halves", choices=["halves", "interleaved"])
    ap.add_argument("--ab", nargs="+", metavar="LIB",
                    help="compare builds of libmla_decode.so on the workload's step (same process, "
                         "alternating order, per-kernel HIP events); one JSON line")
    ap.add_argument("--ab-rounds", type=int, default=6)
    args = ap.parse_args()
    if args.ab:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_ab(args)
        return
    if args.op != "decode":
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        bench_op(args)
        return
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

    line, w, out0, lse0 = measure_decode(args.workload, args.steps, args.warmup, args.no_graph, args.replicas)
    if not args.no_cpu_baseline:
        rec, ref, ref_lse = cpu_baseline(w, args.cpu_budget)
        line["cpu_baseline"] = rec
        line["parity"] = parity_record(out0, lse0, ref, ref_lse)
    # The other full-size workloads, measured the same way in the same run
    # (outside the metric, which is the primary workload's): a compact
    # record each, with parity over the rows the oracle finishes.
    also = args.also.split(",") if args.also is not None else (["long", "batched"] if args.workload == "ragged" else [])
    others = {}
    del w, out0, lse0
    for name in [n for n in also if n and n != "none"]:
        import torch
        torch.cuda.empty_cache()
        try:
            ln, w, out0, lse0 = measure_decode(name, args.steps, args.warmup, args.no_graph, args.replicas)
        except Exception as e:          # the primary line is printed whatever happens here
            others[name] = {"error": f"{type(e).__name__}: {e}"}
            continue
        keep = ("value", "ms_per_step", "kernel_ms", "attention_frac", "attention_core_frac", "end_to_end_frac",
                "mfma_pct", "stream_copy_gb_s")
        rec = {k: ln[k] for k in keep}
        rec["config"] = ln["config"]
        rec["roofline"] = {k: ln["roofline"][k] for k in ("achieved", "frac", "traffic", "algorithmic_bytes",
                                                           "frac_of_copy", "traffic_gb_s",
                                                           "traffic_frac_of_copy")}
        if not args.no_cpu_baseline:
            _, ref, ref_lse = cpu_baseline(w, args.cpu_budget)
            rec["parity"] = parity_record(out0, lse0, ref, ref_lse)
        others[name] = rec
        del w, out0, lse0
    if others:
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
