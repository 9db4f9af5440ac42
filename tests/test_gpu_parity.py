"""Parity of the HIP path (through the C ABI) with the CPU fp64 oracle.

Tolerances: max per-row relative L2 error 1e-5 for fp32 inputs and 1e-2 for
bf16 inputs (fp32 accumulation); the log-sum-exp output is compared with an
absolute error against the same bound.  Index handling is bit-exact.
"""
import numpy as np
import pytest

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_attention_absorbed_amd import mla  # noqa: E402
from gpu_util import Dev, oracle_ref, rel_l2_rows  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 1e-2}


def _check(dev, out, lse, batch=None, heads=None):
    w = dev.w
    ref, ref_lse = oracle_ref(w, batch=batch, heads=heads)
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    if batch is not None:
        o, l = o[batch], l[batch]
    if heads is not None:
        o, l = o[:, heads], l[:, heads]
    tol = TOL[w.dtype_act]
    err = rel_l2_rows(o, ref).max()
    lerr = np.abs(l - ref_lse).max()
    print(f"[{w.name}] max rel L2 {err:.3e}  max |dLSE| {lerr:.3e}  (tol {tol})", flush=True)
    assert err <= tol
    assert lerr <= tol
    return err


# ---------------------------------------------------------------------------
# a1: rotation table
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rope", [W.ROPE_YARN, W.ROPE_PLAIN], ids=["yarn", "plain"])
def test_rope_table_matches_oracle(rope):
    table = mla.rope_freqs(rope)
    torch.cuda.synchronize()
    got = table.cpu().numpy().astype(np.float64)
    cfg = oracle.RopeConfig(**rope)
    ref = oracle.rope_cos_sin(np.arange(rope["max_seq_len"]), cfg)
    assert got.shape == ref.shape
    # fp32 storage of exactly computed values: half an ulp of 1 at most
    assert np.abs(got - ref).max() <= 6e-8


def test_softmax_scale_matches_oracle():
    for rope in (W.ROPE_YARN, W.ROPE_PLAIN):
        assert mla.softmax_scale(192, rope) == pytest.approx(
            oracle.softmax_scale(192, oracle.RopeConfig(**rope)), rel=1e-15)


# ---------------------------------------------------------------------------
# Whole decode step: the pages' workloads
# ---------------------------------------------------------------------------
def test_tiny_fp32():
    dev = Dev(W.workload("tiny"))
    out, lse, _ = dev.run()
    _check(dev, out, lse)


def test_page_decode_example_bf16():
    dev = Dev(W.workload("page"))
    out, lse, _ = dev.run()
    _check(dev, out, lse)


# Small cases spanning several tiles, ragged tails, padding and head counts
# that are not multiples of the workgroup's head group.
CASES = [
    # name, B, H, lens, K, dtype_act, dtype_w, selection
    ("h128_ragged", 4, 128, [100, 777, 33, 2500], 640, "bf16", "bf16", "random"),
    ("h128_recent", 3, 128, [64, 65, 129], 96, "bf16", "f32", "recent"),
    ("h64", 3, 64, [300, 1, 1000], 257, "bf16", "bf16", "random"),
    ("h32", 2, 32, [500, 70], 130, "bf16", "bf16", "random"),
    ("h16", 2, 16, [77, 600], 200, "bf16", "f32", "random"),
    ("h96", 2, 96, [333, 444], 150, "bf16", "bf16", "random"),
    ("f32_h128", 2, 128, [300, 129], 200, "f32", "f32", "random"),
    ("f32_h16_bf16w", 2, 16, [50, 900], 64, "f32", "bf16", "random"),
    # more than one 128-head group per sequence, the second one partial
    ("h160", 2, 160, [300, 700], 300, "bf16", "bf16", "random"),
    ("h256", 1, 256, [1000], 512, "bf16", "f32", "recent"),
    # a single head; a single cached row
    ("h1", 3, 1, [40, 300, 1], 64, "bf16", "bf16", "random"),
    ("f32_h1", 2, 1, [1, 77], 16, "f32", "f32", "random"),
    # fp32 with enough (sequence, 16-head group) pairs for 16-head workgroups,
    # the last group of each sequence partial
    ("f32_h20_b40", 40, 20, [37 * (i % 7) + 5 for i in range(40)], 120, "f32", "f32", "random"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_small_cases(case):
    name, B, H, lens, K, da, dw, sel = case
    w = W.build(name, B, H, lens, K, da, dw, W.ROPE_YARN, seed=7 + len(name), selection=sel)
    dev = Dev(w)
    out, lse, _ = dev.run()
    _check(dev, out, lse)


# More than 128 sequences: the absorption handles sequences 128 at a time
# (the query chunk in LDS, the accumulators, the rotary query of each
# group), so these take its later groups, the last one partial, with both
# weight dtypes.
BIG_BATCH = [
    ("b130_h2_f32w", 130, 2, 40, "f32", "random", 0),
    ("b257_h3_bf16w", 257, 3, 24, "bf16", "alternate", 2),
]


@pytest.mark.parametrize("case", BIG_BATCH, ids=[c[0] for c in BIG_BATCH])
def test_batch_over_128_sequences(case):
    name, B, H, K, dw, sel, splits = case
    lens = np.random.default_rng(B).integers(1, 300, size=B)
    w = W.build(name, B, H, lens, K, "bf16", dw, W.ROPE_YARN, seed=B + H, selection=sel)
    dev = Dev(w)
    out, lse, _ = dev.run(num_splits=splits)
    _check(dev, out, lse)


def _sweep_cases(n=24, seed=2024):
    """Seeded random configurations: head counts around the 32-head wave and
    128-head workgroup boundaries, ragged lengths down to a single row, K not
    a multiple of the 32-row tile, both dtypes, forced split counts, and rows
    with -1 slots and duplicates in random places."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 7))
        H = int(rng.choice([1, 2, 16, 31, 33, 64, 100, 128, 129, 200]))
        lens = [int(x) for x in rng.integers(1, 2200, size=B)]
        if rng.random() < 0.3:
            lens[int(rng.integers(B))] = 1
        K = int(rng.integers(1, 400))
        da = "f32" if rng.random() < 0.25 else "bf16"
        dw = "f32" if rng.random() < 0.5 else "bf16"
        sel = str(rng.choice(["random", "recent", "alternate"]))
        splits = int(rng.choice([0, 1])) if da == "f32" else int(rng.choice([0, 0, 1, 2, 3, 7]))
        cases.append((f"sweep{i}", B, H, lens, K, da, dw, sel, splits, bool(rng.random() < 0.5),
                      int(rng.integers(1 << 30))))
    return cases


def _scramble(w, seed):
    """Move -1 slots to random places and fill some of them (or some taken
    slots) with duplicates of selected positions; every row keeps at least
    one position."""
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        row = w.topk_indices[b]
        valid = row[row >= 0]
        holes = np.flatnonzero(row < 0)
        if len(holes) == 0 and len(row) > 1:
            holes = rng.choice(len(row), size=max(1, len(row) // 8), replace=False)
            keep = np.setdiff1d(np.arange(len(row)), holes)
            valid = row[keep]
            row[holes] = -1
        dup = holes[: len(holes) // 2]
        row[dup] = rng.choice(valid, size=len(dup))
        w.topk_indices[b] = rng.permutation(row)
        assert (w.topk_indices[b] >= 0).any()


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: c[0])
def test_random_configurations(case):
    name, B, H, lens, K, da, dw, sel, splits, scramble, seed = case
    w = W.build(name, B, H, lens, K, da, dw, W.ROPE_YARN, seed=seed, selection=sel)
    if scramble:
        _scramble(w, seed + 1)
    print(f"[{name}] B={B} H={H} K={K} lens={lens} {da}/{dw} {sel} splits={splits} scrambled={scramble}",
          flush=True)
    dev = Dev(w)
    out, lse, _ = dev.run(num_splits=splits)
    _check(dev, out, lse)


def test_bf16_output():
    w = W.build("bf16out", 3, 128, [400, 50, 999], 256, "bf16", "bf16", W.ROPE_YARN, seed=11)
    dev = Dev(w)
    out32, lse32, _ = dev.run()
    out16, lse16, _ = dev.run(out_dtype=torch.bfloat16)
    assert out16.dtype == torch.bfloat16
    # the bf16 output is the fp32 one rounded to nearest even
    assert torch.equal(out16, out32.to(torch.bfloat16))
    assert torch.equal(lse16, lse32)


# ---------------------------------------------------------------------------
# Scores spread far beyond the N(0, 1) workloads (softmax over any masked
# scores, excerpt mla-decode).  The bf16 kernel exponentiates against the
# floored maximum of each split's first 32 rows and redoes a split with the
# exact maximum when a later score lies more than 64 units (log2) above it.
# The inputs push chosen rows down by c units for every head at once:
#   late150: the 3 last rows lie ~156 units above the rest: 2^156 overflows
#            fp32, so a correct result shows the second pass ran;
#   late90:  ~96 units: above the limit but below overflow;
#   late54:  ~60 units, just under the limit: the first pass stands, with
#            probabilities up to 2^60;
#   first200: the first 32 rows hold the maximum and every later row lies
#            ~200 units below it (its probability underflows to zero).
# Each with one split and with three (the last split holds the maximum).
# ---------------------------------------------------------------------------
import spread_inputs as SI  # noqa: E402

SPREAD = [("late", 150), ("late", 90), ("late", 54), ("first", 200)]


@pytest.mark.parametrize("mode,c", SPREAD, ids=[f"{m}{c}" for m, c in SPREAD])
@pytest.mark.parametrize("splits", [1, 3])
def test_wide_score_spread_bf16(mode, c, splits):
    w = SI.build(f"spread_{mode}{c}", mode, c)
    print(f"[{w.name}] splits={splits} excess per split "
          f"{[[round(e, 1) for e in SI.excess_log2(w, b, splits)] for b in range(w.B)]}", flush=True)
    dev = Dev(w)
    out, lse, _ = dev.run(num_splits=splits)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _check(dev, out, lse)


@pytest.mark.parametrize("mode,c", SPREAD, ids=[f"{m}{c}" for m, c in SPREAD])
def test_wide_score_spread_f32(mode, c):
    w = SI.build(f"spread32_{mode}{c}", mode, c, dtype_act="f32", dtype_w="f32", H=16)
    dev = Dev(w)
    out, lse, _ = dev.run()
    _check(dev, out, lse)


# ---------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the bench times, checked
# on every sequence and head against the oracle.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["batched", "long", "ragged", "ragged_h16"])
def test_full_size_every_sequence(name):
    w = W.workload(name)
    dev = Dev(w)
    out, lse, _ = dev.run()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    ref, ref_lse = oracle_ref(w)
    err = rel_l2_rows(out.cpu().numpy(), ref)
    dl = np.abs(lse.cpu().numpy() - ref_lse)
    print(f"[{name}] {err.size} rows: max rel L2 {err.max():.3e}  p99 {np.percentile(err, 99):.3e}  "
          f"median {np.median(err):.3e}  max |dLSE| {dl.max():.3e}", flush=True)
    assert err.max() <= TOL["bf16"]
    assert dl.max() <= TOL["bf16"]
    del dev
    torch.cuda.empty_cache()


def test_max_cache_length():
    # the longest cache the host checks accept (2^19 rows): the selection
    # bitmap fills the prep kernel's 64 KB of LDS, the compacted list is
    # written straight to the workspace (the LDS staging covers up to 16384
    # rows), the newest row sits at the top of the 32-bit row offsets, and
    # the rotation table has 2^19 rows
    rope = dict(W.ROPE_YARN, max_seq_len=1 << 19)
    w = W.build("maxlen", 2, 16, [1 << 19, 20000], 512, "bf16", "bf16", rope, seed=1401)
    dev = Dev(w)
    out, lse, (rc, st) = dev.run(validate=True)
    assert rc == mla.MLA_OK and st == 0
    _check(dev, out, lse)
    del dev
    torch.cuda.empty_cache()


def test_long_selection():
    # 20000 selected rows: more than the 16384-entry LDS list, hundreds of
    # tiles per split
    rope = dict(W.ROPE_YARN, max_seq_len=40000)
    w = W.build("longsel", 2, 32, [40000, 30000], 20000, "bf16", "bf16", rope, seed=1404,
                k_per_seq=[20000, 17000])
    dev = Dev(w)
    out, lse, (rc, st) = dev.run(validate=True)
    assert rc == mla.MLA_OK and st == 0
    _check(dev, out, lse)


def test_many_workgroups_and_query_chunks():
    # 300 sequences: more attention workgroups than compute units, three
    # 128-sequence query chunks in the absorption, ten merge batches
    rng = np.random.default_rng(1402)
    lens = rng.integers(1, 600, size=300)
    w = W.build("manyseq", 300, 32, list(lens), 128, "bf16", "f32", W.ROPE_YARN, seed=1403)
    dev = Dev(w)
    out, lse, _ = dev.run()
    _check(dev, out, lse)


# ---------------------------------------------------------------------------
# Index handling (bit-exact)
# ---------------------------------------------------------------------------
def _poison_unselected(w, kv, pe):
    """NaN in every cache row that is not selected, including rows >= L_b."""
    kv = kv.clone()
    pe = pe.clone()
    for b in range(w.B):
        keep = np.zeros(w.L_max, dtype=bool)
        row = w.topk_indices[b]
        keep[row[row >= 0]] = True
        drop = torch.from_numpy(~keep).cuda()
        kv[b][drop] = float("nan")
        pe[b][drop] = float("nan")
    return kv, pe


@pytest.mark.parametrize("da", ["bf16", "f32"])
def test_unselected_rows_never_read(da):
    w = W.build("poison", 3, 128 if da == "bf16" else 16, [700, 1500, 64], 300, da, "bf16", W.ROPE_YARN,
                seed=21, L_max=1600)
    dev = Dev(w)
    out0, lse0, _ = dev.run()
    kv, pe = _poison_unselected(w, dev.kv, dev.pe)
    out1, lse1, _ = dev.run(kv=kv, pe=pe)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    assert torch.isfinite(out1).all()


def test_padding_order_and_duplicates_bit_exact():
    w = W.build("pad", 3, 128, [900, 2000, 300], 256, "bf16", "bf16", W.ROPE_YARN, seed=22, L_max=2048)
    dev = Dev(w)
    out0, lse0, _ = dev.run(num_splits=2)
    rng = np.random.default_rng(5)
    idx = np.full((w.B, 700), -1, dtype=np.int32)
    for b in range(w.B):
        row = w.topk_indices[b]
        sel = row[row >= 0]
        ext = np.concatenate([sel, rng.choice(sel, size=100), np.full(700 - sel.size - 100, -1)])
        idx[b] = rng.permutation(ext)
    kv, pe = _poison_unselected(w, dev.kv, dev.pe)
    out1, lse1, _ = dev.run(idx=torch.from_numpy(idx).cuda(), kv=kv, pe=pe, num_splits=2)
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_validate_mode_flags_planted_errors():
    w = W.build("val", 5, 64, [100, 200, 300, 400, 500], 64, "bf16", "bf16", W.ROPE_YARN, seed=23, L_max=512)
    dev = Dev(w)
    out, lse, (rc, st) = dev.run(validate=True)
    assert rc == mla.MLA_OK and st == 0
    cases = []
    idx = w.topk_indices.copy(); idx[1, 3] = 200                  # == L_1: out of range
    cases.append((idx, w.cache_lens, mla.MLA_BAD_INDEX_RANGE))
    idx = w.topk_indices.copy(); idx[2, 5] = -7                   # negative, not -1
    cases.append((idx, w.cache_lens, mla.MLA_BAD_INDEX_RANGE))
    idx = w.topk_indices.copy(); idx[3, 9] = idx[3, 10]           # duplicate
    cases.append((idx, w.cache_lens, mla.MLA_BAD_DUPLICATE))
    idx = w.topk_indices.copy(); idx[4, :] = -1                   # empty
    cases.append((idx, w.cache_lens, mla.MLA_BAD_EMPTY))
    lens = w.cache_lens.copy(); lens[0] = 513                     # > max_cache_len
    cases.append((w.topk_indices, lens, mla.MLA_BAD_CACHE_LEN))
    lens = w.cache_lens.copy(); lens[0] = 0
    cases.append((w.topk_indices, lens, mla.MLA_BAD_CACHE_LEN | mla.MLA_BAD_INDEX_RANGE | mla.MLA_BAD_EMPTY))
    for idx, lens, want in cases:
        _, _, (rc, st) = dev.run(validate=True, idx=torch.from_numpy(np.ascontiguousarray(idx)).cuda(),
                                 lens=torch.from_numpy(lens).cuda(), check=False)
        assert rc == mla.MLA_ERR_INVALID_INDEX
        assert st == want, (st, want)


def test_empty_selection_gives_nan_without_validate():
    w = W.build("empty", 2, 128, [100, 200], 16, "bf16", "bf16", W.ROPE_YARN, seed=24)
    dev = Dev(w)
    idx = w.topk_indices.copy()
    idx[1, :] = -1
    out, lse, (rc, st) = dev.run(idx=torch.from_numpy(idx).cuda())
    assert rc == mla.MLA_OK
    assert torch.isnan(out[1]).all()
    ref, _ = oracle_ref(w, batch=[0])
    assert rel_l2_rows(out[0:1].cpu().numpy(), ref).max() <= 1e-2


# ---------------------------------------------------------------------------
# Split plan, strided inputs
# ---------------------------------------------------------------------------
def test_split_count_invariance():
    w = W.workload("batched", batch_limit=4)
    dev = Dev(w)
    planned = mla.num_splits(w.B, w.H, w.K, mla.MLA_DTYPE_BF16)
    assert planned > 1
    outs = {}
    for S in (1, 2, planned, 7):
        out, lse, _ = dev.run(num_splits=S)
        outs[S] = (out, lse)
        _check(dev, out, lse)
    base, base_lse = outs[1]
    for S, (out, lse) in outs.items():
        # Every plan rounds the same probabilities to bf16 (the reference
        # maximum is floored, so moving a split boundary scales them by powers
        # of two only).  What differs is where latent sums are rounded to bf16:
        # each split's normalised partial (at most 2^-9 relative per element;
        # the merge projects the bf16 partials and combines the projections in
        # fp32).  Their difference stays within 3.5e-3 per output row (about
        # 3.1e-3 at most on these inputs), well inside the 1e-2 parity bar;
        # a dropped, doubled or misweighted split moves rows by far more.  The
        # log-sum-exp is formed from fp32 sums and agrees to fp32 rounding.
        err = rel_l2_rows(out.cpu().numpy(), base.cpu().numpy()).max()
        print(f"splits {S}: max rel L2 vs one split {err:.3e}", flush=True)
        assert err <= 3.5e-3, (S, err)
        assert (lse - base_lse).abs().max().item() <= 1e-5


def test_graph_replay_matches_eager():
    # The throughput measurement replays the step from a HIP graph.  Every
    # replay, with eager steps on other inputs and synchronisations between
    # the replays, gives the eager step's outputs bit for bit; so does the
    # step with the fused append (rewriting the same rows is idempotent).
    w = W.build("graph", 8, 128, [3000, 64, 1500, 777, 4096, 1, 2048, 300], 1024, "bf16", "f32",
                W.ROPE_YARN, seed=31)
    dev = Dev(w)
    other = Dev(W.build("graph_other", 8, 128, [900, 4000, 2, 1200, 50, 3333, 640, 2100], 1024, "bf16",
                        "f32", W.ROPE_YARN, seed=32))
    kv_new, pe_new = W.new_rows(w.B, "bf16", seed=33)
    kn = torch.from_numpy(kv_new).to(torch.bfloat16).cuda()
    pn = torch.from_numpy(pe_new).to(torch.bfloat16).cuda()
    n = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(dev.kv), mla._dtype_code(dev.w_uk), 0, 0)
    assert mla.num_splits(w.B, w.H, w.K, mla._dtype_code(dev.kv)) > 1
    for append in (False, True):
        out = torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        extra = dict(kv_new=kn, pe_new=pn) if append else {}
        p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                             dev.rope_table, dev.scale, out, lse, ws, **extra)
        mla.decode_attn(p)
        torch.cuda.synchronize()
        ref_out, ref_lse = out.clone(), lse.clone()
        if not append:
            _check(dev, out, lse, batch=[0, 3, 5, 7])
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            mla.decode_attn(p)
        for r in range(4):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            ws.fill_(0xFF)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), (append, r)
            other.run()                     # an eager step on other inputs (synchronises)
        del graph


GRAPH_SMALL = [
    # below 128 heads: the merge's batch split (second grid dimension) and the
    # absorption's sequence-group split; the fp32 path's kernels
    ("graph_h16_b130", 130, 16, 256, "bf16", "f32"),
    ("graph_f32_h20_b40", 40, 20, 120, "f32", "f32"),
]


@pytest.mark.parametrize("case", GRAPH_SMALL, ids=[c[0] for c in GRAPH_SMALL])
def test_graph_replay_other_launch_shapes(case):
    # as above, for the launch shapes the 128-head case does not take
    name, B, H, K, da, dw = case
    lens = [int(x) for x in np.random.default_rng(B + H).integers(1, 3000, size=B)]
    w = W.build(name, B, H, lens, K, da, dw, W.ROPE_YARN, seed=B * H)
    dev = Dev(w)
    n = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(dev.kv), mla._dtype_code(dev.w_uk), 0, 0)
    out = torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                         dev.rope_table, dev.scale, out, lse, ws)
    mla.decode_attn(p)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    _check(dev, out, lse, batch=[0, w.B // 2, w.B - 1])
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        mla.decode_attn(p)
    for r in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xFF)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), r
        dev.run()                           # an eager step in between (synchronises)
    del graph


def test_concurrent_streams_match_serial():
    # Calls on two streams, each with its own workspace, overlap on the device
    # and still give the outputs of the same calls run one after the other,
    # bit for bit: a call keeps no state outside its workspace and outputs.
    rng = np.random.default_rng(41)
    ws_a = W.build("streams_a", 16, 128, list(rng.integers(1, 6000, 16)), 2048, "bf16", "f32", W.ROPE_YARN,
                   seed=42)
    ws_b = W.build("streams_b", 24, 128, list(rng.integers(1, 5000, 24)), 1024, "bf16", "bf16", W.ROPE_YARN,
                   seed=43)
    calls = []
    for dev in (Dev(ws_a), Dev(ws_b)):
        w = dev.w
        out = torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
        n = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(dev.kv), mla._dtype_code(dev.w_uk), 0, 0)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                             dev.rope_table, dev.scale, out, lse, ws)
        calls.append((p, out, lse, ws))
    for p, *_ in calls:
        mla.decode_attn(p)
    torch.cuda.synchronize()
    refs = [(out.clone(), lse.clone()) for _, out, lse, _ in calls]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for _, out, lse, ws in calls:
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            ws.fill_(0xFF)
        torch.cuda.synchronize()
        for _ in range(4):                  # several calls in flight on each stream
            for (p, *_), st in zip(calls, streams):
                mla.decode_attn(p, stream=st)
        torch.cuda.synchronize()
        for (_, out, lse, _), (ro, rl) in zip(calls, refs):
            assert torch.equal(out, ro) and torch.equal(lse, rl), rep


def test_fused_buffers_match_separate():
    w = W.build("fused", 3, 128, [300, 900, 50], 200, "bf16", "bf16", W.ROPE_YARN, seed=25)
    dev = Dev(w)
    out0, lse0, _ = dev.run()
    fused = torch.cat([dev.kv, dev.pe], dim=-1).contiguous()            # [B, L, 576]
    kv, pe = fused[..., :512], fused[..., 512:]
    wkv_b = torch.cat([dev.w_uk, dev.w_uv], dim=1).contiguous()         # [H, 256, 512]
    out1, lse1, _ = dev.run(kv=kv, pe=pe, w_uk=wkv_b[:, :128], w_uv=wkv_b[:, 128:])
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)


def test_strided_queries_and_output():
    # the model's own layouts: q_nope and q_pe as views of one [B, H, 192]
    # query tensor, and the output written into a wider [B, H, 256] buffer;
    # same arithmetic, so the result is bit-identical to the contiguous call
    w = W.build("strided", 3, 128, [300, 900, 50], 200, "bf16", "bf16", W.ROPE_YARN, seed=26)
    dev = Dev(w)
    out0, lse0, _ = dev.run()
    q = torch.cat([dev.q_nope, dev.q_pe], dim=-1).contiguous()          # [B, H, 192]
    wide = torch.full((w.B, w.H, 256), float("nan"), dtype=torch.float32, device="cuda")
    out1 = wide[..., :128]
    lse1 = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    n = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(dev.kv), mla._dtype_code(dev.w_uk), 0, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    p = mla.build_params(q[..., :128], q[..., 128:], dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                         dev.rope_table, dev.scale, out1, lse1, ws)
    assert p.q_nope_stride_h == 192 and p.out_stride_h == 256
    mla.decode_attn(p)
    torch.cuda.synchronize()
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    assert torch.isnan(wide[..., 128:]).all()                            # nothing written past the rows


def test_host_errors_launch_nothing():
    w = W.build("err", 2, 128, [100, 100], 16, "bf16", "bf16", W.ROPE_YARN, seed=26)
    dev = Dev(w)
    out = torch.zeros((2, 128, 128), device="cuda")
    p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                         dev.rope_table, dev.scale, out, None, torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert mla.decode_attn(p, check=False) == mla.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 0).all()
