"""Parity of mla_topk (the top-k selection step) with the oracle's topk_select.

Index output is compared bit-exactly: both sides use the same order (NaN
lowest, -0 == +0, ties to the lower position), so the selected set, its
ascending order and the -1 padding are unique.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_attention_absorbed_amd import mla  # noqa: E402


def _expected(scores, lens, k):
    B = scores.shape[0]
    out = np.full((B, k), -1, dtype=np.int64)
    for b in range(B):
        sel = oracle.topk_select(scores[b], int(lens[b]), k)
        out[b, :sel.size] = sel
    return out


def _run(scores, lens, k):
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).cuda()
    l = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    got = mla.topk(s, l, k)
    torch.cuda.synchronize()
    return got.cpu().numpy().astype(np.int64)


def _check(scores, lens, k, name):
    got = _run(scores, lens, k)
    want = _expected(scores.astype(np.float32).astype(np.float64), lens, k)
    bad = np.nonzero((got != want).any(axis=1))[0]
    print(f"[topk {name}] B={scores.shape[0]} L={scores.shape[1]} k={k}: {bad.size} rows differ", flush=True)
    assert bad.size == 0, f"rows {bad[:5]} differ: got {got[bad[0]][:10]} want {want[bad[0]][:10]}"


def test_topk_random_ragged():
    rng = np.random.default_rng(1101)
    B, L, k = 12, 5000, 300
    scores = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.array([0, 1, 299, 300, 301, 5000, 4096, 1234, 2, 3000, 4999, 777])
    _check(scores, lens, k, "random ragged")


def test_topk_ties_nan_signed_zero():
    rng = np.random.default_rng(1102)
    B, L, k = 8, 3000, 257
    scores = rng.integers(-3, 4, size=(B, L)).astype(np.float32)   # heavy ties at the threshold
    scores[rng.random((B, L)) < 0.05] = np.nan
    scores[rng.random((B, L)) < 0.1] = -0.0
    scores[rng.random((B, L)) < 0.02] = -np.inf
    scores[rng.random((B, L)) < 0.01] = np.inf
    lens = rng.integers(200, L + 1, size=B)
    _check(scores, lens, k, "ties")


def test_topk_all_equal_and_k_one():
    B, L = 3, 1000
    scores = np.zeros((B, L), dtype=np.float32)
    _check(scores, np.array([1000, 10, 500]), 64, "all equal")
    rng = np.random.default_rng(1103)
    _check(rng.standard_normal((B, L)).astype(np.float32), np.array([1000, 1, 999]), 1, "k=1")


def test_topk_rows_beyond_lds():
    # rows longer than 32768 positions (keys re-read from the scores each
    # pass), and a shorter row of the same launch (keys in LDS)
    rng = np.random.default_rng(1104)
    B, L, k = 3, 70000, 2048
    scores = rng.standard_normal((B, L)).astype(np.float32)
    _check(scores, np.array([70000, 40000, 20000]), k, "long rows")


def test_topk_rows_up_to_32768():
    # 32 keys per thread: rows in (16384, 32768], with ties, NaN and -0
    rng = np.random.default_rng(1108)
    B, L, k = 4, 32768, 2048
    scores = rng.standard_normal((B, L)).astype(np.float32)
    scores[2] = rng.integers(-2, 3, size=L).astype(np.float32)
    scores[2, rng.random(L) < 0.05] = np.nan
    scores[2, rng.random(L) < 0.1] = -0.0
    _check(scores, np.array([32768, 20000, 30001, 16385]), k, "32 per thread")


def test_topk_all_equal_full_row():
    # every key equal on a 32768-position row: the packed (above, equal)
    # counts reach their largest values
    scores = np.full((2, 32768), 1.5, dtype=np.float32)
    _check(scores, np.array([32768, 32767]), 100, "all equal 32768")


def test_topk_unaligned_rows():
    # a row stride of L + 1 floats leaves odd rows off 16-byte alignment
    rng = np.random.default_rng(1109)
    B, L, k = 4, 3001, 257
    full = rng.standard_normal((B, L + 1)).astype(np.float32)
    s = torch.from_numpy(full).cuda()[:, :L]
    lens = torch.from_numpy(np.array([3001, 3000, 2999, 400], dtype=np.int32)).cuda()
    got = mla.topk(s, lens, k)
    torch.cuda.synchronize()
    want = _expected(full[:, :L].astype(np.float64), [3001, 3000, 2999, 400], k)
    assert np.array_equal(got.cpu().numpy().astype(np.int64), want)


def test_topk_decode_shape_every_row():
    # the long-context decode shape: 64 rows of 16384 scores, k = 2048
    rng = np.random.default_rng(1105)
    B, L, k = 64, 16384, 2048
    scores = rng.standard_normal((B, L)).astype(np.float32)
    lens = np.full(B, L)
    got = _run(scores, lens, k)
    for b in range(B):
        want = oracle.topk_select(scores[b].astype(np.float64), L, k)
        assert np.array_equal(got[b], want), b


def test_topk_narrow_band_large_k():
    # every score of a row in [1, 1 + 1/16) (one radix digit of sign,
    # exponent and the leading mantissa bits), ties at many ranks in one row;
    # selections past 4096 positions (written without LDS staging), rows of
    # 65536 positions and short rows in the same launch
    rng = np.random.default_rng(1112)
    B, L = 3, 65536
    scores = (1.0 + rng.random((B, L)) / 16.0).astype(np.float32)
    scores[1, rng.random(L) < 0.2] = np.float32(1.03125)
    _check(scores, np.array([65536, 20000, 4097]), 5000, "narrow band, k=5000")
    _check(scores, np.array([65536, 20000, 4097]), 30000, "narrow band, k=30000")
    _check(scores[:, :16384], np.array([16384, 5000, 4100]), 4096, "narrow band, k=4096")


def test_topk_feeds_decode():
    # mla_topk's rows used as the decode step's selection give the oracle's
    # output for the oracle's selection
    import workloads as W
    from gpu_util import Dev, oracle_ref, rel_l2_rows
    w = W.build("topk_feed", 2, 128, [700, 1500], 512, "bf16", "bf16", W.ROPE_YARN, seed=1106)
    rng = np.random.default_rng(1107)
    scores = rng.standard_normal((2, w.L_max)).astype(np.float32)
    sel = _run(scores, w.cache_lens, 512)
    w.topk_indices = sel.astype(np.int32)
    dev = Dev(w)
    out, lse, _ = dev.run()
    ref, _ = oracle_ref(w)
    err = rel_l2_rows(out.float().cpu().numpy(), ref).max()
    print(f"[topk feed] max rel L2 {err:.3e}", flush=True)
    assert err <= 1e-2


def _topk_sweep(n=20, seed=1200):
    """Seeded random shapes over all three kernel forms (rows up to 16384 and
    up to 32768 keys in registers, longer rows re-read), k from 1 to past the
    row length, and score mixes: normal, heavy ties, a narrow band of nearby
    floats, magnitudes from denormals to 1e38, with NaN / -0 / +-inf mixed in."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        L = int(rng.choice([1, 37, 2048, 9000, 16384, 16385, 25000, 32768, 40000]))
        B = int(rng.integers(1, 9))
        k = int(rng.choice([1, 2, 100, 1024, 2048, 3000]))
        kind = str(rng.choice(["normal", "ties", "band", "wide"]))
        cases.append((f"sweep{i}", B, L, k, kind, bool(rng.random() < 0.5), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _topk_sweep(), ids=lambda c: c[0])
def test_topk_random_shapes(case):
    name, B, L, k, kind, specials, seed = case
    rng = np.random.default_rng(seed)
    if kind == "normal":
        scores = rng.standard_normal((B, L)).astype(np.float32)
    elif kind == "ties":
        scores = rng.integers(-4, 5, size=(B, L)).astype(np.float32)
    elif kind == "band":
        # consecutive floats around 1.0: keys differ only in their low bits
        scores = (np.float32(1.0) + rng.integers(-300, 300, size=(B, L)).astype(np.float32)
                  * np.float32(2.0 ** -23)).astype(np.float32)
    else:
        mag = 10.0 ** rng.uniform(-44, 38, size=(B, L))
        scores = (np.sign(rng.standard_normal((B, L))) * mag).astype(np.float32)
    if specials:
        for v, p in ((np.nan, 0.03), (-0.0, 0.05), (0.0, 0.02), (np.inf, 0.005), (-np.inf, 0.01)):
            scores[rng.random((B, L)) < p] = v
    lens = rng.integers(0, L + 1, size=B)
    lens[0] = L
    _check(scores, lens, k, f"{name} {kind}{' +specials' if specials else ''}")


def test_topk_bucket_edge_cases():
    # rows whose value range defeats the linear bucket map: a span past the
    # float range (one bucket for all finite scores), only NaN and -inf, a
    # tiny range near zero, and one outlier far above a tight cluster (most
    # keys share a bucket: the radix passes over the candidates and over the
    # registers)
    rng = np.random.default_rng(1110)
    B, L, k = 6, 16384, 2048
    scores = rng.standard_normal((B, L)).astype(np.float32)
    scores[0, :2] = [3e38, -3e38]
    scores[1] = np.nan
    scores[1, ::7] = -np.inf
    scores[2] *= np.float32(1e-30)
    scores[3] = 1.0 + rng.standard_normal(L).astype(np.float32) * np.float32(1e-6)
    scores[3, 5] = 1e30
    scores[4, rng.random(L) < 0.5] = np.inf
    scores[5] = np.float32(2.0)
    scores[5, rng.random(L) < 0.3] = np.nan
    _check(scores, np.array([L, L, L, L, L, 9000]), k, "bucket edges")
