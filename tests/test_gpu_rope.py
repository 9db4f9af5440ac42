"""Parity of mla_rope_apply (rotary embedding at per-row positions, both
feature layouts) with the oracle's rope_rotate (interleaved pairs) and
rope_rotate_halves (pairs (i, i+32)).

Bars: per-vector relative L2 1e-2 for bf16 output, 1e-5 for float32.  The
two layouts run the same per-pair arithmetic, so permuting the features
between them must give bit-identical results.
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

CFG = oracle.RopeConfig(**W.ROPE_YARN)
_TABLE = {}


def _table():
    if "t" not in _TABLE:
        _TABLE["t"] = mla.rope_freqs(W.ROPE_YARN)
    return _TABLE["t"]


def _reference(x64, pos, interleaved):
    f = oracle.rope_rotate if interleaved else oracle.rope_rotate_halves
    return np.stack([f(x64[n], int(pos[n]), CFG) for n in range(x64.shape[0])])


def _rel_l2(got, ref):
    g = got.reshape(-1, 64)
    r = ref.reshape(-1, 64)
    return (np.linalg.norm(g - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)).max()


def _case(N, H, dtype, interleaved, seed, name):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H, 64)).astype(np.float32)
    pos = rng.integers(0, W.ROPE_YARN["max_seq_len"], size=N).astype(np.int32)
    pos[0] = 0
    pos[-1] = W.ROPE_YARN["max_seq_len"] - 1
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    xd = torch.from_numpy(x).cuda().to(td)
    pd = torch.from_numpy(pos).cuda()
    print(f"[rope {name}] N={N} H={H} {dtype} interleaved={interleaved}", flush=True)
    y = mla.rope_apply(xd, pd, _table(), interleaved)
    torch.cuda.synchronize()
    ref = _reference(xd.float().cpu().numpy().astype(np.float64), pos, interleaved)
    return y, ref, xd, pd


@pytest.mark.parametrize("interleaved", [True, False])
@pytest.mark.parametrize("dtype,bar", [("bf16", 1e-2), ("f32", 1e-5)])
def test_rope_apply_matches_oracle(interleaved, dtype, bar):
    y, ref, _, _ = _case(37, 5, dtype, interleaved, 1201 + interleaved, "random")
    err = _rel_l2(y.float().cpu().numpy(), ref)
    print(f"  max rel L2 {err:.3e}", flush=True)
    assert err <= bar


@pytest.mark.parametrize("interleaved", [True, False])
def test_rope_apply_indexer_shape(interleaved):
    # 64 sequences x 64 indexer heads of 64 rotary features, bf16
    y, ref, _, _ = _case(64, 64, "bf16", interleaved, 1203, "indexer shape")
    assert _rel_l2(y.float().cpu().numpy(), ref) <= 1e-2


def test_rope_apply_layouts_agree_bitwise():
    # permuting the features from one layout into the other commutes with
    # the rotation, bit for bit (same per-pair arithmetic)
    rng = np.random.default_rng(1204)
    N = 50
    x = torch.from_numpy(rng.standard_normal((N, 64)).astype(np.float32)).cuda()
    pos = torch.from_numpy(rng.integers(0, 16384, size=N).astype(np.int32)).cuda()
    perm = torch.empty(64, dtype=torch.long)
    perm[0::2] = torch.arange(32)
    perm[1::2] = torch.arange(32) + 32
    perm = perm.cuda()
    for td in (torch.float32, torch.bfloat16):
        xh = x.to(td)
        y_half = mla.rope_apply(xh, pos, _table(), False)
        y_int = mla.rope_apply(xh[:, perm].contiguous(), pos, _table(), True)
        torch.cuda.synchronize()
        assert torch.equal(y_int, y_half[:, perm]), td


def test_rope_apply_in_place_and_strided():
    # rotate the rotary slice [512:576] of 576-wide rows in place, as a
    # cache row or a rotary query sits in memory
    rng = np.random.default_rng(1205)
    N = 33
    buf = torch.from_numpy(rng.standard_normal((N, 576)).astype(np.float32)).cuda().to(torch.bfloat16)
    before = buf.clone()
    pos = torch.from_numpy(rng.integers(0, 16384, size=N).astype(np.int32)).cuda()
    view = buf[:, 512:576]
    fresh = mla.rope_apply(view, pos, _table(), True)
    out = mla.rope_apply(view, pos, _table(), True, out=view)
    torch.cuda.synchronize()
    assert out.data_ptr() == view.data_ptr()
    assert torch.equal(buf[:, :512], before[:, :512])
    assert torch.equal(buf[:, 512:], fresh)
    ref = _reference(before[:, 512:].float().cpu().numpy().astype(np.float64), pos.cpu().numpy(), True)
    assert _rel_l2(fresh.float().cpu().numpy(), ref) <= 1e-2


def test_rope_apply_position_out_of_table_gives_nan():
    rng = np.random.default_rng(1206)
    x = torch.from_numpy(rng.standard_normal((4, 2, 64)).astype(np.float32)).cuda()
    pos = torch.tensor([5, -1, 16384, 16383], dtype=torch.int32).cuda()
    y = mla.rope_apply(x, pos, _table(), False)
    torch.cuda.synchronize()
    y = y.cpu()
    assert torch.isnan(y[1]).all() and torch.isnan(y[2]).all()
    assert torch.isfinite(y[0]).all() and torch.isfinite(y[3]).all()
    ref = _reference(x.cpu().numpy().astype(np.float64)[[0, 3]], [5, 16383], False)
    assert _rel_l2(y[[0, 3]].numpy(), ref) <= 1e-5


def _rope_sweep(n=16, seed=1300):
    """Seeded random shapes: row and vector strides padded by multiples of 8
    elements, both dtypes and layouts, in place or into a separate tensor."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        cases.append((f"sweep{i}", int(rng.integers(1, 3000)), int(rng.choice([1, 3, 16, 64, 128])),
                      str(rng.choice(["bf16", "f32"])), bool(rng.random() < 0.5), int(rng.integers(0, 3)),
                      int(rng.integers(0, 3)), bool(rng.random() < 0.5), int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _rope_sweep(), ids=lambda c: c[0])
def test_rope_apply_random_shapes(case):
    name, N, H, dtype, interleaved, pad_h, pad_n, in_place, seed = case
    rng = np.random.default_rng(seed)
    T = W.ROPE_YARN["max_seq_len"]
    sh = 64 + 8 * pad_h
    sn = (H - 1) * sh + 64 + 8 * pad_n
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    buf = torch.from_numpy(rng.standard_normal(N * sn).astype(np.float32)).to(td).cuda()
    before = buf.clone()
    x = buf.as_strided((N, H, 64), (sn, sh, 1))
    pos = rng.integers(0, T, size=N).astype(np.int32)
    pos[0] = 0
    pos[-1] = T - 1
    pd = torch.from_numpy(pos).cuda()
    print(f"[rope {name}] N={N} H={H} {dtype} interleaved={interleaved} strides ({sn}, {sh}) "
          f"in_place={in_place}", flush=True)
    x64 = x.float().cpu().numpy().astype(np.float64)
    y = mla.rope_apply(x, pd, _table(), interleaved, out=x if in_place else None)
    torch.cuda.synchronize()
    ref = _reference(x64, pos, interleaved)
    bar = 1e-2 if dtype == "bf16" else 1e-5
    assert _rel_l2(y.float().cpu().numpy(), ref) <= bar
    # the elements between the vectors are never written
    mask = torch.ones(N * sn, dtype=torch.bool)
    mask.as_strided((N, H, 64), (sn, sh, 1)).fill_(False)
    assert torch.equal(buf.cpu()[mask], before.cpu()[mask])
    if not in_place:
        assert torch.equal(buf.cpu(), before.cpu())
