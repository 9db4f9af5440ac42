"""CPU-side checks of the C ABI: the library builds and loads, exports every
symbol the header declares, and its host logic (argument checks, planner,
workspace sizing, softmax scale) behaves as documented.  No GPU work."""
import ctypes
import os
import re

import pytest

import oracle
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def mla():
    from decode_attention_absorbed_amd import build, mla as m
    if not os.path.exists(m.LIB_PATH):
        build.build()
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("mla_rope_freqs", "mla_softmax_scale", "mla_decode_workspace_size", "mla_decode_attn",
                 "mla_decode_num_splits", "mla_last_error", "mla_decode_params_size", "mla_topk",
                 "mla_rope_apply"):
        assert want in names


def test_library_exports_every_declared_symbol(mla):
    L = ctypes.CDLL(mla.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_params_layout_matches(mla):
    assert mla.lib().mla_decode_params_size() == ctypes.sizeof(mla.DecodeParams)


def test_softmax_scale_host(mla):
    for rope in (W.ROPE_YARN, W.ROPE_PLAIN):
        assert mla.softmax_scale(192, rope) == pytest.approx(
            oracle.softmax_scale(192, oracle.RopeConfig(**rope)), rel=1e-15)
    assert mla.lib().mla_softmax_scale(0, ctypes.byref(mla.rope_cfg(W.ROPE_YARN))) < 0


def test_planner_and_workspace(mla):
    # one attention workgroup per CU: B * head_groups * splits <= CUs, where
    # a workgroup takes 128 heads
    for H, hg in ((128, 1), (16, 1), (256, 2)):
        for B in (1, 2, 8, 32, 64, 128, 300):
            S = mla.num_splits(B, H, 2048, mla.MLA_DTYPE_BF16, 256)
            assert S >= 1
            if B * hg < 256:
                assert B * hg * S <= 256 and B * hg * (S + 1) > 256 or S == 32
            else:
                assert S == 1
    assert mla.num_splits(1, 128, 1001, mla.MLA_DTYPE_BF16, 256) == 16  # >= 2 tiles of 32 rows each
    # long selections on few sequences: the automatic plan stops at 64 splits
    # instead of failing (B = 1..3 would otherwise ask for 85..256)
    for B in (1, 2, 3):
        assert mla.num_splits(B, 32, 20000, mla.MLA_DTYPE_BF16, 256) == 64
        assert mla.workspace_size(B, 32, 20000, 1, 1, 256, 0) > 0
    assert mla.num_splits(4, 16, 65, mla.MLA_DTYPE_F32, 256) == 1
    a = mla.workspace_size(32, 128, 2048, 1, 1, 256, 0)
    b = mla.workspace_size(32, 128, 2048, 1, 1, 256, 16)
    assert 0 < a < b
    assert mla.workspace_size(0, 128, 2048, 1, 1, 256, 0) == 0
    assert mla.workspace_size(4, 128, 2048, 7, 1, 256, 0) == 0
    assert mla.workspace_size(4, 16, 64, 0, 0, 256, 2) == 0          # fp32 path does not split


def _params(mla, **kw):
    p = mla.DecodeParams()
    p.B, p.H, p.K = 2, 128, 16
    p.d_nope, p.d_rope, p.d_v, p.kv_rank = 128, 64, 128, 512
    p.max_cache_len, p.rope_table_len = 64, 64
    p.dtype_act = p.dtype_w = 1
    p.dtype_out = 0
    p.num_cus = 256
    p.softmax_scale = 0.1
    fake = 1 << 20                                   # never dereferenced: checks fail first
    for f in ("q_nope", "q_pe", "w_uk", "w_uv", "kv_cache", "pe_cache", "topk_indices", "cache_lens",
              "rope_table", "out", "workspace"):
        setattr(p, f, fake)
    p.q_nope_stride_b, p.q_nope_stride_h = 128 * 128, 128
    p.q_pe_stride_b, p.q_pe_stride_h = 128 * 64, 64
    p.w_uk_stride_h = p.w_uv_stride_h = 128 * 512
    p.kv_stride_b, p.kv_stride_t = 64 * 512, 512
    p.pe_stride_b, p.pe_stride_t = 64 * 64, 64
    p.idx_stride_b = 16
    p.out_stride_b, p.out_stride_h = 128 * 128, 128
    p.workspace_size = 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("field,value,code", [
    ("d_nope", 64, 2), ("kv_rank", 256, 2), ("dtype_act", 5, 2),
    ("B", 0, 1), ("K", 0, 1), ("q_nope", 0, 1), ("kv_cache", (1 << 20) + 2, 1),
    ("kv_stride_t", 513, 1), ("pe_stride_t", 32, 1), ("idx_stride_b", 8, 1),
    ("q_pe_stride_h", 68, 1), ("w_uk_stride_h", 128 * 512 + 4, 1),
    ("softmax_scale", -1.0, 1), ("num_splits", 65, 1), ("flags", 2, 1), ("max_cache_len", 0, 1),
    ("workspace_size", 0, 3),
])
def test_host_checks(mla, field, value, code):
    p = _params(mla, **{field: value})
    rc = mla.lib().mla_decode_attn(ctypes.byref(p), None)
    assert rc == code, mla.last_error()
    assert mla.last_error()


def test_rope_freqs_host_checks(mla):
    cfg = mla.rope_cfg(dict(W.ROPE_YARN, rope_dim=32))
    assert mla.lib().mla_rope_freqs(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), None) == mla.MLA_ERR_UNSUPPORTED
    cfg = mla.rope_cfg(W.ROPE_YARN)
    assert mla.lib().mla_rope_freqs(ctypes.byref(cfg), None, None) == mla.MLA_ERR_INVALID_ARG
    cfg = mla.rope_cfg(dict(W.ROPE_YARN, theta=0.5))
    assert mla.lib().mla_rope_freqs(ctypes.byref(cfg), ctypes.c_void_p(1 << 20), None) == mla.MLA_ERR_INVALID_ARG


def _topk_params(mla, **kw):
    p = mla.TopkParams()
    p.B, p.k, p.max_len, p.reserved = 4, 64, 1000, 0
    p.scores, p.score_stride = 1 << 20, 1000
    p.cache_lens = 1 << 21
    p.topk_indices, p.idx_stride = 1 << 22, 64
    for name, v in kw.items():
        setattr(p, name, v)
    return p


@pytest.mark.parametrize("field,value", [
    ("B", 0), ("k", 0), ("max_len", 0), ("max_len", (1 << 19) + 1), ("reserved", 1),
    ("scores", 0), ("cache_lens", 0), ("topk_indices", 0), ("score_stride", 999), ("idx_stride", 63),
])
def test_topk_host_checks(mla, field, value):
    p = _topk_params(mla, **{field: value})
    assert mla.lib().mla_topk(ctypes.byref(p), None) == mla.MLA_ERR_INVALID_ARG
    assert "mla_topk" in mla.last_error()
    assert mla.lib().mla_topk(None, None) == mla.MLA_ERR_INVALID_ARG


def _rope_params(mla, **kw):
    p = mla.RopeApplyParams()
    p.N, p.H, p.dtype, p.interleaved, p.table_len, p.reserved = 8, 4, mla.MLA_DTYPE_BF16, 0, 4096, 0
    p.x, p.x_stride_n, p.x_stride_h = 1 << 20, 256, 64
    p.y, p.y_stride_n, p.y_stride_h = 1 << 22, 256, 64
    p.positions, p.rope_table = 1 << 23, 1 << 24
    for name, v in kw.items():
        setattr(p, name, v)
    return p


@pytest.mark.parametrize("field,value", [
    ("N", 0), ("H", 0), ("H", 4097), ("table_len", 0), ("reserved", 1), ("dtype", 2), ("interleaved", 2),
    ("x", 0), ("y", 0), ("positions", 0), ("rope_table", 0),
    ("x_stride_h", 60), ("x_stride_h", 68), ("x_stride_n", 248), ("y_stride_n", 200), ("y_stride_h", 4),
    ("x", (1 << 20) + 8), ("rope_table", (1 << 24) + 4),
])
def test_rope_apply_host_checks(mla, field, value):
    p = _rope_params(mla, **{field: value})
    assert mla.lib().mla_rope_apply(ctypes.byref(p), None) == mla.MLA_ERR_INVALID_ARG
    assert "mla_rope_apply" in mla.last_error()


def test_rope_apply_host_checks_size_and_alias(mla):
    # N*H above 2^27 vectors
    p = _rope_params(mla, N=1 << 24, H=16, x_stride_n=1024, y_stride_n=1024)
    assert mla.lib().mla_rope_apply(ctypes.byref(p), None) == mla.MLA_ERR_INVALID_ARG
    # in place with different strides
    p = _rope_params(mla, y=1 << 20, y_stride_n=512)
    assert mla.lib().mla_rope_apply(ctypes.byref(p), None) == mla.MLA_ERR_INVALID_ARG
    assert mla.lib().mla_rope_apply(None, None) == mla.MLA_ERR_INVALID_ARG


_APPEND_OK = dict(kv_new=1 << 21, kv_new_stride_b=512, pe_new=1 << 22, pe_new_stride_b=64)


@pytest.mark.parametrize("change,code", [
    ({}, 3),                                              # valid append fields: fails later, on the workspace
    ({"pe_new": 0}, 1), ({"kv_new": 0}, 1),               # only one of the pair
    ({"kv_new": (1 << 21) + 8}, 1), ({"pe_new": (1 << 22) + 4}, 1),
    ({"kv_new_stride_b": 500}, 1), ({"pe_new_stride_b": 60}, 1), ({"kv_new_stride_b": 4}, 1),
    ({"pe_new_stride_b": -8}, 1),
])
def test_append_host_checks(mla, change, code):
    p = _params(mla, **{**_APPEND_OK, **change})
    rc = mla.lib().mla_decode_attn(ctypes.byref(p), None)
    assert rc == code, mla.last_error()


@pytest.mark.parametrize("extra", [[], ["--op", "topk"], ["--ab", "x.so", "y.so"]])
def test_bench_refuses_more_than_one_gpu(extra):
    # one GPU only: the refusal comes before any GPU work
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", *extra],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


# ---------------------------------------------------------------------------
# The binding's own checks (mla.build_params / topk / rope_apply): wrong
# dtypes, layouts and leading dimensions raise before any pointer reaches the
# library.  CPU tensors serve as stand-ins; the last check rejects them.
# ---------------------------------------------------------------------------
def _decode_tensors(B=2, H=4, L=16, K=8, act="bf16", wdt="f32"):
    import torch
    a = torch.bfloat16 if act == "bf16" else torch.float32
    w = torch.bfloat16 if wdt == "bf16" else torch.float32
    return dict(q_nope=torch.zeros(B, H, 128, dtype=a), q_pe=torch.zeros(B, H, 64, dtype=a),
                w_uk=torch.zeros(H, 128, 512, dtype=w), w_uv=torch.zeros(H, 128, 512, dtype=w),
                kv_cache=torch.zeros(B, L, 512, dtype=a), pe_cache=torch.zeros(B, L, 64, dtype=a),
                topk_indices=torch.zeros(B, K, dtype=torch.int32), cache_lens=torch.full((B,), L, dtype=torch.int32),
                rope_table=torch.zeros(64, 32, 2), softmax_scale=0.1, out=torch.zeros(B, H, 128),
                lse=torch.zeros(B, H))


def _bad_decode_cases():
    import torch
    return [
        ("q_pe_dtype", dict(q_pe=torch.zeros(2, 4, 64)), TypeError),            # fp32 q_pe, bf16 caches
        ("q_nope_dtype", dict(q_nope=torch.zeros(2, 4, 128)), TypeError),
        ("pe_cache_dtype", dict(pe_cache=torch.zeros(2, 16, 64)), TypeError),
        ("w_mixed", dict(w_uv=torch.zeros(4, 128, 512, dtype=torch.bfloat16)), TypeError),
        ("lse_dtype", dict(lse=torch.zeros(2, 4, dtype=torch.float64)), ValueError),
        ("lse_strided", dict(lse=torch.zeros(4, 2).t()), ValueError),
        ("lse_shape", dict(lse=torch.zeros(2, 3)), ValueError),
        ("out_short_b", dict(out=torch.zeros(1, 4, 128)), ValueError),
        ("out_short_h", dict(out=torch.zeros(2, 3, 128)), ValueError),
        ("idx_short_b", dict(topk_indices=torch.zeros(1, 8, dtype=torch.int32)), ValueError),
        ("idx_dtype", dict(topk_indices=torch.zeros(2, 8, dtype=torch.int64)), TypeError),
        ("lens_short", dict(cache_lens=torch.zeros(1, dtype=torch.int32)), ValueError),
        ("lens_dtype", dict(cache_lens=torch.zeros(2, dtype=torch.int64)), TypeError),
        ("kv_short_b", dict(kv_cache=torch.zeros(1, 16, 512, dtype=torch.bfloat16)), ValueError),
        ("pe_short_rows", dict(pe_cache=torch.zeros(2, 8, 64, dtype=torch.bfloat16)), ValueError),
        ("w_short_h", dict(w_uk=torch.zeros(3, 128, 512)), ValueError),
        ("q_pe_shape", dict(q_pe=torch.zeros(2, 3, 64, dtype=torch.bfloat16)), ValueError),
        ("table_dtype", dict(rope_table=torch.zeros(64, 32, 2, dtype=torch.float64)), ValueError),
        ("table_shape", dict(rope_table=torch.zeros(64, 64)), ValueError),
        ("act_f16", dict(kv_cache=torch.zeros(2, 16, 512, dtype=torch.float16)), TypeError),
        ("cpu_tensors", dict(), ValueError),                                     # all valid, but on the host
    ]


@pytest.mark.parametrize("case", range(21))
def test_binding_rejects_bad_decode_tensors(case):
    pytest.importorskip("torch")
    from decode_attention_absorbed_amd import mla as m
    name, change, exc = _bad_decode_cases()[case]
    t = {**_decode_tensors(), **change}
    with pytest.raises(exc):
        m.build_params(**t)


def test_binding_rejects_bad_topk_and_rope_tensors():
    torch = pytest.importorskip("torch")
    from decode_attention_absorbed_amd import mla as m
    scores = torch.zeros(4, 100)
    with pytest.raises(m.MLAError):
        m.topk(scores, torch.zeros(4, dtype=torch.int64), 8)                   # int64 lengths
    with pytest.raises(m.MLAError):
        m.topk(scores, torch.zeros(3, dtype=torch.int32), 8)                   # too few lengths
    with pytest.raises(m.MLAError):
        m.topk(scores, torch.zeros(4, dtype=torch.int32), 8)                   # host tensors
    x = torch.zeros(8, 4, 64, dtype=torch.bfloat16)
    table = torch.zeros(16, 32, 2)
    with pytest.raises(m.MLAError):
        m.rope_apply(x, torch.zeros(8, dtype=torch.int64), table, True)        # int64 positions
    with pytest.raises(m.MLAError):
        m.rope_apply(x, torch.zeros(8, dtype=torch.int32), table.double(), True)
    with pytest.raises(m.MLAError):
        m.rope_apply(x, torch.zeros(8, dtype=torch.int32), table, True)        # host tensors


def test_noalloc_size_limit_host(mla):
    # the allocation-free entry point refuses sizes beyond its buffer before
    # it touches the device (no GPU needed for this path)
    p = _params(mla, B=4096, K=2048, num_splits=8, idx_stride_b=2048)
    assert mla.lib().mla_decode_attn_noalloc(ctypes.byref(p), None) == mla.MLA_ERR_WORKSPACE
    assert "scratch" in mla.last_error()
    assert mla.lib().mla_decode_attn_noalloc(None, None) == mla.MLA_ERR_INVALID_ARG
    need = mla.workspace_size(128, 128, 2048, mla.MLA_DTYPE_BF16, mla.MLA_DTYPE_F32, 256, 0)
    assert 0 < need <= mla.MLA_NOALLOC_SCRATCH_BYTES     # the ragged batch fits
