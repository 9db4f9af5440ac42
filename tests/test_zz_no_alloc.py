"""mla_decode_attn_noalloc, through the C ABI: the same outputs as
mla_decode_attn on the same inputs, bit for bit, on two calls in a row (the
second with smaller sizes, so stale contents of the shared scratch buffer
would show), and the size limit refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from decode_attention_absorbed_amd import mla  # noqa: E402
from gpu_util import Dev, oracle_ref, rel_l2_rows  # noqa: E402


def _both(dev, num_splits=0):
    """(out, lse) of mla_decode_attn with a caller workspace, then of
    mla_decode_attn_noalloc, on the same inputs."""
    w = dev.w
    res = []
    for noalloc in (False, True):
        out = torch.full((w.B, w.H, 128), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
        ws = None
        if not noalloc:
            n = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(dev.kv), mla._dtype_code(dev.w_uk), 0,
                                   num_splits)
            ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                             dev.rope_table, dev.scale, out, lse, ws, num_splits=num_splits)
        if noalloc:
            assert p.workspace is None
            mla.decode_attn_noalloc(p)
        else:
            mla.decode_attn(p)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big = W.build("noalloc_big", 16, 128, [3000, 64, 1500, 777, 4096, 1, 2048, 300] * 2, 1024, "bf16", "f32",
                  W.ROPE_YARN, seed=61)
    small = W.build("noalloc_small", 3, 64, [500, 70, 1200], 256, "bf16", "bf16", W.ROPE_YARN, seed=62)
    for w, splits in ((big, 0), (small, 3)):
        print(f"[{w.name}] B={w.B} H={w.H} K={w.K} splits={splits}", flush=True)
        dev = Dev(w)
        (o0, l0), (o1, l1) = _both(dev, splits)
        assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        # and the parity bar against the oracle, on a few sequences
        batch = [0, w.B - 1]
        ref, ref_lse = oracle_ref(w, batch=batch)
        assert rel_l2_rows(o1.cpu().numpy()[batch], ref).max() <= 1e-2
        assert np.abs(l1.cpu().numpy()[batch] - ref_lse).max() <= 1e-2


def test_noalloc_fp32_path():
    w = W.build("noalloc_f32", 2, 16, [300, 65], 128, "f32", "f32", W.ROPE_PLAIN, seed=63)
    dev = Dev(w)
    (o0, l0), (o1, l1) = _both(dev)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_noalloc_refuses_sizes_beyond_its_buffer():
    w = W.build("noalloc_ref", 2, 128, [300, 65], 128, "bf16", "bf16", W.ROPE_YARN, seed=64)
    dev = Dev(w)
    out = torch.zeros((w.B, w.H, 128), dtype=torch.float32, device="cuda")
    p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                         dev.rope_table, dev.scale, out, None, None)
    # claim a batch whose split partials alone exceed the buffer; the size
    # check comes first, so nothing is read or launched
    p.B, p.K, p.num_splits, p.num_cus = 4096, 2048, 8, 256
    rc = mla.decode_attn_noalloc(p, check=False)
    assert rc == mla.MLA_ERR_WORKSPACE
    assert "scratch" in mla.last_error()
    torch.cuda.synchronize()
    assert (out == 0).all()
