"""The fused append of mla_decode_attn (kv_new / pe_new set): each sequence's
row p_b = L_b - 1 is written before it is attended to.  Checked against the
oracle's cache_append followed by its decode step:

* the latent row is a copy: bit-exact;
* the rotary row is pe_new rotated at p_b: per-row relative L2 1e-2 (bf16
  caches) or 1e-5 (fp32), against the fp64 rotation;
* every other cache row is untouched: bit-exact;
* the step's output: per-row relative L2 1e-2 (bf16) / 1e-5 (fp32) against
  the oracle on the appended caches.
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
from gpu_util import Dev, rel_l2_rows  # noqa: E402


def _run_append(w, kv_new, pe_new, validate=False, check=True):
    dev = Dev(w)
    act = dev.kv.dtype
    kn = torch.from_numpy(kv_new).to(act).cuda()
    pn = torch.from_numpy(pe_new).to(act).cuda()
    kv_before, pe_before = dev.kv.clone(), dev.pe.clone()
    out = torch.empty((w.B, w.H, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    n = mla.workspace_size(w.B, w.H, w.K, mla._dtype_code(dev.kv), mla._dtype_code(dev.w_uk), 0, 0)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    p = mla.build_params(dev.q_nope, dev.q_pe, dev.w_uk, dev.w_uv, dev.kv, dev.pe, dev.idx, dev.lens,
                         dev.rope_table, dev.scale, out, lse, ws, validate=validate, kv_new=kn, pe_new=pn)
    rc = mla.decode_attn(p, check=check)
    torch.cuda.synchronize()
    return dict(out=out, rc=rc, status=p.validate_status, kv=dev.kv, pe=dev.pe, kv0=kv_before, pe0=pe_before)


def _check(w, kv_new, pe_new, bar, name):
    print(f"[append {name}] B={w.B} H={w.H} lens={list(w.cache_lens)} {w.dtype_act}", flush=True)
    r = _run_append(w, kv_new, pe_new)
    cfg = oracle.RopeConfig(**w.rope)
    C2, R2 = oracle.cache_append(w.kv_cache, w.pe_cache, kv_new, pe_new, w.cache_lens, cfg)
    kv = r["kv"].float().cpu().numpy()
    pe = r["pe"].float().cpu().numpy()
    kv0 = r["kv0"].float().cpu().numpy()
    pe0 = r["pe0"].float().cpu().numpy()
    for b, L in enumerate(w.cache_lens):
        p = int(L) - 1
        assert np.array_equal(kv[b, p], kv_new[b].astype(np.float32)), b
        err = np.linalg.norm(pe[b, p] - R2[b, p]) / np.linalg.norm(R2[b, p])
        assert err <= bar, (b, err)
        keep = np.ones(w.L_max, dtype=bool)
        keep[p] = False
        assert np.array_equal(kv[b, keep], kv0[b, keep]) and np.array_equal(pe[b, keep], pe0[b, keep]), b
    ref, _ = oracle.decode_attention(w.q_nope, w.q_pe, w.w_uk, w.w_uv, C2, R2, w.topk_indices, w.cache_lens, cfg)
    err = rel_l2_rows(r["out"].cpu().numpy(), ref).max()
    print(f"  max rel L2 {err:.3e}", flush=True)
    assert err <= bar


def test_append_bf16_ragged():
    lens = [1, 2, 700, 2048, 2049, 3000]
    w = W.build("append", 6, 128, lens, 512, "bf16", "bf16", W.ROPE_YARN, seed=1301)
    kv_new, pe_new = W.new_rows(6, "bf16", 1302)
    _check(w, kv_new, pe_new, 1e-2, "bf16 ragged")


def test_append_fp32():
    w = W.build("append32", 3, 16, [5, 65, 300], 64, "f32", "f32", W.ROPE_PLAIN, seed=1303)
    kv_new, pe_new = W.new_rows(3, "f32", 1304)
    _check(w, kv_new, pe_new, 1e-5, "fp32")


def test_append_only_new_row_selected():
    # the new row alone: out[b, h] = W_UV[h] kv_new[b]
    w = W.build("append1", 4, 32, [10, 4096, 333, 16384], 8, "bf16", "bf16", W.ROPE_YARN, seed=1305)
    w.topk_indices[:] = -1
    w.topk_indices[:, 3] = w.cache_lens - 1
    kv_new, pe_new = W.new_rows(4, "bf16", 1306)
    r = _run_append(w, kv_new, pe_new)
    want = np.einsum("hdc,bc->bhd", w.w_uv.astype(np.float64), kv_new.astype(np.float64))
    err = rel_l2_rows(r["out"].cpu().numpy(), want).max()
    print(f"[append only-new-row] max rel L2 {err:.3e}", flush=True)
    assert err <= 1e-2


def test_append_skipped_for_invalid_cache_length():
    # L_b beyond the cache: flagged in validate mode, and nothing is written
    w = W.build("append_bad", 2, 16, [40, 50], 16, "bf16", "bf16", W.ROPE_YARN, seed=1307, L_max=64)
    w.cache_lens = np.array([40, 65], dtype=np.int32)
    w.topk_indices[1, :] = -1
    w.topk_indices[1, 0] = 3
    kv_new, pe_new = W.new_rows(2, "bf16", 1308)
    r = _run_append(w, kv_new, pe_new, validate=True, check=False)
    assert r["rc"] == mla.MLA_ERR_INVALID_INDEX and (r["status"] & 8)
    kv, kv0 = r["kv"].float().cpu().numpy(), r["kv0"].float().cpu().numpy()
    pe, pe0 = r["pe"].float().cpu().numpy(), r["pe0"].float().cpu().numpy()
    assert np.array_equal(kv[1], kv0[1]) and np.array_equal(pe[1], pe0[1])
    assert np.array_equal(kv[0, 39], kv_new[0])
