"""Helpers shared by the GPU tests: upload a workload, run one decode step
through the C ABI, and run the oracle on the same inputs."""
import numpy as np

import oracle
import workloads as W


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


class Dev:
    """A workload's inputs on the GPU (torch tensors) plus the rotation table."""

    def __init__(self, w: W.Workload, rope_table=None):
        import torch
        from decode_attention_absorbed_amd import mla
        act, wt = torch_dtype(w.dtype_act), torch_dtype(w.dtype_w)
        cuda = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
        self.w = w
        self.q_nope = cuda(w.q_nope, act)
        self.q_pe = cuda(w.q_pe, act)
        self.w_uk = cuda(w.w_uk, wt)
        self.w_uv = cuda(w.w_uv, wt)
        self.kv = cuda(w.kv_cache, act)
        self.pe = cuda(w.pe_cache, act)
        self.idx = torch.from_numpy(w.topk_indices).cuda()
        self.lens = torch.from_numpy(w.cache_lens).cuda()
        self.rope_table = rope_table if rope_table is not None else mla.rope_freqs(w.rope)
        self.scale = mla.softmax_scale(192, w.rope)

    def run(self, out_dtype=None, num_splits=0, validate=False, kv=None, pe=None, idx=None, lens=None,
            w_uk=None, w_uv=None, check=True):
        """One decode step; returns (out, lse, status) as torch tensors."""
        import torch
        from decode_attention_absorbed_amd import mla
        w = self.w
        out = torch.empty((w.B, w.H, 128), dtype=out_dtype or torch.float32, device="cuda")
        lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
        kv = self.kv if kv is None else kv
        idx = self.idx if idx is None else idx
        n = mla.workspace_size(w.B, w.H, idx.shape[1], mla._dtype_code(kv), mla._dtype_code(self.w_uk), 0,
                               num_splits)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        p = mla.build_params(self.q_nope, self.q_pe, self.w_uk if w_uk is None else w_uk,
                             self.w_uv if w_uv is None else w_uv, kv, self.pe if pe is None else pe,
                             idx, self.lens if lens is None else lens, self.rope_table, self.scale, out, lse,
                             ws, num_splits=num_splits, validate=validate)
        rc = mla.decode_attn(p, check=check)
        torch.cuda.synchronize()
        return out, lse, (rc, p.validate_status)


def oracle_ref(w: W.Workload, batch=None, heads=None, form="restricted"):
    cfg = oracle.RopeConfig(**w.rope)
    return oracle.decode_attention(w.q_nope, w.q_pe, w.w_uk, w.w_uv, w.kv_cache, w.pe_cache,
                                   w.topk_indices, w.cache_lens, cfg, form=form, batch=batch, heads=heads)


def rel_l2_rows(got, ref):
    """Per-row relative L2 error (rows = last axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
