"""ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: tensors are passed by device pointer, strides and
dtype codes; every step of the decode runs in the library's HIP kernels.
PyTorch provides device memory and the stream.  There is no fallback: if the
library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_INVALID_INDEX, MLA_ERR_HIP = range(6)
MLA_DTYPE_F32, MLA_DTYPE_BF16 = 0, 1
MLA_FLAG_VALIDATE = 1
MLA_BAD_INDEX_RANGE, MLA_BAD_DUPLICATE, MLA_BAD_EMPTY, MLA_BAD_CACHE_LEN = 1, 2, 4, 8
MLA_NUM_KERNELS = 3
KERNEL_NAMES = ("prep", "attention", "merge")


class RopeCfg(ctypes.Structure):
    _fields_ = [("rope_dim", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("original_seq_len", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("theta", ctypes.c_double), ("factor", ctypes.c_double),
                ("beta_fast", ctypes.c_double), ("beta_slow", ctypes.c_double),
                ("mscale", ctypes.c_double)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class DecodeParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("K", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("kv_rank", ctypes.c_int32), ("max_cache_len", ctypes.c_int32),
                ("rope_table_len", ctypes.c_int32),
                ("dtype_act", ctypes.c_int32), ("dtype_w", ctypes.c_int32), ("dtype_out", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("softmax_scale", ctypes.c_float),
                ("q_nope", _P), ("q_nope_stride_b", _I64), ("q_nope_stride_h", _I64),
                ("q_pe", _P), ("q_pe_stride_b", _I64), ("q_pe_stride_h", _I64),
                ("w_uk", _P), ("w_uk_stride_h", _I64),
                ("w_uv", _P), ("w_uv_stride_h", _I64),
                ("kv_cache", _P), ("kv_stride_b", _I64), ("kv_stride_t", _I64),
                ("pe_cache", _P), ("pe_stride_b", _I64), ("pe_stride_t", _I64),
                ("topk_indices", _P), ("idx_stride_b", _I64),
                ("cache_lens", _P),
                ("rope_table", _P),
                ("out", _P), ("out_stride_b", _I64), ("out_stride_h", _I64),
                ("lse_out", _P),
                ("workspace", _P), ("workspace_size", ctypes.c_size_t),
                ("profile_events", _P),
                ("validate_status", ctypes.c_uint32), ("reserved0", ctypes.c_uint32),
                ("kv_new", _P), ("kv_new_stride_b", _I64),
                ("pe_new", _P), ("pe_new_stride_b", _I64)]


class TopkParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("reserved", ctypes.c_int32),
                ("scores", _P), ("score_stride", _I64),
                ("cache_lens", _P),
                ("topk_indices", _P), ("idx_stride", _I64)]


class RopeApplyParams(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("H", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("interleaved", ctypes.c_int32), ("table_len", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("x", _P), ("x_stride_n", _I64), ("x_stride_h", _I64),
                ("y", _P), ("y_stride_n", _I64), ("y_stride_h", _I64),
                ("positions", _P), ("rope_table", _P)]


_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with decode_attention_absorbed_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.mla_rope_freqs.argtypes = [ctypes.POINTER(RopeCfg), _P, _P]
        L.mla_rope_freqs.restype = ctypes.c_int
        L.mla_softmax_scale.argtypes = [ctypes.c_int, ctypes.POINTER(RopeCfg)]
        L.mla_softmax_scale.restype = ctypes.c_double
        L.mla_decode_num_splits.argtypes = [ctypes.c_int] * 5
        L.mla_decode_num_splits.restype = ctypes.c_int
        L.mla_decode_workspace_size.argtypes = [ctypes.c_int] * 7
        L.mla_decode_workspace_size.restype = ctypes.c_size_t
        L.mla_decode_attn.argtypes = [ctypes.POINTER(DecodeParams), _P]
        L.mla_decode_attn.restype = ctypes.c_int
        L.mla_decode_attn_noalloc.argtypes = [ctypes.POINTER(DecodeParams), _P]
        L.mla_decode_attn_noalloc.restype = ctypes.c_int
        L.mla_decode_params_size.argtypes = []
        L.mla_decode_params_size.restype = ctypes.c_size_t
        L.mla_topk.argtypes = [ctypes.POINTER(TopkParams), _P]
        L.mla_topk.restype = ctypes.c_int
        L.mla_rope_apply.argtypes = [ctypes.POINTER(RopeApplyParams), _P]
        L.mla_rope_apply.restype = ctypes.c_int
        L.mla_last_error.argtypes = []
        L.mla_last_error.restype = ctypes.c_char_p
        if L.mla_decode_params_size() != ctypes.sizeof(DecodeParams):
            raise RuntimeError("mla_decode_params_t layout mismatch between the binding and the library")
        _lib = L
    return _lib


def last_error() -> str:
    return lib().mla_last_error().decode()


class MLAError(RuntimeError):
    def __init__(self, code, msg, status=0):
        super().__init__(f"mla error {code}: {msg}")
        self.code = code
        self.status = status


def rope_cfg(rope: dict) -> RopeCfg:
    return RopeCfg(rope_dim=int(rope["rope_dim"]), max_seq_len=int(rope["max_seq_len"]),
                   original_seq_len=int(rope["original_seq_len"]), reserved=0,
                   theta=float(rope["theta"]), factor=float(rope["factor"]),
                   beta_fast=float(rope["beta_fast"]), beta_slow=float(rope["beta_slow"]),
                   mscale=float(rope["mscale"]))


def softmax_scale(qk_head_dim: int, rope: dict) -> float:
    cfg = rope_cfg(rope)
    return lib().mla_softmax_scale(qk_head_dim, ctypes.byref(cfg))


def num_splits(B, H, K, dtype_act, num_cus=0) -> int:
    return lib().mla_decode_num_splits(B, H, K, dtype_act, num_cus)


def workspace_size(B, H, K, dtype_act, dtype_w, num_cus=0, num_splits=0) -> int:
    return lib().mla_decode_workspace_size(B, H, K, dtype_act, dtype_w, num_cus, num_splits)


# ---------------------------------------------------------------------------
# torch-facing helpers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MLA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def rope_freqs(rope: dict, table=None, stream=None):
    """Fill (or allocate) the fp32 [max_seq_len, 32, 2] rotation table."""
    torch = _torch()
    if table is None:
        table = torch.empty((int(rope["max_seq_len"]), int(rope["rope_dim"]) // 2, 2),
                            dtype=torch.float32, device="cuda")
    cfg = rope_cfg(rope)
    rc = lib().mla_rope_freqs(ctypes.byref(cfg), ctypes.c_void_p(table.data_ptr()), _stream_handle(stream))
    if rc != MLA_OK:
        raise MLAError(rc, last_error())
    return table


def _inner_contig(name, t, width):
    if t.shape[-1] != width or t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be {width} and contiguous")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (the library takes device pointers)")


def _rope_table_ok(rope_table):
    torch = _torch()
    if rope_table.dtype != torch.float32 or rope_table.dim() != 3 or tuple(rope_table.shape[1:]) != (32, 2) \
            or not rope_table.is_contiguous():
        raise ValueError("rope_table must be a contiguous float32 [T, 32, 2] table from rope_freqs")


def _check_decode_tensors(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices, cache_lens, rope_table,
                          out, lse):
    """Shapes, dtypes and layouts the header requires of the decode step's
    tensors; raises before anything is passed to the library."""
    torch = _torch()
    dims = (("q_nope", q_nope, 3), ("q_pe", q_pe, 3), ("w_uk", w_uk, 3), ("w_uv", w_uv, 3),
            ("kv_cache", kv_cache, 3), ("pe_cache", pe_cache, 3), ("topk_indices", topk_indices, 2),
            ("cache_lens", cache_lens, 1), ("out", out, 3))
    for name, t, d in dims:
        if t.dim() != d:
            raise ValueError(f"{name} must have {d} dimensions, got shape {tuple(t.shape)}")
    B, H = q_nope.shape[0], q_nope.shape[1]
    for name, t, w in (("q_nope", q_nope, 128), ("q_pe", q_pe, 64), ("w_uk", w_uk, 512), ("w_uv", w_uv, 512),
                       ("kv_cache", kv_cache, 512), ("pe_cache", pe_cache, 64), ("out", out, 128)):
        _inner_contig(name, t, w)
    # one activation dtype for the queries and both caches (dtype_act)
    act = kv_cache.dtype
    if act not in (torch.bfloat16, torch.float32):
        raise TypeError(f"kv_cache must be bfloat16 or float32, got {act}")
    for name, t in (("q_nope", q_nope), ("q_pe", q_pe), ("pe_cache", pe_cache)):
        if t.dtype != act:
            raise TypeError(f"{name} is {t.dtype} but kv_cache is {act}: queries and caches share one dtype")
    if w_uk.dtype not in (torch.bfloat16, torch.float32) or w_uv.dtype != w_uk.dtype:
        raise TypeError("w_uk and w_uv must both be bfloat16 or both float32")
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    # leading dimensions: B sequences, H heads
    if tuple(q_pe.shape[:2]) != (B, H):
        raise ValueError(f"q_pe must be [{B}, {H}, 64] like q_nope, got {tuple(q_pe.shape)}")
    for name, t in (("w_uk", w_uk), ("w_uv", w_uv)):
        if t.shape[0] < H or t.shape[1] != 128 or t.stride(1) != 512:
            raise ValueError(f"{name} must be [H={H}, 128, 512] with contiguous rows, got {tuple(t.shape)}")
    if kv_cache.shape[0] < B or pe_cache.shape[0] < B:
        raise ValueError(f"kv_cache / pe_cache must hold B={B} sequences")
    if pe_cache.shape[1] < kv_cache.shape[1]:
        raise ValueError("pe_cache must have as many rows per sequence as kv_cache")
    if topk_indices.dtype != torch.int32 or cache_lens.dtype != torch.int32:
        raise TypeError("topk_indices and cache_lens must be int32")
    if topk_indices.shape[0] < B or topk_indices.stride(1) != 1:
        raise ValueError(f"topk_indices must be [B={B}, K] with contiguous rows")
    if cache_lens.shape[0] < B or cache_lens.stride(0) != 1:
        raise ValueError(f"cache_lens must be a contiguous int32 [B={B}]")
    if out.shape[0] < B or out.shape[1] < H:
        raise ValueError(f"out must be [B={B}, H={H}, 128], got {tuple(out.shape)}")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H) or not lse.is_contiguous()):
        raise ValueError(f"lse must be a contiguous float32 [B={B}, H={H}] tensor")
    _rope_table_ok(rope_table)


def build_params(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices, cache_lens, rope_table,
                 softmax_scale, out, lse=None, workspace=None, num_splits=0, num_cus=0, validate=False,
                 events=None, kv_new=None, pe_new=None) -> DecodeParams:
    """Fill mla_decode_params_t from torch tensors (shapes as in the header).
    kv_new [B, 512] and pe_new [B, 64] (both or neither) switch on the fused
    append of each sequence's row p_b = L_b - 1 into kv_cache / pe_cache.
    Every tensor must live on the GPU; shapes, dtypes and layouts are checked
    first (ValueError / TypeError)."""
    _check_decode_tensors(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices, cache_lens, rope_table,
                          out, lse)
    B, H = q_nope.shape[0], q_nope.shape[1]
    K = topk_indices.shape[1]
    p = DecodeParams()
    p.B, p.H, p.K = B, H, K
    p.d_nope, p.d_rope, p.d_v, p.kv_rank = 128, 64, 128, 512
    p.max_cache_len = kv_cache.shape[1]
    p.rope_table_len = rope_table.shape[0]
    p.dtype_act = _dtype_code(kv_cache)
    p.dtype_w = _dtype_code(w_uk)
    p.dtype_out = _dtype_code(out)
    p.num_cus = num_cus
    p.num_splits = num_splits
    p.flags = MLA_FLAG_VALIDATE if validate else 0
    p.softmax_scale = softmax_scale
    p.q_nope, p.q_nope_stride_b, p.q_nope_stride_h = q_nope.data_ptr(), q_nope.stride(0), q_nope.stride(1)
    p.q_pe, p.q_pe_stride_b, p.q_pe_stride_h = q_pe.data_ptr(), q_pe.stride(0), q_pe.stride(1)
    p.w_uk, p.w_uk_stride_h = w_uk.data_ptr(), w_uk.stride(0)
    p.w_uv, p.w_uv_stride_h = w_uv.data_ptr(), w_uv.stride(0)
    p.kv_cache, p.kv_stride_b, p.kv_stride_t = kv_cache.data_ptr(), kv_cache.stride(0), kv_cache.stride(1)
    p.pe_cache, p.pe_stride_b, p.pe_stride_t = pe_cache.data_ptr(), pe_cache.stride(0), pe_cache.stride(1)
    p.topk_indices, p.idx_stride_b = topk_indices.data_ptr(), topk_indices.stride(0)
    p.cache_lens = cache_lens.data_ptr()
    p.rope_table = rope_table.data_ptr()
    p.out, p.out_stride_b, p.out_stride_h = out.data_ptr(), out.stride(0), out.stride(1)
    p.lse_out = lse.data_ptr() if lse is not None else None
    if workspace is not None:
        p.workspace, p.workspace_size = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    p.profile_events = events
    if (kv_new is None) != (pe_new is None):
        raise ValueError("kv_new and pe_new go together")
    if kv_new is not None:
        _inner_contig("kv_new", kv_new, 512)
        _inner_contig("pe_new", pe_new, 64)
        if kv_new.dtype != kv_cache.dtype or pe_new.dtype != kv_cache.dtype:
            raise TypeError("kv_new / pe_new must have the caches' dtype")
        if kv_new.dim() != 2 or pe_new.dim() != 2 or kv_new.shape[0] < B or pe_new.shape[0] < B:
            raise ValueError(f"kv_new / pe_new must be [B={B}, 512] / [B={B}, 64]")
        p.kv_new, p.kv_new_stride_b = kv_new.data_ptr(), kv_new.stride(0)
        p.pe_new, p.pe_new_stride_b = pe_new.data_ptr(), pe_new.stride(0)
    if workspace is not None and workspace.dtype != _torch().uint8:
        raise TypeError("workspace must be a uint8 tensor")
    _on_gpu(q_nope=q_nope, q_pe=q_pe, w_uk=w_uk, w_uv=w_uv, kv_cache=kv_cache, pe_cache=pe_cache,
            topk_indices=topk_indices, cache_lens=cache_lens, rope_table=rope_table, out=out, lse=lse,
            workspace=workspace, kv_new=kv_new, pe_new=pe_new)
    return p


def decode_attn(params: DecodeParams, stream=None, check=True) -> int:
    """Run mla_decode_attn; raises MLAError on a non-zero code when check."""
    rc = lib().mla_decode_attn(ctypes.byref(params), _stream_handle(stream))
    if check and rc != MLA_OK:
        raise MLAError(rc, last_error(), params.validate_status)
    return rc


MLA_NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_attn_noalloc(params: DecodeParams, stream=None, check=True) -> int:
    """Run mla_decode_attn_noalloc (scratch in the library's own per-device
    buffer; params.workspace is ignored); raises MLAError when check."""
    rc = lib().mla_decode_attn_noalloc(ctypes.byref(params), _stream_handle(stream))
    if check and rc != MLA_OK:
        raise MLAError(rc, last_error(), params.validate_status)
    return rc


def decode(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices, cache_lens, rope_table,
           softmax_scale, out=None, lse=None, workspace=None, out_dtype=None, num_splits=0,
           validate=False, stream=None, with_lse=True, kv_new=None, pe_new=None):
    """Allocate what is missing, run one decode step; returns (out, lse).
    With kv_new / pe_new the step first appends each sequence's new row."""
    torch = _torch()
    B, H = q_nope.shape[0], q_nope.shape[1]
    if out is None:
        out = torch.empty((B, H, 128), dtype=out_dtype or torch.float32, device=q_nope.device)
    if lse is None and with_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
    if workspace is None:
        n = workspace_size(B, H, topk_indices.shape[1], _dtype_code(kv_cache), _dtype_code(w_uk), 0, num_splits)
        if n == 0:
            raise MLAError(MLA_ERR_INVALID_ARG, "no workspace size for these sizes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q_nope.device)
    p = build_params(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices, cache_lens, rope_table,
                     softmax_scale, out, lse, workspace, num_splits=num_splits, validate=validate,
                     kv_new=kv_new, pe_new=pe_new)
    decode_attn(p, stream)
    return out, lse


def topk(scores, cache_lens, k, out=None, stream=None):
    """mla_topk: int32 [B, k] ascending positions of the min(k, L_b) largest
    scores per row (-1 padded).  scores: float32 [B, L] (inner dim contiguous),
    cache_lens: int32 [B]; all on the device."""
    torch = _torch()
    if scores.dim() != 2:
        raise MLAError(MLA_ERR_INVALID_ARG, "scores must be [B, L]")
    B, L = scores.shape
    if scores.dtype != torch.float32 or scores.stride(1) != 1:
        raise MLAError(MLA_ERR_INVALID_ARG, "scores must be float32 with a contiguous inner dimension")
    if cache_lens.dtype != torch.int32 or cache_lens.dim() != 1 or cache_lens.shape[0] < B \
            or cache_lens.stride(0) != 1:
        raise MLAError(MLA_ERR_INVALID_ARG, f"cache_lens must be a contiguous int32 [B={B}]")
    if out is None:
        out = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    if out.dtype != torch.int32 or out.dim() != 2 or out.shape[0] < B or out.shape[1] < k or out.stride(1) != 1:
        raise MLAError(MLA_ERR_INVALID_ARG, f"out must be int32 [B={B}, >={k}] with contiguous rows")
    try:
        _on_gpu(scores=scores, cache_lens=cache_lens, out=out)
    except ValueError as e:
        raise MLAError(MLA_ERR_INVALID_ARG, str(e))
    p = TopkParams()
    p.B, p.k, p.max_len, p.reserved = B, k, L, 0
    p.scores, p.score_stride = scores.data_ptr(), scores.stride(0)
    p.cache_lens = cache_lens.data_ptr()
    p.topk_indices, p.idx_stride = out.data_ptr(), out.stride(0)
    rc = lib().mla_topk(ctypes.byref(p), _stream_handle(stream))
    if rc != MLA_OK:
        raise MLAError(rc, last_error())
    return out


def rope_apply(x, positions, rope_table, interleaved, out=None, stream=None):
    """mla_rope_apply: rotate every 64-wide vector of x ([N, 64] or [N, H, 64],
    bf16 or float32, last dim contiguous) at positions[n] (int32 [N]) with the
    table from rope_freqs.  interleaved=True pairs (2i, 2i+1), False pairs
    (i, i+32).  out may be x itself (in place); by default a new tensor."""
    torch = _torch()
    squeeze = x.dim() == 2
    xv = x.unsqueeze(1) if squeeze else x
    if xv.dim() != 3 or xv.shape[2] != 64 or xv.stride(2) != 1:
        raise MLAError(MLA_ERR_INVALID_ARG, "x must be [N, 64] or [N, H, 64] with a contiguous last dim")
    if x.dtype == torch.bfloat16:
        dt = MLA_DTYPE_BF16
    elif x.dtype == torch.float32:
        dt = MLA_DTYPE_F32
    else:
        raise MLAError(MLA_ERR_INVALID_ARG, "x must be bfloat16 or float32")
    if positions.dtype != torch.int32 or positions.dim() != 1 or positions.shape[0] < xv.shape[0] \
            or positions.stride(0) != 1:
        raise MLAError(MLA_ERR_INVALID_ARG, f"positions must be a contiguous int32 [N={xv.shape[0]}]")
    try:
        _rope_table_ok(rope_table)
    except ValueError as e:
        raise MLAError(MLA_ERR_INVALID_ARG, str(e))
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    if out.shape != x.shape or out.dtype != x.dtype:
        raise MLAError(MLA_ERR_INVALID_ARG, "out must match x in shape and dtype")
    try:
        _on_gpu(x=x, positions=positions, rope_table=rope_table, out=out)
    except ValueError as e:
        raise MLAError(MLA_ERR_INVALID_ARG, str(e))
    yv = out.unsqueeze(1) if squeeze else out
    p = RopeApplyParams()
    p.N, p.H = xv.shape[0], xv.shape[1]
    p.dtype, p.interleaved, p.table_len, p.reserved = dt, 1 if interleaved else 0, rope_table.shape[0], 0
    p.x, p.x_stride_n, p.x_stride_h = xv.data_ptr(), xv.stride(0), xv.stride(1)
    p.y, p.y_stride_n, p.y_stride_h = yv.data_ptr(), yv.stride(0), yv.stride(1)
    p.positions, p.rope_table = positions.data_ptr(), rope_table.data_ptr()
    rc = lib().mla_rope_apply(ctypes.byref(p), _stream_handle(stream))
    if rc != MLA_OK:
        raise MLAError(rc, last_error())
    return out
