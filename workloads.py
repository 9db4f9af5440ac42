"""Seeded synthetic inputs for the absorbed-MLA sparse decode step.

This module only draws random numbers, rounds them to the storage dtype and
builds index sets.  It holds none of the attention arithmetic: both the HIP
path and the CPU oracle consume what it returns, and neither imports the other.

Five workloads, shaped like the atlas pages' decode example (page "Attention
weights": 128 heads, rows of 576 = latent 512 + rotary 64, L = P + 1 keys for
P = 1000 cached positions) and the batched sparse decodes it generalises to:

  tiny      B=1,   H=16,  L=65,    all positions,  fp32 everything, no YaRN
  page      B=1,   H=128, L=1001,  all positions,  bf16, YaRN (max_seq_len 16384)
  batched   B=32,  H=128, L=4096,  top-k 2048 random incl. newest, bf16
  long      B=64,  H=128, L=16384, top-k 2048 random incl. newest, bf16
  ragged    B=128, H=128, L_b ~ U{1024..16384}, k_b = min(2048, L_b);
            even b random, odd b the most recent k_b; bf16 caches and
            queries, fp32 weights; index rows -1 padded to width 2048.

Value recipe: numpy PCG64 ``default_rng(seed)``; q and both caches N(0, 1);
W_UK and W_UV N(0, 1/512); values rounded to bf16 by round-to-nearest-even
where the dtype is bf16 (arrays stay float32 holding bf16-exact values).
Draw order: cache lengths (ragged only), q_nope, q_pe, W_UK, W_UV, latent
cache (sequence by sequence, rows < L_b), rope-key cache (same), indices.

The rope-key cache is drawn directly as N(0, 1).  A cached rope key is a raw
N(0, 1) key rotated at its own position; rotating an isotropic Gaussian pair
gives an isotropic Gaussian pair, so the cached keys have exactly the
distribution drawn here, and no rotation arithmetic is needed in this module.
Rows at or beyond L_b are zero.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_NOPE, D_ROPE, D_V, KV_RANK = 128, 64, 128, 512

# Rotary settings as plain numbers (the pages' ModelArgs defaults; the tiny
# workload keeps max_seq_len at the original 4096, so no interpolation).
ROPE_YARN = dict(rope_dim=64, theta=10000.0, max_seq_len=16384, original_seq_len=4096,
                 factor=40.0, beta_fast=32.0, beta_slow=1.0, mscale=1.0)
ROPE_PLAIN = dict(ROPE_YARN, max_seq_len=4096)


@dataclass
class Workload:
    name: str
    B: int
    H: int
    L_max: int            # rows per sequence in the caches
    K: int                # width of the index array
    dtype_act: str        # "f32" or "bf16": queries and caches
    dtype_w: str          # "f32" or "bf16": W_UK, W_UV
    rope: dict
    seed: int
    q_nope: np.ndarray = field(repr=False, default=None)     # [B, H, 128] float32
    q_pe: np.ndarray = field(repr=False, default=None)       # [B, H, 64]
    w_uk: np.ndarray = field(repr=False, default=None)       # [H, 128, 512]
    w_uv: np.ndarray = field(repr=False, default=None)       # [H, 128, 512]
    kv_cache: np.ndarray = field(repr=False, default=None)   # [B, L_max, 512]
    pe_cache: np.ndarray = field(repr=False, default=None)   # [B, L_max, 64]
    topk_indices: np.ndarray = field(repr=False, default=None)  # [B, K] int32
    cache_lens: np.ndarray = field(repr=False, default=None)    # [B] int32

    def selected_rows(self) -> int:
        """Number of distinct selected positions over the batch."""
        n = 0
        for b in range(self.B):
            row = self.topk_indices[b]
            n += np.unique(row[row >= 0]).size
        return n


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), in place;
    the result stays float32 and is exactly representable in bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    flat = a.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        u = flat[s:s + step].view(np.uint32)
        u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        u &= np.uint32(0xFFFF0000)
    return a


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def random_selection(rng, L_b: int, k: int) -> np.ndarray:
    """The newest position plus k-1 distinct draws from [0, L_b - 1), in a
    random order (as a top-k by score would list them)."""
    if k >= L_b:
        return rng.permutation(L_b).astype(np.int32)
    picks = rng.choice(L_b - 1, size=k - 1, replace=False)
    sel = np.concatenate([picks, [L_b - 1]]).astype(np.int32)
    return rng.permutation(sel).astype(np.int32)


def recent_selection(L_b: int, k: int) -> np.ndarray:
    """The k most recent positions, ascending."""
    return np.arange(L_b - k, L_b, dtype=np.int32)


def build(name, B, H, cache_lens, K, dtype_act, dtype_w, rope, seed, L_max=None,
          selection="random", k_per_seq=None) -> Workload:
    """Draw one workload.  ``cache_lens`` is a list of L_b (or None to draw
    U{1024..16384} first, as the ragged workload does); ``selection`` is
    "random", "recent", "alternate" (even b random, odd b recent) or "all"."""
    rng = np.random.default_rng(seed)
    if cache_lens is None:
        cache_lens = rng.integers(1024, 16384, size=B, endpoint=True)
    cache_lens = np.asarray(cache_lens, dtype=np.int32).reshape(B)
    if L_max is None:
        L_max = int(cache_lens.max())
    w = Workload(name=name, B=B, H=H, L_max=L_max, K=K, dtype_act=dtype_act, dtype_w=dtype_w,
                 rope=dict(rope), seed=seed)
    act = round_bf16 if dtype_act == "bf16" else (lambda a: a)
    wt = round_bf16 if dtype_w == "bf16" else (lambda a: a)
    w.cache_lens = cache_lens
    w.q_nope = act(_normal(rng, (B, H, D_NOPE)))
    w.q_pe = act(_normal(rng, (B, H, D_ROPE)))
    wstd = 512 ** -0.5
    w.w_uk = wt(_normal(rng, (H, D_NOPE, KV_RANK), wstd))
    w.w_uv = wt(_normal(rng, (H, D_V, KV_RANK), wstd))
    w.kv_cache = np.zeros((B, L_max, KV_RANK), dtype=np.float32)
    for b in range(B):
        w.kv_cache[b, :cache_lens[b]] = _normal(rng, (int(cache_lens[b]), KV_RANK))
    act(w.kv_cache)
    w.pe_cache = np.zeros((B, L_max, D_ROPE), dtype=np.float32)
    for b in range(B):
        w.pe_cache[b, :cache_lens[b]] = _normal(rng, (int(cache_lens[b]), D_ROPE))
    act(w.pe_cache)
    idx = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        L_b = int(cache_lens[b])
        k = min(K, L_b) if k_per_seq is None else int(k_per_seq[b])
        mode = selection
        if selection == "alternate":
            mode = "random" if b % 2 == 0 else "recent"
        if mode == "all":
            sel = rng.permutation(L_b).astype(np.int32)
        elif mode == "random":
            sel = random_selection(rng, L_b, k)
        elif mode == "recent":
            sel = recent_selection(L_b, k)
        else:
            raise ValueError(selection)
        idx[b, :sel.size] = sel
    w.topk_indices = idx
    return w


def new_rows(B: int, dtype_act: str, seed: int):
    """The new token's latent [B, 512] and raw rotary key [B, 64] for a fused
    append, drawn like the cached rows (N(0, 1), rounded to bf16 for bf16
    activations)."""
    rng = np.random.default_rng(seed)
    act = round_bf16 if dtype_act == "bf16" else (lambda a: a)
    return act(_normal(rng, (B, KV_RANK))), act(_normal(rng, (B, D_ROPE)))


def workload(name: str, batch_limit: int | None = None) -> Workload:
    """The named workload (tiny, page, batched, long, ragged, ragged_h16).  ``batch_limit``
    draws a smaller batch with the same recipe and seed (its values differ
    from the first sequences of the full batch)."""
    if name == "tiny":
        return build("tiny", 1, 16, [65], 65, "f32", "f32", ROPE_PLAIN, 101, selection="all")
    if name == "page":
        return build("page", 1, 128, [1001], 1001, "bf16", "bf16", ROPE_YARN, 102, selection="all")
    if name == "batched":
        B = 32 if batch_limit is None else batch_limit
        return build("batched", B, 128, [4096] * B, 2048, "bf16", "bf16", ROPE_YARN, 103)
    if name == "long":
        B = 64 if batch_limit is None else batch_limit
        return build("long", B, 128, [16384] * B, 2048, "bf16", "bf16", ROPE_YARN, 104)
    if name == "ragged":
        B = 128 if batch_limit is None else batch_limit
        return build("ragged", B, 128, None, 2048, "bf16", "f32", ROPE_YARN, 105,
                     L_max=16384, selection="alternate")
    if name == "ragged_h16":
        # the ragged batch at a 16-head shard (128 heads over 8 GPUs): the
        # same recipe with its own seed
        B = 128 if batch_limit is None else batch_limit
        return build("ragged_h16", B, 16, None, 2048, "bf16", "f32", ROPE_YARN, 106,
                     L_max=16384, selection="alternate")
    raise KeyError(name)


WORKLOADS = ("tiny", "page", "batched", "long", "ragged", "ragged_h16")
