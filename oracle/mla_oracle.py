"""CPU fp64 oracle for the absorbed-MLA sparse decode step (DeepSeek-V3.2-Exp).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this module: only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code, table or helper with the HIP
library; both sides only consume the same seeded inputs.

What it computes is the *non-absorbed* definition of one decode step: per head
it materialises the keys ``k = [W_UK c ; k_pe]`` and values ``v = W_UV c`` from
the latent cache, adds a -inf mask outside the top-k selection, and applies the
softmax and the weighted sum.  The absorbed form (attend over the latent cache
directly) reaches the same result by associativity; ``decode_attention_absorbed``
below writes that form out so a test can check the two agree.

Sources (the atlas pages on DeepSeek-V3.2-Exp's sparse latent attention):
  [rope]        page "Transformer blocks / RoPE coefficients" and page
                "Rotated query part": excerpt ``rope`` (precompute of the
                rotation coefficients with YaRN interpolation).
  [apply-rope]  page "Rotated query part": excerpt ``apply-rope``.
  [model-args]  page "Transformer blocks / RoPE coefficients": excerpt
                ``model-args`` (max_seq_len, original_seq_len, rope_theta,
                rope_factor, beta_fast, beta_slow, mscale defaults).
  [mla-init]    page "Query rotary features": excerpt ``mla-init`` (softmax
                scale with the mscale correction).
  [mla-queries] page "Query rotary features" / "Query content heads": excerpt
                ``mla-queries`` (q split into content and rotary parts; the
                rotary part is rotated, interleaved by default).
  [mla-decode]  pages "Rotated query part", "Query content heads",
                "Attention weights": excerpt ``mla-decode`` (the MQA decode
                branch: W_UK absorption, latent + rotary scores times the
                scale, the top-k index mask, softmax, weighted latent sum,
                W_UV up-projection).
  [attn-weights] page "Attention weights": node shapes (576 = latent 512 +
                rotary 64 per cached position; L = P + 1 keys in decode) and
                the note that the causal mask is folded into the selection.

Readings where the pages are silent:
  * YaRN correction range (the two helpers are omitted on the pages): the
    YaRN paper's correction dimension D(beta) = d ln(T0 / (2 pi beta)) /
    (2 ln base), lo = max(floor(D(beta_fast)), 0), hi = min(ceil(D(beta_slow)),
    d - 1), hi += 0.001 if equal, and a ramp linear in the pair index i.
  * Angles are exact (fp64); the page computes them in fp32.
  * The query of sequence b sits at position p_b = L_b - 1 (L = P + 1 keys).
  * The rope-key cache already holds keys rotated at their own positions.
  * A fused append writes the new token's latent unchanged and its rotary
    key rotated at p_b (interleaved) into row p_b (cache_append).
  * Selection is a set shared by all heads; -1 marks an unused slot;
    duplicates count once; an index outside [0, L_b) or an empty set is an
    error.
  * Arithmetic is fp64 throughout; inputs are upcast exactly.

Parity pins: every function here is pinned by a test in
``tests/test_oracle_pins.py`` against closed forms, invariants, brute force
or the pages' printed constants.  Nothing in this module is parity unpinned.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------------------
# Configuration (defaults printed on the pages)
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class RopeConfig:
    """Rotary / YaRN settings.  Defaults are the [model-args] values."""

    rope_dim: int = 64            # qk_rope_head_dim (64 rotary features per head)
    theta: float = 10000.0        # rope_theta
    max_seq_len: int = 4096 * 4   # max_seq_len
    original_seq_len: int = 4096  # original_seq_len
    factor: float = 40.0          # rope_factor
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0

    @property
    def yarn(self) -> bool:
        # [rope]: interpolation is applied when max_seq_len > original_seq_len.
        return self.max_seq_len > self.original_seq_len


# ---------------------------------------------------------------------------
# a1: rotation frequencies and the (cos, sin) table
# ---------------------------------------------------------------------------
def yarn_correction_dim(beta: float, cfg: RopeConfig) -> float:
    """Dimension index at which the rotary wavelength completes ``beta`` turns
    over the original context (YaRN paper, correction range)."""
    return (cfg.rope_dim * math.log(cfg.original_seq_len / (2.0 * math.pi * beta))
            / (2.0 * math.log(cfg.theta)))


def inv_freq(cfg: RopeConfig) -> np.ndarray:
    """theta'_i for i < rope_dim/2, fp64.  [rope]: base frequencies
    base^(-2i/d); with YaRN, blend theta/factor and theta with the ramp."""
    d = cfg.rope_dim
    i = np.arange(d // 2, dtype=np.float64)
    theta = cfg.theta ** (-(2.0 * i) / d)
    if not cfg.yarn:
        return theta
    lo = max(math.floor(yarn_correction_dim(cfg.beta_fast, cfg)), 0)
    hi = min(math.ceil(yarn_correction_dim(cfg.beta_slow, cfg)), d - 1)
    lo, hi = float(lo), float(hi)
    if hi == lo:
        hi += 0.001
    # gamma_i: 0 below lo (pairs that keep their frequency), 1 above hi
    # (pairs slowed by the factor), linear in between
    gamma = np.clip((i - lo) / (hi - lo), 0.0, 1.0)
    # [rope] (page "Transformer blocks / RoPE coefficients"): each frequency
    # is a gamma-weighted mix of theta_i / factor and theta_i
    return theta / cfg.factor * gamma + theta * (1.0 - gamma)


def rope_cos_sin(positions, cfg: RopeConfig) -> np.ndarray:
    """(cos, sin) of t * theta'_i for the given positions: [len, d/2, 2] fp64.
    [rope]: the table is the outer product of positions and frequencies,
    turned into unit complex numbers."""
    t = np.asarray(positions, dtype=np.float64).reshape(-1)
    ang = np.outer(t, inv_freq(cfg))
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1)


# ---------------------------------------------------------------------------
# a2: softmax scale
# ---------------------------------------------------------------------------
def softmax_scale(qk_head_dim: int, cfg: RopeConfig) -> float:
    """[mla-init]: qk_head_dim^-1/2, times mscale^2 with
    mscale = 0.1 * cfg.mscale * ln(factor) + 1 when YaRN is on."""
    s = qk_head_dim ** -0.5
    if cfg.yarn:
        m = 0.1 * cfg.mscale * math.log(cfg.factor) + 1.0
        s = s * m * m
    return s


# ---------------------------------------------------------------------------
# a3: interleaved rotary embedding
# ---------------------------------------------------------------------------
def rope_rotate(x: np.ndarray, position: int, cfg: RopeConfig) -> np.ndarray:
    """Rotate the last axis (rope_dim features) at one position.
    [apply-rope], interleaved layout: features (2i, 2i+1) form the complex
    number x[2i] + 1j*x[2i+1], multiplied by exp(1j * position * theta'_i)."""
    x = np.asarray(x, dtype=np.float64)
    cs = rope_cos_sin([position], cfg)[0]          # [d/2, 2]
    a = x[..., 0::2]
    b = x[..., 1::2]
    c, s = cs[:, 0], cs[:, 1]
    y = np.empty_like(x)
    y[..., 0::2] = a * c - b * s
    y[..., 1::2] = a * s + b * c
    return y


def rope_rotate_halves(x: np.ndarray, position: int, cfg: RopeConfig) -> np.ndarray:
    """Rotate the last axis at one position in the non-interleaved layout
    (NEXT row f2; the indexer's layout).  [apply-rope] with interleaved=False:
    the features are viewed as [2, d/2] and transposed, so pair i is
    (x[i], x[i + d/2]); after the complex multiplication the real parts come
    first, then the imaginary parts."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    pairs = np.swapaxes(x.reshape(*x.shape[:-1], 2, d // 2), -1, -2)   # [..., d/2, 2]
    z = pairs[..., 0] + 1j * pairs[..., 1]
    cs = rope_cos_sin([position], cfg)[0]
    z = z * (cs[:, 0] + 1j * cs[:, 1])
    return np.concatenate([z.real, z.imag], axis=-1)


def cache_append(kv_cache, pe_cache, kv_new, pe_new, cache_lens, cfg: RopeConfig):
    """The new token's row written into the caches before it is attended to
    (NEXT row f3).  [mla-init]: the joint down-projection emits the latent
    (RMS-normalised before caching; that step stays outside, kv_new is the
    normalised latent) and one rotary key shared by all heads.  The write
    itself is not on the pages; the reading taken: for each sequence b the
    row p_b = L_b - 1 (the new token's own position, [attn-weights]) gets
    C[b, p_b] = kv_new[b] and R[b, p_b] = the rotary key rotated at p_b with
    the same table and interleaved layout as the query ([apply-rope]), so a
    query-key dot product depends on the positions only through their
    difference.  Returns new fp64 arrays; the inputs are not modified."""
    C = _f64(kv_cache).copy()
    R = _f64(pe_cache).copy()
    kv_new = _f64(kv_new)
    pe_new = _f64(pe_new)
    for b, L in enumerate(np.asarray(cache_lens).reshape(-1)):
        L = int(L)
        if L < 1 or L > C.shape[1]:
            raise ValueError(f"sequence {b}: cache length {L} outside [1, {C.shape[1]}]")
        C[b, L - 1] = kv_new[b]
        R[b, L - 1] = rope_rotate(pe_new[b], L - 1, cfg)
    return C, R


# ---------------------------------------------------------------------------
# a5: selection
# ---------------------------------------------------------------------------
class SelectionError(ValueError):
    pass


def selection_set(indices_row, L_b: int) -> np.ndarray:
    """The selected positions of one sequence, ascending, duplicates removed.
    [mla-decode]: the mask is -inf everywhere and 0 scattered at the indices,
    so an index listed twice selects its position once.  -1 marks an unused
    slot.  Out-of-range indices and an empty set are errors."""
    idx = np.asarray(indices_row, dtype=np.int64).reshape(-1)
    idx = idx[idx != -1]
    if idx.size and (idx.min() < 0 or idx.max() >= L_b):
        raise SelectionError(f"index outside [0, {L_b})")
    sel = np.unique(idx)
    if sel.size == 0:
        raise SelectionError("empty selection")
    return sel


def selection_mask(indices_row, L_b: int) -> np.ndarray:
    """The literal additive mask over [0, L_b): -inf, with 0 at the selected
    positions ([mla-decode] index_mask)."""
    mask = np.full(L_b, -np.inf)
    mask[selection_set(indices_row, L_b)] = 0.0
    return mask


def topk_select(scores_row, L_b: int, k: int) -> np.ndarray:
    """The indexer's selection step (NEXT row f1): positions of the
    min(k, L_b) largest of scores_row[0:L_b], ascending.  [mla-decode]:
    ``topk_indices = self.indexer(...)`` supplies the positions the index
    mask opens; the indexer's scoring is not on the pages, only that its
    output is a set of positions in [0, L_b).  Reading (the pages leave the
    order of equal scores open): scores compare as real numbers (-0 == +0),
    NaN ranks below every other value, and among equal scores the lower
    position ranks higher.  Written as a plain sort over (rank key, position)."""
    L_b = max(0, int(L_b))
    s = np.asarray(scores_row, dtype=np.float64).reshape(-1)[:L_b]

    def rank_key(p):
        v = s[p]
        if v != v:                                   # NaN: lowest class
            return (0, 0.0, -p)
        return (1, float(v) + 0.0, -p)               # + 0.0 folds -0 into +0

    order = sorted(range(L_b), key=rank_key, reverse=True)
    return np.array(sorted(order[:min(k, L_b)]), dtype=np.int64)


# ---------------------------------------------------------------------------
# The decode step, non-absorbed definition (a3..a11 as one definition)
# ---------------------------------------------------------------------------
def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def decode_attention(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices,
                     cache_lens, cfg: RopeConfig, sm_scale: float | None = None,
                     form: str = "masked", batch=None, heads=None):
    """One decode step for each sequence, by the non-absorbed definition.

    Shapes (inputs upcast exactly to fp64):
      q_nope [B, H, 128], q_pe [B, H, 64] (raw, rotated here at p_b = L_b - 1),
      w_uk, w_uv [H, 128, 512] (latent index c contiguous),
      kv_cache [B, >=L_b, 512], pe_cache [B, >=L_b, 64] (keys already rotated),
      topk_indices [B, K] int (-1 = unused slot), cache_lens [B] (L_b).

    For each head h and position t < L_b:
      k_{h,t} = [W_UK[h] @ C[t] ; R[t]],  v_{h,t} = W_UV[h] @ C[t],
      q_h = [q_nope[h] ; rope(q_pe[h], p_b)],
      s_{h,t} = sm_scale * q_h . k_{h,t} + mask_t,
      out[h] = sum_t softmax(s_h)_t v_{h,t},  lse[h] = log sum_t exp(s_{h,t}).

    ``form="masked"`` builds the scores over every t < L_b and adds the
    literal -inf mask; ``form="restricted"`` evaluates only the selected t
    (identical, since exp(-inf) = 0) and is what large inputs use.
    ``batch``/``heads`` restrict the work to a sample of outputs.

    Returns (out [nb, nh, 128], lse [nb, nh]) in fp64.
    """
    if sm_scale is None:
        sm_scale = softmax_scale(q_nope.shape[-1] + q_pe.shape[-1], cfg)
    B = q_nope.shape[0]
    H = q_nope.shape[1]
    batch = list(range(B)) if batch is None else list(batch)
    heads = list(range(H)) if heads is None else list(heads)
    w_uk_s = _f64(np.asarray(w_uk)[heads])         # [h, 128, 512]
    w_uv_s = _f64(np.asarray(w_uv)[heads])
    nh = len(heads)
    out = np.zeros((len(batch), nh, w_uv_s.shape[1]))
    lse = np.zeros((len(batch), nh))
    for bi, b in enumerate(batch):
        L_b = int(cache_lens[b])
        if L_b < 1:
            raise SelectionError("empty cache")
        p_b = L_b - 1                                   # query position
        if form == "masked":
            rows = np.arange(L_b)
            mask = selection_mask(topk_indices[b], L_b)
        elif form == "restricted":
            rows = selection_set(topk_indices[b], L_b)
            mask = np.zeros(rows.size)
        else:
            raise ValueError(form)
        C = _f64(kv_cache[b][rows])                     # [n, 512]
        R = _f64(pe_cache[b][rows])                     # [n, 64]
        qn = _f64(np.asarray(q_nope[b])[heads])         # [h, 128]
        qr = rope_rotate(np.asarray(q_pe[b])[heads], p_b, cfg)   # [h, 64]
        n = rows.size
        # Materialised keys and values, one GEMM each over all sampled heads.
        k_nope = (w_uk_s.reshape(nh * w_uk_s.shape[1], -1) @ C.T).reshape(nh, w_uk_s.shape[1], n)
        v = (w_uv_s.reshape(nh * w_uv_s.shape[1], -1) @ C.T).reshape(nh, w_uv_s.shape[1], n)
        # s[h, t] = q_h . k_{h,t}: content part per head, rotary part shared (MQA).
        s = np.einsum("hd,hdt->ht", qn, k_nope) + qr @ R.T
        s = s * sm_scale + mask[None, :]
        mu = s.max(axis=1, keepdims=True)
        e = np.exp(s - mu)
        Z = e.sum(axis=1, keepdims=True)
        P = e / Z
        out[bi] = np.einsum("ht,hdt->hd", P, v)
        lse[bi] = (mu + np.log(Z))[:, 0]
    return out, lse


def decode_attention_absorbed(q_nope, q_pe, w_uk, w_uv, kv_cache, pe_cache, topk_indices,
                              cache_lens, cfg: RopeConfig, sm_scale: float | None = None):
    """The absorbed form of the same step, fp64, for the equivalence pin.
    [mla-decode]: q_abs = q_nope W_UK[h] (into the 512-d latent), scores over
    the latent cache plus the rotary cache, softmax over the selection, the
    weighted latent sum, then W_UV[h]."""
    if sm_scale is None:
        sm_scale = softmax_scale(q_nope.shape[-1] + q_pe.shape[-1], cfg)
    B, H = q_nope.shape[:2]
    out = np.zeros((B, H, np.asarray(w_uv).shape[1]))
    lse = np.zeros((B, H))
    wuk = _f64(w_uk)
    wuv = _f64(w_uv)
    for b in range(B):
        L_b = int(cache_lens[b])
        rows = selection_set(topk_indices[b], L_b)
        C = _f64(kv_cache[b][rows])
        R = _f64(pe_cache[b][rows])
        q_abs = np.einsum("hd,hdc->hc", _f64(q_nope[b]), wuk)          # [H, 512]
        qr = rope_rotate(q_pe[b], L_b - 1, cfg)                        # [H, 64]
        s = (q_abs @ C.T + qr @ R.T) * sm_scale
        mu = s.max(axis=1, keepdims=True)
        e = np.exp(s - mu)
        Z = e.sum(axis=1, keepdims=True)
        o_lat = (e / Z) @ C                                             # [H, 512]
        out[b] = np.einsum("hc,hdc->hd", o_lat, wuv)
        lse[b] = (mu + np.log(Z))[:, 0]
    return out, lse


def max_rel_l2(got, ref) -> float:
    """Max over output rows (last axis) of ||got - ref||_2 / ||ref||_2."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(num / den))
