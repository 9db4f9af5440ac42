"""Decode inputs whose scores spread far beyond the N(0, 1) workloads.

With N(0, 1) queries and caches the scaled scores of one head stay within a
few units of each other.  A legal input can spread them much further.  Here
a chosen set of selected rows of each sequence gets the latent
C[t] = alpha * u, where u is the least-norm vector with q_abs_h . u = -1 for
every head h (q_abs_h = q_nope[b, h] . W_UK[h]), so that the latent part of
those rows' scores is -alpha * scale for all heads at once: about c_log2
units (log2 domain) below the rows left untouched, whose scores stay
ordinary.

  mode "late":  every selected row except the 3 highest positions is pushed
                down: the maximum of every head comes from the last rows of
                the last split, far above that split's first 32 rows.
  mode "first": every selected row except the 32 lowest positions is pushed
                down: the first rows hold the maximum and every later row
                lies far below it.

This module builds inputs and evaluates scores for the checks; it draws its
values from workloads.py and evaluates the scores with the oracle's own
rotary and scale functions.
"""
import math

import numpy as np

import oracle
import workloads as W

LN2 = math.log(2.0)


def scores_log2(w, b, rows):
    """x[h, t] = scale * (q_abs_h . C[t] + rope(q_pe_h, p_b) . R[t]) / ln 2
    for the given rows of sequence b, in fp64 (the softmax in base 2)."""
    cfg = oracle.RopeConfig(**w.rope)
    scale = oracle.softmax_scale(192, cfg)
    qa = np.einsum("hd,hdc->hc", w.q_nope[b].astype(np.float64), w.w_uk.astype(np.float64))
    qr = oracle.rope_rotate(w.q_pe[b], int(w.cache_lens[b]) - 1, cfg)
    C = w.kv_cache[b][rows].astype(np.float64)
    R = w.pe_cache[b][rows].astype(np.float64)
    return (qa @ C.T + qr @ R.T) * scale / LN2


def split_ranges(count, splits):
    """The rows [start, end) of each split of a sequence's ascending list of
    `count` selected positions: ceil(count / splits) rounded up to a multiple
    of 8 per split (the library's partition)."""
    rps = -(-count // splits)
    rps = (rps + 7) & ~7
    out = []
    for s in range(splits):
        start = min(s * rps, count)
        out.append((start, min(start + rps, count)))
    return out


def excess_log2(w, b, splits):
    """Per split: the largest, over heads, of (maximum score of the split)
    minus (the maximum over the split's first 32 rows, floored), in log2
    units.  Splits without rows give -inf."""
    row = w.topk_indices[b]
    sel = np.unique(row[row >= 0])
    x = scores_log2(w, b, sel)
    out = []
    for start, end in split_ranges(sel.size, splits):
        if end <= start:
            out.append(-math.inf)
            continue
        first = np.floor(x[:, start:min(start + 32, end)].max(axis=1))
        out.append(float((x[:, start:end].max(axis=1) - first).max()))
    return out


def build(name, mode, c_log2, dtype_act="bf16", dtype_w="bf16", seed=41, H=128, lens=(1500, 1200), K=1000):
    lens = list(lens)
    w = W.build(name, len(lens), H, lens, K, dtype_act, dtype_w, W.ROPE_YARN, seed=seed)
    cfg = oracle.RopeConfig(**w.rope)
    scale = oracle.softmax_scale(192, cfg)
    for b in range(w.B):
        row = w.topk_indices[b]
        sel = np.unique(row[row >= 0])
        qa = np.einsum("hd,hdc->hc", w.q_nope[b].astype(np.float64), w.w_uk.astype(np.float64))
        # least-norm u with qa @ u = -1 for every head
        u = -qa.T @ np.linalg.solve(qa @ qa.T, np.ones(w.H))
        alpha = c_log2 * LN2 / scale
        target = sel[:-3] if mode == "late" else sel[32:]
        w.kv_cache[b, target] = (alpha * u).astype(np.float32)
    if dtype_act == "bf16":
        W.round_bf16(w.kv_cache)
    return w
