"""Pins of the CPU oracle against things other than itself: the pages' printed
constants, closed forms, invariants and brute force on tiny inputs.

Each test names the plausible oracle mistake it would catch.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import RopeConfig

YARN = RopeConfig()                              # the pages' defaults
PLAIN = RopeConfig(max_seq_len=4096)             # no interpolation


# ---------------------------------------------------------------------------
# Defaults and shapes printed on the pages
# ---------------------------------------------------------------------------
def test_defaults_match_pages(page_constants):
    c = page_constants
    assert YARN.max_seq_len == c["max_seq_len"]
    assert YARN.original_seq_len == c["original_seq_len"]
    assert YARN.theta == c["rope_theta"]
    assert YARN.factor == c["rope_factor"]
    assert YARN.beta_fast == c["beta_fast"] and YARN.beta_slow == c["beta_slow"]
    assert YARN.mscale == c["mscale"]
    assert YARN.rope_dim == c["rope_dim"] == 2 * c["rope_pairs"]
    assert c["nope_dim"] + c["rope_dim"] == 192
    assert c["row_width"] - c["rope_dim"] == 512          # latent rank
    assert c["decode_keys"] == c["decode_cached"] + 1
    assert oracle.inv_freq(YARN).shape == (int(c["rope_pairs"]),)


# ---------------------------------------------------------------------------
# a2: softmax scale
# ---------------------------------------------------------------------------
def test_scale_plain_is_inverse_sqrt(closed_forms):
    # No interpolation: qk_head_dim^-1/2 exactly (catches a missing sqrt or
    # a correction applied without YaRN).
    assert oracle.softmax_scale(64, PLAIN) == 0.125
    assert oracle.softmax_scale(192, PLAIN) == pytest.approx(closed_forms["inv_sqrt_192"], rel=1e-15)


def test_scale_mscale_special_cases():
    # factor = e^10 makes 0.1*ln(factor) + 1 = 2: the correction is 2^2 = 4,
    # so qk_head_dim = 16 gives exactly 1.  A log10, a missing square or a
    # dropped 0.1 all move this value.
    cfg = RopeConfig(factor=math.exp(10.0))
    assert oracle.softmax_scale(16, cfg) == pytest.approx(1.0, rel=1e-14)
    # mscale = 0 switches the correction off.
    assert oracle.softmax_scale(64, RopeConfig(mscale=0.0)) == pytest.approx(0.125, rel=1e-15)
    # mscale = 2 with factor e^5: 0.1*2*5 + 1 = 2 again.
    assert oracle.softmax_scale(16, RopeConfig(mscale=2.0, factor=math.exp(5.0))) == pytest.approx(1.0, rel=1e-14)


# ---------------------------------------------------------------------------
# a1: frequencies
# ---------------------------------------------------------------------------
def test_plain_freqs_closed_form(closed_forms):
    f = oracle.inv_freq(PLAIN)
    assert f[0] == 1.0
    assert f[16] == pytest.approx(0.01, rel=1e-14)          # 10000^(-1/2)
    assert f[8] == pytest.approx(0.1, rel=1e-14)            # 10000^(-1/4)
    assert f[24] == pytest.approx(0.001, rel=1e-14)         # 10000^(-3/4)
    assert f[1] == pytest.approx(closed_forms["theta_1"], rel=1e-14)
    ratio = f[1:] / f[:-1]                                    # geometric progression
    assert np.allclose(ratio, 10000.0 ** (-1.0 / 32), rtol=1e-13)


def test_yarn_off_at_or_below_original_length():
    # The interpolation branch depends on max_seq_len > original_seq_len only.
    for T in (64, 1024, 4096):
        assert np.array_equal(oracle.inv_freq(RopeConfig(max_seq_len=T)), oracle.inv_freq(PLAIN))


def test_yarn_freqs_pinned_values(closed_forms):
    f = oracle.inv_freq(YARN)
    plain = oracle.inv_freq(PLAIN)
    # Below the correction range: untouched; above it: divided by the factor.
    assert np.array_equal(f[:11], plain[:11])
    assert np.allclose(f[23:], plain[23:] / 40.0, rtol=1e-14)
    # Inside: linear ramp in the pair index between dims 10 and 23.
    assert f[16] == pytest.approx(closed_forms["yarn_theta_16"], rel=1e-13)
    g = 1.0 / 13.0
    assert f[11] == pytest.approx(plain[11] * (1 - g) + plain[11] / 40 * g, rel=1e-14)
    assert f[10] == pytest.approx(closed_forms["theta_10"], rel=1e-14)
    assert f[22] != pytest.approx(plain[22] / 40, rel=1e-6)   # still inside the ramp
    assert np.all(np.diff(f) < 0)                            # monotone decreasing
    assert f[0] == 1.0


def test_yarn_factor_one_is_identity():
    assert np.allclose(oracle.inv_freq(RopeConfig(factor=1.0)), oracle.inv_freq(PLAIN), rtol=1e-15)


# ---------------------------------------------------------------------------
# a3: interleaved rotation
# ---------------------------------------------------------------------------
def test_rope_worked_values(closed_forms):
    cs = oracle.rope_cos_sin([1, 1000, 16383], YARN)
    c = closed_forms
    assert cs[0, 0] == pytest.approx([c["cos_1"], c["sin_1"]], abs=1e-15)
    assert cs[1, 0] == pytest.approx([c["cos_1000"], c["sin_1000"]], abs=1e-13)
    assert cs[2, 0] == pytest.approx([c["cos_16383"], c["sin_16383"]], abs=1e-12)


def test_rope_pairing_and_sign(closed_forms):
    # e0 at p=1 -> (cos 1, sin 1) in features (0, 1); e1 -> (-sin 1, cos 1).
    # e2 pairs with feature 3 (interleaved, not half-split) at theta'_1.
    e = np.eye(64)
    c = closed_forms
    y0 = oracle.rope_rotate(e[0], 1, YARN)
    assert y0[:2] == pytest.approx([c["cos_1"], c["sin_1"]], abs=1e-15)
    assert np.all(y0[2:] == 0)
    y1 = oracle.rope_rotate(e[1], 1, YARN)
    assert y1[:2] == pytest.approx([-c["sin_1"], c["cos_1"]], abs=1e-15)
    y2 = oracle.rope_rotate(e[2], 1, YARN)
    t1 = c["theta_1"]
    assert y2[2:4] == pytest.approx([math.cos(t1), math.sin(t1)], abs=1e-15)
    assert np.all(y2[:2] == 0) and np.all(y2[4:] == 0)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(0)
    q = rng.standard_normal(64)
    k = rng.standard_normal(64)
    assert np.array_equal(oracle.rope_rotate(q, 0, YARN), q)
    for p in (1, 77, 4095, 16383):
        y = oracle.rope_rotate(q, p, YARN)
        assert np.allclose(np.hypot(y[0::2], y[1::2]), np.hypot(q[0::2], q[1::2]), rtol=1e-13)
    # <rot_m q, rot_n k> depends on m - n only.
    for m, n in ((5, 2), (1003, 1000), (16383, 16380)):
        lhs = oracle.rope_rotate(q, m, YARN) @ oracle.rope_rotate(k, n, YARN)
        rhs = oracle.rope_rotate(q, m - n, YARN) @ k
        assert lhs == pytest.approx(rhs, rel=1e-10, abs=1e-10)


# ---------------------------------------------------------------------------
# a5: selection
# ---------------------------------------------------------------------------
def test_selection_set_semantics():
    assert list(oracle.selection_set([3, -1, 1, 3, 0, -1], 4)) == [0, 1, 3]
    m = oracle.selection_mask([2, 2, -1], 4)
    assert list(m) == [-np.inf, -np.inf, 0.0, -np.inf]
    with pytest.raises(oracle.SelectionError):
        oracle.selection_set([4], 4)
    with pytest.raises(oracle.SelectionError):
        oracle.selection_set([-2], 4)
    with pytest.raises(oracle.SelectionError):
        oracle.selection_set([-1, -1], 4)


# ---------------------------------------------------------------------------
# The decode step
# ---------------------------------------------------------------------------
def _tiny(rng, B=1, H=2, L=6, dn=4, dr=4, r=6, dv=3, K=None):
    K = L if K is None else K
    return dict(
        q_nope=rng.standard_normal((B, H, dn)), q_pe=rng.standard_normal((B, H, dr)),
        w_uk=rng.standard_normal((H, dn, r)), w_uv=rng.standard_normal((H, dv, r)),
        kv_cache=rng.standard_normal((B, L, r)), pe_cache=rng.standard_normal((B, L, dr)),
        topk_indices=np.tile(np.arange(K), (B, 1)), cache_lens=np.full(B, L))


def _brute_dense_causal(inp, cfg, scale):
    """Dense causal softmax attention over explicitly built per-head keys and
    values, with plain Python loops (query at the last position)."""
    B, H, dn = inp["q_nope"].shape
    dr = inp["q_pe"].shape[2]
    r = inp["kv_cache"].shape[2]
    dv = inp["w_uv"].shape[1]
    out = np.zeros((B, H, dv))
    lse = np.zeros((B, H))
    freqs = oracle.inv_freq(cfg)
    for b in range(B):
        L = int(inp["cache_lens"][b])
        p = L - 1
        for h in range(H):
            q = list(inp["q_nope"][b, h])
            qp = inp["q_pe"][b, h]
            for i in range(dr // 2):
                a, c = qp[2 * i], qp[2 * i + 1]
                ang = p * freqs[i]
                q += [None, None]
                q[dn + 2 * i] = a * math.cos(ang) - c * math.sin(ang)
                q[dn + 2 * i + 1] = a * math.sin(ang) + c * math.cos(ang)
            scores, vals = [], []
            for t in range(L):                         # causal: every t <= p
                key = [sum(inp["w_uk"][h, d, cc] * inp["kv_cache"][b, t, cc] for cc in range(r))
                       for d in range(dn)] + list(inp["pe_cache"][b, t])
                scores.append(scale * sum(x * y for x, y in zip(q, key)))
                vals.append([sum(inp["w_uv"][h, d, cc] * inp["kv_cache"][b, t, cc] for cc in range(r))
                             for d in range(dv)])
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            Z = sum(w)
            for d in range(dv):
                out[b, h, d] = sum(wi * v[d] for wi, v in zip(w, vals)) / Z
            lse[b, h] = mx + math.log(Z)
    return out, lse


@pytest.mark.parametrize("max_seq_len", [4096, 16384])
def test_full_selection_equals_dense_causal_bruteforce(max_seq_len):
    rng = np.random.default_rng(1)
    cfg = RopeConfig(rope_dim=4, max_seq_len=max_seq_len)
    for L in (1, 2, 5, 8):
        inp = _tiny(rng, B=2, H=2, L=L)
        scale = 0.37
        out, lse = oracle.decode_attention(**inp, cfg=cfg, sm_scale=scale)
        ref, ref_lse = _brute_dense_causal(inp, cfg, scale)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_single_selected_row_is_w_uv_times_latent():
    # P = 1 on the one selected row: out[h] = W_UV[h] @ C[t], lse = its score.
    rng = np.random.default_rng(2)
    cfg = RopeConfig(rope_dim=4)
    inp = _tiny(rng, B=1, H=3, L=7)
    t = 4
    inp["topk_indices"] = np.array([[t, -1, t, -1]])
    out, lse = oracle.decode_attention(**inp, cfg=cfg, sm_scale=0.5)
    for h in range(3):
        want = [sum(inp["w_uv"][h, d, c] * inp["kv_cache"][0, t, c] for c in range(6)) for d in range(3)]
        assert np.allclose(out[0, h], want, rtol=1e-13)
    # a second head must not reuse the first head's weights
    assert not np.allclose(out[0, 0], out[0, 1])


def test_zero_query_gives_uniform_average():
    rng = np.random.default_rng(3)
    cfg = RopeConfig(rope_dim=4)
    inp = _tiny(rng, B=1, H=2, L=9)
    inp["q_nope"][:] = 0
    inp["q_pe"][:] = 0
    sel = [8, 1, 5, 2]
    inp["topk_indices"] = np.array([sel])
    out, lse = oracle.decode_attention(**inp, cfg=cfg, sm_scale=1.7)
    mean_c = inp["kv_cache"][0, sel].mean(axis=0)
    for h in range(2):
        assert np.allclose(out[0, h], inp["w_uv"][h] @ mean_c, rtol=1e-13)
    assert np.allclose(lse, math.log(len(sel)), rtol=1e-14)


def test_rotary_term_closed_form():
    # Only the rotary part scores: q_nope = 0, R[t*] = e0, other rows 0,
    # q_pe = e1.  The rotated query's feature 0 is -sin(p * theta'_0) with
    # p = L - 1, so s_{t*} = -scale * sin(L - 1) and every other score is 0.
    cfg = RopeConfig(rope_dim=4)
    rng = np.random.default_rng(4)
    L = 12
    inp = _tiny(rng, B=1, H=1, L=L)
    inp["q_nope"][:] = 0
    inp["q_pe"][:] = 0
    inp["q_pe"][0, 0, 1] = 1.0
    inp["pe_cache"][:] = 0
    ts, t2 = 3, 7
    inp["pe_cache"][0, ts, 0] = 1.0
    inp["topk_indices"] = np.array([[t2, ts]])
    scale = 0.9
    out, lse = oracle.decode_attention(**inp, cfg=cfg, sm_scale=scale)
    s = -scale * math.sin(L - 1)
    p = math.exp(s) / (math.exp(s) + 1.0)
    v = lambda t: inp["w_uv"][0] @ inp["kv_cache"][0, t]
    assert np.allclose(out[0, 0], p * v(ts) + (1 - p) * v(t2), rtol=1e-13)
    assert lse[0, 0] == pytest.approx(math.log(math.exp(s) + 1.0), rel=1e-13)


def test_masked_form_equals_restricted_form_and_absorbed_form():
    rng = np.random.default_rng(5)
    B, H, L = 3, 4, 40
    inp = dict(
        q_nope=rng.standard_normal((B, H, 128)), q_pe=rng.standard_normal((B, H, 64)),
        w_uk=rng.standard_normal((H, 128, 512)) / 22.6, w_uv=rng.standard_normal((H, 128, 512)) / 22.6,
        kv_cache=rng.standard_normal((B, L, 512)), pe_cache=rng.standard_normal((B, L, 64)),
        topk_indices=np.stack([rng.permutation(L)[:17] for _ in range(B)]),
        cache_lens=np.array([L, L - 3, 25]))
    for b in range(B):
        inp["topk_indices"][b] = np.where(inp["topk_indices"][b] < inp["cache_lens"][b],
                                          inp["topk_indices"][b], -1)
    a, la = oracle.decode_attention(**inp, cfg=YARN, form="masked")
    b, lb = oracle.decode_attention(**inp, cfg=YARN, form="restricted")
    c, lc = oracle.decode_attention_absorbed(**inp, cfg=YARN)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13) and np.allclose(la, lb, rtol=1e-13)
    assert np.allclose(a, c, rtol=1e-10, atol=1e-12) and np.allclose(la, lc, rtol=1e-12)
    # sampled heads/sequences give the same rows
    d, ld = oracle.decode_attention(**inp, cfg=YARN, form="restricted", batch=[2, 0], heads=[3, 1])
    assert np.allclose(d, b[[2, 0]][:, [3, 1]], rtol=1e-13) and np.allclose(ld, lb[[2, 0]][:, [3, 1]])


def test_order_and_duplicate_invariance():
    rng = np.random.default_rng(6)
    cfg = RopeConfig(rope_dim=4)
    inp = _tiny(rng, B=1, H=2, L=10)
    inp["topk_indices"] = np.array([[9, 0, 4, 7]])
    base, lb = oracle.decode_attention(**inp, cfg=cfg, sm_scale=0.8)
    for perm in itertools.permutations(range(4)):
        inp["topk_indices"] = np.array([[9, 0, 4, 7]])[:, list(perm)]
        out, l = oracle.decode_attention(**inp, cfg=cfg, sm_scale=0.8)
        assert np.allclose(out, base, rtol=1e-13) and np.allclose(l, lb, rtol=1e-13)
    inp["topk_indices"] = np.array([[9, 9, 0, -1, 4, 7, 0, 7]])
    out, l = oracle.decode_attention(**inp, cfg=cfg, sm_scale=0.8)
    assert np.allclose(out, base, rtol=1e-13) and np.allclose(l, lb, rtol=1e-13)


def test_position_shift_invariance():
    # Rotating every cached key at t + D and the query at p + D leaves every
    # score unchanged: the output must not move.
    rng = np.random.default_rng(7)
    L = 16
    inp = _tiny(rng, B=1, H=2, L=L, dr=64, dn=8, r=8, dv=5)
    raw_k = rng.standard_normal((L, 64))
    outs = []
    for D in (0, 1000, 9000):
        cfg = YARN
        pe = np.stack([oracle.rope_rotate(raw_k[t], t + D, cfg) for t in range(L)])
        x = dict(inp)
        x["pe_cache"] = np.concatenate([np.zeros((1, D, 64)), pe[None]], axis=1) if D else pe[None]
        x["kv_cache"] = np.concatenate([np.zeros((1, D, 8)), inp["kv_cache"]], axis=1) if D else inp["kv_cache"]
        x["topk_indices"] = np.array([[D + t for t in (0, 3, 8, 15, 11)]])
        x["cache_lens"] = np.array([L + D])
        out, _ = oracle.decode_attention(**x, cfg=cfg, sm_scale=0.3)
        outs.append(out)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=1e-9, atol=1e-11)


def test_max_rel_l2():
    ref = np.array([[3.0, 4.0], [1.0, 0.0]])
    got = np.array([[3.0, 4.5], [1.0, 0.001]])
    assert oracle.max_rel_l2(got, ref) == pytest.approx(0.1)


# ---------------------------------------------------------------------------
# NEXT row f1: top-k selection.  The oracle sorts; the pins below use a
# different, order-free definition (a position is selected iff fewer than
# k_b positions outrank it) and hand-worked cases.
# ---------------------------------------------------------------------------
def _outranks(s, q, p):
    """Does position q rank above position p?  NaN lowest, -0 == +0, ties to the lower position."""
    a, b = s[q], s[p]
    a_nan, b_nan = a != a, b != b
    if a_nan or b_nan:
        if a_nan and b_nan:
            return q < p
        return b_nan
    if a != b:
        return a > b
    return q < p


def _topk_by_rank_count(s, L_b, k):
    L_b = max(0, L_b)
    kb = min(k, L_b)
    return [p for p in range(L_b) if sum(_outranks(s, q, p) for q in range(L_b) if q != p) < kb]


def test_topk_hand_cases():
    s = [0.5, 3.0, -1.0, 3.0, 2.0, float("nan"), 0.0]
    assert list(oracle.topk_select(s, 7, 2)) == [1, 3]
    assert list(oracle.topk_select(s, 7, 3)) == [1, 3, 4]
    # the tie at the threshold goes to the lower position
    assert list(oracle.topk_select([1.0, 2.0, 2.0, 2.0], 4, 2)) == [1, 2]
    # -0 equals +0: the tie keeps the lower position
    assert list(oracle.topk_select([-0.0, 0.0, -5.0], 3, 1)) == [0]
    # NaN ranks below -inf
    assert list(oracle.topk_select([float("nan"), -np.inf], 2, 1)) == [1]
    # only positions below L_b count; k >= L_b selects them all
    assert list(oracle.topk_select([1.0, 9.0, 9.0, 9.0], 2, 1)) == [1]
    assert list(oracle.topk_select([1.0, 2.0, 3.0], 3, 5)) == [0, 1, 2]
    assert list(oracle.topk_select([1.0], 0, 3)) == []


@pytest.mark.parametrize("seed", range(6))
def test_topk_equals_rank_count_definition(seed):
    rng = np.random.default_rng(900 + seed)
    for _ in range(20):
        L = int(rng.integers(1, 24))
        k = int(rng.integers(1, 26))
        L_b = int(rng.integers(0, L + 1))
        s = rng.integers(-3, 4, size=L).astype(np.float64)      # many ties
        s[rng.random(L) < 0.1] = np.nan
        s[rng.random(L) < 0.1] = -0.0
        s[rng.random(L) < 0.05] = -np.inf
        assert list(oracle.topk_select(s, L_b, k)) == _topk_by_rank_count(s, L_b, k)


def test_topk_invariants_on_continuous_scores():
    rng = np.random.default_rng(77)
    s = rng.standard_normal(5000)
    sel = oracle.topk_select(s, 4000, 300)
    assert sel.size == 300 and np.all(np.diff(sel) > 0) and sel.max() < 4000
    rest = np.setdiff1d(np.arange(4000), sel)
    assert s[sel].min() > s[rest].max()


# ---------------------------------------------------------------------------
# NEXT row f2: the non-interleaved (half-split) rotary layout
# ---------------------------------------------------------------------------
def test_rope_halves_is_interleaved_under_the_pair_permutation():
    # pair i is (x[i], x[i+32]) in the half-split layout and (x[2i], x[2i+1])
    # interleaved: permuting the input into interleaved order, rotating, and
    # permuting back gives the same vector
    rng = np.random.default_rng(55)
    x = rng.standard_normal(64)
    perm = np.empty(64, dtype=int)
    perm[0::2] = np.arange(32)
    perm[1::2] = np.arange(32) + 32
    for p in (0, 1, 17, 4095, 16383):
        y_int = oracle.rope_rotate(x[perm], p, YARN)
        y = np.empty(64)
        y[:32] = y_int[0::2]
        y[32:] = y_int[1::2]
        assert np.allclose(oracle.rope_rotate_halves(x, p, YARN), y, rtol=0, atol=1e-13)


def test_rope_halves_pair0_worked_value(closed_forms):
    # pair 0 = (x[0], x[32]) rotated by t * theta'_0 = t (theta'_0 = 1)
    x = np.zeros(64)
    x[0], x[32] = 1.0, 0.0
    y = oracle.rope_rotate_halves(x, 1, YARN)
    assert abs(y[0] - math.cos(1.0)) < 1e-15 and abs(y[32] - math.sin(1.0)) < 1e-15
    x[0], x[32] = 0.0, 1.0
    y = oracle.rope_rotate_halves(x, 1, YARN)
    assert abs(y[0] + math.sin(1.0)) < 1e-15 and abs(y[32] - math.cos(1.0)) < 1e-15


def test_rope_halves_identity_norm_relative_position():
    rng = np.random.default_rng(56)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.allclose(oracle.rope_rotate_halves(q, 0, YARN), q, atol=1e-15)
    assert abs(np.linalg.norm(oracle.rope_rotate_halves(q, 999, YARN)) - np.linalg.norm(q)) < 1e-12
    d1 = oracle.rope_rotate_halves(q, 700, YARN) @ oracle.rope_rotate_halves(k, 500, YARN)
    d2 = oracle.rope_rotate_halves(q, 1200, YARN) @ oracle.rope_rotate_halves(k, 1000, YARN)
    assert abs(d1 - d2) < 1e-10


# ---------------------------------------------------------------------------
# NEXT row f3: the fused cache append
# ---------------------------------------------------------------------------
def test_cache_append_writes_only_row_p_b():
    rng = np.random.default_rng(57)
    B, Lmax = 3, 9
    C = rng.standard_normal((B, Lmax, 512))
    R = rng.standard_normal((B, Lmax, 64))
    kv_new = rng.standard_normal((B, 512))
    pe_new = rng.standard_normal((B, 64))
    lens = np.array([1, 9, 4])
    C2, R2 = oracle.cache_append(C, R, kv_new, pe_new, lens, YARN)
    for b, L in enumerate(lens):
        other = [t for t in range(Lmax) if t != L - 1]
        assert np.array_equal(C2[b, other], C[b, other]) and np.array_equal(R2[b, other], R[b, other])
        assert np.array_equal(C2[b, L - 1], kv_new[b])              # latent copied, not transformed
    # position 0 rotates by nothing
    assert np.allclose(R2[0, 0], pe_new[0], rtol=0, atol=1e-15)
    # the inputs are left alone
    assert not np.array_equal(C[1, 8], kv_new[1])
    with pytest.raises(ValueError):
        oracle.cache_append(C, R, kv_new, pe_new, np.array([0, 1, 1]), YARN)


def test_cache_append_key_matches_query_at_zero_offset():
    # a query rotated at p_b and the appended key (rotated at its own p_b)
    # have the dot product of the raw vectors, at any p_b; a key rotated at
    # another position, in the other layout or not at all would not
    rng = np.random.default_rng(58)
    B, Lmax = 4, 16384
    lens = np.array([2, 4097, 9000, 16384])
    C = np.zeros((B, Lmax, 512))
    R = np.zeros((B, Lmax, 64))
    kv_new = rng.standard_normal((B, 512))
    pe_new = rng.standard_normal((B, 64))
    _, R2 = oracle.cache_append(C, R, kv_new, pe_new, lens, YARN)
    for b, L in enumerate(lens):
        q = rng.standard_normal(64)
        got = oracle.rope_rotate(q, int(L) - 1, YARN) @ R2[b, L - 1]
        assert abs(got - q @ pe_new[b]) < 1e-11
        assert abs(oracle.rope_rotate(q, int(L) - 1, YARN) @ pe_new[b] - q @ pe_new[b]) > 1e-3


def test_cache_append_then_single_row_decode_is_w_uv_times_new_latent():
    # selecting only the new row after the append gives out[h] = W_UV[h] kv_new
    rng = np.random.default_rng(59)
    B, H, Lmax = 2, 3, 12
    C = rng.standard_normal((B, Lmax, 512))
    R = rng.standard_normal((B, Lmax, 64))
    kv_new = rng.standard_normal((B, 512))
    pe_new = rng.standard_normal((B, 64))
    lens = np.array([5, 12])
    C2, R2 = oracle.cache_append(C, R, kv_new, pe_new, lens, YARN)
    idx = np.array([[4, -1], [11, -1]], dtype=np.int32)
    q_nope = rng.standard_normal((B, H, 128))
    q_pe = rng.standard_normal((B, H, 64))
    w_uk = rng.standard_normal((H, 128, 512)) * 0.05
    w_uv = rng.standard_normal((H, 128, 512)) * 0.05
    out, _ = oracle.decode_attention(q_nope, q_pe, w_uk, w_uv, C2, R2, idx, lens, YARN)
    for b in range(B):
        for h in range(H):
            assert np.allclose(out[b, h], w_uv[h] @ kv_new[b], rtol=1e-12, atol=1e-12)
