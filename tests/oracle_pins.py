"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin takes an ``oracle.OracleLib`` and raises AssertionError when the
oracle disagrees with a value fixed by the page or by mathematics: the IEEE
binary16 definition (via numpy's own conversion), exact rational arithmetic,
closed forms, invariants, an independent direct formula and torch's own
scaled-dot-product attention.  ``test_oracle.py`` runs every pin on the real
oracle; ``test_oracle_mutants.py`` runs them on deliberately broken copies of
the oracle source and requires each copy to fail at least one pin.

The page is "Developing Apple Metal Kernels in Rust - A Deep Dive Through
Attention": section "The MSL, briefly" defines the computation, section
"Testing" the worked cases in ``golden/page_cases.json``.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def page_cases():
    with open(os.path.join(GOLDEN, "page_cases.json")) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _randn_f16(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float16)


def _page_fill(n):
    """(i % 10) * 0.1 computed in f32, then rounded to f16 (page "Testing")."""
    i = np.arange(n)
    return ((i % 10).astype(np.float32) * np.float32(0.1)).astype(np.float16)


# ---------------------------------------------------------------- decoder


def pin_half_decoder_all_patterns(orc):
    """Every binary16 pattern decodes to numpy's own fp16->fp64 value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "finite/inf patterns differ"
    # sign of zero is kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


# ---------------------------------------------------------------- scores


def pin_one_hot_query_scores(orc):
    """q = e_i gives s[h,p] = k[p,h,i] / sqrt(D); D = 64 makes the scale 1/8 exact."""
    rng = _rng(1)
    S, H, D = 9, 3, 64
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    q = np.zeros((H, D), np.float16)
    picks = [5, 17, 63]
    for h, i in enumerate(picks):
        q[h, i] = 1.0
    _, s, _ = orc.decode(q, k, v, S - 1, want_scores=True)
    for h, i in enumerate(picks):
        assert np.array_equal(s[h], k[:, h, i].astype(np.float64) / 8.0), h


def pin_all_ones_score(orc):
    """q = k = 1 gives s = D / sqrt(D) = sqrt(D) (exact for D = 16, 64, 256)."""
    for D in (16, 64, 256):
        q = np.ones((2, D), np.float16)
        k = np.ones((3, 2, D), np.float16)
        _, s, _ = orc.decode(q, k, k, 2, want_scores=True)
        assert np.all(s == math.sqrt(D)), D


def pin_page_cases_exact_scores(orc):
    """The page's three test cases: scores equal the exact dot product times
    1/sqrt(D) (to 1e-14 relative, far inside the page's 0.5), and every
    position after current_pos reads back as exactly -inf.

    Exactness: every finite fp16 value times 2^24 is an integer, so the dot
    product times 2^48 is an exact int64 sum here (|values| < 1)."""
    meta = page_cases()
    for case in meta["cases"]:
        H, D, S, cp = case["n_heads"], case["head_dim"], case["seq_len"], case["current_pos"]
        q = _page_fill(H * D).reshape(H, D)
        k = _page_fill(S * H * D).reshape(S, H, D)
        _, s, _ = orc.decode(q, k, k, cp, want_scores=True)
        qi = (q.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        ki = (k.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        assert np.all(q.astype(np.float64) * 2.0 ** 24 == qi)
        assert np.abs(qi).max() * np.abs(ki).max() * D < 2 ** 62
        exact = np.einsum("hd,phd->hp", qi, ki)          # int64, exact
        ref = exact.astype(np.float64) / 2.0 ** 48 / math.sqrt(D)
        L = cp + 1
        assert np.all(s[:, L:] == -math.inf), case["name"]
        err = np.abs(s[:, :L] - ref[:, :L])
        assert np.all(err <= 1e-14 * np.maximum(1.0, np.abs(ref[:, :L]))), case["name"]
        assert np.all(err < meta["score_tolerance_abs"])


# ---------------------------------------------------------------- softmax


def pin_weights_sum_to_one(orc):
    rng = _rng(2)
    for (S, H, D, cp) in [(50, 3, 16, 49), (70, 2, 40, 20), (5, 1, 8, 0)]:
        q = _randn_f16(rng, (H, D), 3.0)
        k = _randn_f16(rng, (S, H, D))
        _, _, w = orc.decode(q, k, k, cp, want_weights=True)
        assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 1e-12)
        assert np.all(w[:, cp + 1:] == 0.0)
        assert np.all(w[:, : cp + 1] > 0.0)


def pin_two_positions_closed_form(orc):
    """Two positions with s0 = a/2, s1 = b/2 (D = 4, q = e_0): w0 = 1/(1+e^{s1-s0})."""
    D, H = 4, 1
    for a, b in [(1.0, 3.0), (-2.5, 4.0), (7.0, 7.0)]:
        q = np.array([[1, 0, 0, 0]], np.float16)
        k = np.zeros((2, H, D), np.float16)
        k[0, 0, 0], k[1, 0, 0] = a, b
        v = np.zeros((2, H, D), np.float16)
        v[0, 0, :] = [1, 2, -1, 0.5]
        v[1, 0, :] = [-3, 0.25, 4, 1]
        out, s, w = orc.decode(q, k, v, 1, want_scores=True, want_weights=True)
        assert s[0, 0] == a / 2 and s[0, 1] == b / 2
        w0 = 1.0 / (1.0 + math.exp(b / 2 - a / 2))
        assert abs(w[0, 0] - w0) <= 1e-15 and abs(w[0, 1] - (1 - w0)) <= 1e-15
        ref = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
        assert np.allclose(out[0], ref, rtol=0, atol=1e-14)


def pin_large_scores_stay_finite(orc):
    """Scores in the thousands: the max-shifted softmax of the page stays
    finite and picks the largest score's row (exp without the shift overflows)."""
    D, H, S = 16, 2, 6
    q = np.full((H, D), 60.0, np.float16)
    k = np.zeros((S, H, D), np.float16)
    k[:, 0, :] = np.array([10, 20, 30, 40, 50, 45], np.float16)[:, None]   # best p=4
    k[:, 1, :] = -np.array([10, 20, 30, 40, 50, 45], np.float16)[:, None]  # best p=0
    rng = _rng(3)
    v = _randn_f16(rng, (S, H, D))
    out, s, _ = orc.decode(q, k, v, S - 1, want_scores=True)
    assert np.all(np.isfinite(out))
    assert s[0, 4] == 60.0 * 50.0 * D / 4.0
    assert np.array_equal(out[0], v[4, 0].astype(np.float64))
    assert np.array_equal(out[1], v[0, 1].astype(np.float64))


# ---------------------------------------------------------------- PV


def pin_identical_keys_give_mean_of_values(orc):
    rng = _rng(4)
    S, H, D, cp = 40, 3, 24, 29
    q = _randn_f16(rng, (H, D), 2.0)
    k = np.broadcast_to(_randn_f16(rng, (1, H, D)), (S, H, D)).copy()
    v = _randn_f16(rng, (S, H, D))
    out, _, _ = orc.decode(q, k, v, cp)
    ref = v[: cp + 1].astype(np.float64).mean(axis=0)
    assert np.allclose(out, ref, rtol=0, atol=1e-14)


def pin_dominant_score_returns_its_row(orc):
    """K[p*,h] = q[h] and every other K row 0: s_{p*} - s_other = |q|^2/sqrt(D) = 50.9,
    so the output is V[p*] up to about 32 e^-50.9."""
    rng = _rng(5)
    S, H, D = 33, 4, 32
    q = (3.0 * rng.choice([-1.0, 1.0], (H, D))).astype(np.float16)
    k = np.zeros((S, H, D), np.float16)
    stars = [0, 7, 20, 32]
    for h, p in enumerate(stars):
        k[p, h] = q[h]
    v = _randn_f16(rng, (S, H, D))
    out, _, _ = orc.decode(q, k, v, S - 1)
    for h, p in enumerate(stars):
        assert np.allclose(out[h], v[p, h].astype(np.float64), rtol=0, atol=1e-15), h


def pin_first_position_only(orc):
    """current_pos = 0: one weight equal to 1, the output is V[0] exactly."""
    rng = _rng(6)
    S, H, D = 12, 5, 20
    q = _randn_f16(rng, (H, D), 4.0)
    k = _randn_f16(rng, (S, H, D), 4.0)
    v = _randn_f16(rng, (S, H, D))
    out, _, _ = orc.decode(q, k, v, 0)
    assert np.array_equal(out, v[0].astype(np.float64))


def pin_masked_rows_never_matter(orc):
    """Any K/V bits after current_pos (huge, infinite, NaN) leave the output
    bit-identical, and equal to the cache cut at current_pos."""
    rng = _rng(7)
    S, H, D, cp = 30, 3, 16, 17
    q = _randn_f16(rng, (H, D))
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    base, s0, _ = orc.decode(q, k, v, cp, want_scores=True)
    cut, _, _ = orc.decode(q, k[: cp + 1].copy(), v[: cp + 1].copy(), cp)
    assert np.array_equal(base, cut)
    for fill in (np.float16(65504), np.float16(-np.inf), np.float16(np.nan)):
        k2, v2 = k.copy(), v.copy()
        k2[cp + 1:] = fill
        v2[cp + 1:] = -fill
        out, s2, _ = orc.decode(q, k2, v2, cp, want_scores=True)
        assert np.array_equal(out, base)
        assert np.array_equal(s2, s0)
    k3 = k.copy()
    k3[cp + 1:] = _randn_f16(rng, (S - cp - 1, H, D), 10.0)
    out, _, _ = orc.decode(q, k3, v, cp)
    assert np.array_equal(out, base)


def pin_current_pos_beyond_cache_masks_nothing(orc):
    rng = _rng(8)
    S, H, D = 21, 2, 8
    q = _randn_f16(rng, (H, D))
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    a, sa, _ = orc.decode(q, k, v, S - 1, want_scores=True)
    for cp in (S, S + 7, 2 ** 32 - 1):
        b, sb, _ = orc.decode(q, k, v, cp, want_scores=True)
        assert np.array_equal(a, b) and np.array_equal(sa, sb)
    assert np.all(np.isfinite(sa))


# ---------------------------------------------------------------- independent formulas


def direct_formula(q, k, v, cp):
    """exp(s)/sum(exp(s)) with no max shift, from numpy's fp16 decoding
    (valid for small |s|).  Shapes: q [H,D], k/v [S,H,D]."""
    D = q.shape[-1]
    L = min(cp, k.shape[0] - 1) + 1
    qf = q.astype(np.float64)
    kf = k[:L].astype(np.float64)
    vf = v[:L].astype(np.float64)
    s = np.einsum("hd,phd->hp", qf, kf) / np.sqrt(D)
    e = np.exp(s)
    w = e / e.sum(axis=1, keepdims=True)
    return np.einsum("hp,phd->hd", w, vf), s


def pin_direct_formula_bruteforce(orc):
    rng = _rng(9)
    shapes = [(1, 1, 1, 0), (7, 3, 5, 6), (13, 2, 48, 9), (35, 8, 48, 34), (64, 12, 64, 31),
              (3, 5, 130, 2), (100, 4, 256, 99), (17, 9, 7, 16)]
    for (S, H, D, cp) in shapes:
        q = _randn_f16(rng, (H, D))
        k = _randn_f16(rng, (S, H, D))
        v = _randn_f16(rng, (S, H, D))
        out, s, _ = orc.decode(q, k, v, cp, want_scores=True)
        ref, sref = direct_formula(q, k, v, cp)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13), (S, H, D, cp)
        assert np.allclose(s[:, : cp + 1], sref, rtol=1e-12, atol=1e-13), (S, H, D, cp)


def pin_torch_sdpa_float64(orc):
    """torch's own scaled_dot_product_attention in float64 on the CPU, with
    its default 1/sqrt(D) scale and a boolean mask hiding p > current_pos."""
    rng = _rng(10)
    for (S, H, D, cp) in [(40, 4, 64, 25), (19, 3, 48, 18), (9, 2, 128, 0)]:
        q = _randn_f16(rng, (H, D), 2.0)
        k = _randn_f16(rng, (S, H, D))
        v = _randn_f16(rng, (S, H, D))
        out, _, _ = orc.decode(q, k, v, cp)
        qt = torch.from_numpy(q.astype(np.float64)).view(H, 1, D)
        kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).contiguous()
        vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).contiguous()
        mask = (torch.arange(S) <= cp).view(1, 1, S).expand(H, 1, S)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        assert np.allclose(out, ref.view(H, D).numpy(), rtol=1e-12, atol=1e-13), (S, H, D, cp)


# ---------------------------------------------------------------- invariants


def pin_position_permutation_invariance(orc):
    rng = _rng(11)
    S, H, D, cp = 26, 3, 32, 21
    q = _randn_f16(rng, (H, D))
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    base, _, _ = orc.decode(q, k, v, cp)
    perm = np.concatenate([rng.permutation(cp + 1), np.arange(cp + 1, S)])
    out, _, _ = orc.decode(q, k[perm].copy(), v[perm].copy(), cp)
    assert np.allclose(out, base, rtol=0, atol=1e-14)


def pin_linear_in_values(orc):
    """out(V1 + V2) = out(V1) + out(V2) with V1, V2 small integers (exact in fp16)."""
    rng = _rng(12)
    S, H, D, cp = 20, 2, 16, 14
    q = _randn_f16(rng, (H, D))
    k = _randn_f16(rng, (S, H, D))
    v1 = rng.integers(-8, 8, (S, H, D)).astype(np.float16)
    v2 = rng.integers(-8, 8, (S, H, D)).astype(np.float16)
    o1, _, _ = orc.decode(q, k, v1, cp)
    o2, _, _ = orc.decode(q, k, v2, cp)
    o12, _, _ = orc.decode(q, k, (v1 + v2).astype(np.float16), cp)
    assert np.allclose(o12, o1 + o2, rtol=0, atol=1e-13)


def pin_output_within_value_range(orc):
    """The output is a convex combination of the unmasked V rows (weights >= 0
    summing to 1), so min_p V[p,h,d] <= out[h,d] <= max_p V[p,h,d] over the
    positions p <= current_pos, up to rounding of the weighted sum; with V of
    one sign and masked rows far outside that range, the bound also shows
    that no masked row and no negative weight enters."""
    rng = _rng(25)
    S, H, D, cp = 40, 3, 12, 26
    q = _randn_f16(rng, (H, D)) * np.float16(3)
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    v[cp + 1:] = np.float16(1000)               # masked rows far above any valid value
    out, _, w = orc.decode(q, k, v, cp, want_weights=True)
    assert np.all(w[:, :cp + 1] >= 0.0) and np.all(w[:, cp + 1:] == 0.0)
    vv = v[:cp + 1].astype(np.float64)
    lo, hi = vv.min(axis=0), vv.max(axis=0)
    slack = 1e-12 * np.maximum(np.abs(lo), np.abs(hi))
    assert np.all(out >= lo - slack) and np.all(out <= hi + slack)
    vp = np.abs(v[:cp + 1]).astype(np.float16) + np.float16(1)    # all valid values in [1, ...)
    vp = np.concatenate([vp, np.full((S - cp - 1, H, D), -1000, np.float16)])
    out_p, _, _ = orc.decode(q, k, vp, cp)
    assert np.all(out_p >= 1.0 - 1e-12)


def pin_heads_are_independent(orc):
    """Changing the cache of one head leaves every other head's output alone."""
    rng = _rng(13)
    S, H, D, cp = 15, 4, 8, 14
    q = _randn_f16(rng, (H, D))
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    base, _, _ = orc.decode(q, k, v, cp)
    k2, v2 = k.copy(), v.copy()
    k2[:, 2] = _randn_f16(rng, (S, D))
    v2[:, 2] = _randn_f16(rng, (S, D))
    out, _, _ = orc.decode(q, k2, v2, cp)
    for h in (0, 1, 3):
        assert np.array_equal(out[h], base[h])
    assert not np.array_equal(out[2], base[2])


# ---------------------------------------------------------------- second dispatch


def pin_pv_equals_decode_on_representable_scores(orc):
    """With q one-hot and K on a 1/16 grid (D = 64), every score k/8 is an
    fp16 value exactly, so softmax.V from the stored fp16 scores must equal
    the one-pass oracle bit for bit."""
    rng = _rng(20)
    S, H, D, cp = 57, 3, 64, 44
    q = np.zeros((H, D), np.float16)
    for h, i in enumerate([3, 30, 63]):
        q[h, i] = 1.0
    k = (rng.integers(-64, 65, (S, H, D)) / 16.0).astype(np.float16)
    v = _randn_f16(rng, (S, H, D))
    out, s, _ = orc.decode(q, k, v, cp, want_scores=True)
    s16 = s.astype(np.float16)
    assert np.array_equal(s16[:, : cp + 1].astype(np.float64), s[:, : cp + 1])
    assert np.array_equal(orc.pv_from_scores(s16, v, cp), out)


def pin_pv_two_positions_closed_form(orc):
    for a, b in [(0.5, 2.0), (-3.0, 1.25), (7.0, 7.0)]:
        sc = np.array([[a, b]], np.float16)
        v = np.zeros((2, 1, 3), np.float16)
        v[0, 0] = [1, -2, 0.5]
        v[1, 0] = [4, 0.25, -1]
        out = orc.pv_from_scores(sc, v, 1)
        w0 = 1.0 / (1.0 + math.exp(b - a))
        ref = w0 * v[0, 0].astype(np.float64) + (1 - w0) * v[1, 0].astype(np.float64)
        assert np.allclose(out[0], ref, rtol=0, atol=1e-15)


def pin_pv_neg_inf_scores_have_zero_weight(orc):
    """-inf scores inside the valid range weigh nothing, whatever V holds there."""
    rng = _rng(21)
    S, H, D, cp = 20, 2, 8, 15
    sc = _randn_f16(rng, (H, S), 2.0)
    v = _randn_f16(rng, (S, H, D))
    drop = [2, 9, 15]
    sc2, v2 = sc.copy(), v.copy()
    sc2[:, drop] = -np.inf
    v2[drop] = np.nan
    keep = [p for p in range(cp + 1) if p not in drop]
    ref = orc.pv_from_scores(sc[:, keep].copy(), v[keep].copy(), len(keep) - 1)
    out = orc.pv_from_scores(sc2, v2, cp)
    assert np.array_equal(out, ref)


def pin_pv_direct_formula(orc):
    rng = _rng(22)
    for (S, H, D, cp) in [(9, 2, 16, 8), (40, 3, 48, 31), (100, 1, 128, 99)]:
        sc = _randn_f16(rng, (H, S), 1.5)
        v = _randn_f16(rng, (S, H, D))
        out = orc.pv_from_scores(sc, v, cp)
        e = np.exp(sc[:, : cp + 1].astype(np.float64))
        w = e / e.sum(axis=1, keepdims=True)
        ref = np.einsum("hp,phd->hd", w, v[: cp + 1].astype(np.float64))
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13), (S, H, D)


# ------------------------------------------------------- fp16 rounding


def pin_double_to_half_matches_numpy(orc):
    """fp64 -> fp16 rounding agrees with numpy's own conversion everywhere
    that matters: every fp16 value, every midpoint between neighbours (the
    ties), one fp64 step either side of each midpoint, and a log-uniform
    sweep from below the subnormals to past the overflow threshold."""
    bits = np.arange(0x7C01, dtype=np.uint32).astype(np.uint16)   # +0 .. +inf
    vals = bits.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2.0                             # exact in fp64
    rng = _rng(30)
    sweep = np.exp2(rng.uniform(-30.0, 17.5, 200000))
    xs = np.concatenate([vals, mids, np.nextafter(mids, 0.0), np.nextafter(mids, np.inf), sweep,
                         [65504.0, 65519.99, 65520.0, 1e300, 2.0 ** -25, 2.0 ** -26]])
    xs = np.concatenate([xs, -xs])
    got = orc.double_to_half(xs)
    with np.errstate(over="ignore"):
        ref = xs.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, "fp16 rounding differs at %r" % xs[bad[:5]]
    nan = orc.double_to_half(np.array([np.nan]))[0]
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0, "NaN must stay NaN"


def pin_double_to_half_hand_cases(orc):
    """Values fixed by the binary16 format itself."""
    cases = {
        1.0: 0x3C00, -2.0: 0xC000, 65504.0: 0x7BFF, 65520.0: 0x7C00,   # tie at the top: to inf
        2.0 ** -14: 0x0400, 2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000,     # tie to even (0)
        3 * 2.0 ** -25: 0x0002, 1.0 + 2.0 ** -11: 0x3C00,               # ties to even
        1.0 + 3 * 2.0 ** -11: 0x3C02, -0.0: 0x8000, float("inf"): 0x7C00,
    }
    for x, want in cases.items():
        got = int(orc.double_to_half(np.array([x]))[0])
        assert got == want, (x, hex(got), hex(want))


# ----------------------------------------------------------- rotary embedding
# Page "Tutorial 16: Writing Custom Metal Kernels", section "5. Example: Fused
# RoPE Kernel"; test names from the page "Developing Apple Metal Kernels in
# Rust - A Deep Dive Through Attention", section "Testing".


def _dec_pi(prec):
    """pi to `prec` digits by Machin's formula, 16 atan(1/5) - 4 atan(1/239)."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = prec + 10
        eps = Decimal(10) ** -(prec + 8)

        def atan_inv(n):
            x = Decimal(1) / n
            x2, term, total, k = x * x, x, x, 1
            while True:
                term = -term * x2
                k += 2
                t = term / k
                if abs(t) < eps:
                    return total
                total += t

        return +(16 * atan_inv(5) - 4 * atan_inv(239))


def _dec_angle_cos_sin(pos, i, dims, base, prec=50):
    """cos and sin of pos * base^(-2i/dims), in decimal arithmetic (reduction
    modulo 2 pi and Taylor series), independent of the C math library."""
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = prec + 20
        theta = Decimal(base) ** (Decimal(-2 * i) / Decimal(dims))
        t = Decimal(pos) * theta
        two_pi = 2 * _dec_pi(prec + 20)
        r = t - (t / two_pi).to_integral_value() * two_pi
        eps = Decimal(10) ** -(prec + 5)
        c, s = Decimal(0), Decimal(0)
        term, n = Decimal(1), 0   # r^n / n!
        while True:
            if n % 4 == 0:
                c += term
            elif n % 4 == 1:
                s += term
            elif n % 4 == 2:
                c -= term
            else:
                s -= term
            n += 1
            term = term * r / n
            if abs(term) < eps and n > 4:
                break
        return float(c), float(s), float(t)


def _unit(D, j):
    x = np.zeros(D, dtype=np.float16)
    x[j] = 1.0
    return x


def pin_rope_position_zero_is_identity(orc):
    """Position 0 turns every pair by angle 0 (page test
    test_rope_position_zero_is_identity)."""
    rng = _rng(31)
    for D, dims, trad in [(64, 64, False), (128, 128, True), (96, 32, False), (10, 6, True)]:
        x = _randn_f16(rng, (5, D))
        out = orc.rope(x, 0, dims=dims, traditional=trad)
        assert np.array_equal(out, x.astype(np.float64)), (D, dims, trad)


def pin_rope_positions_differ(orc):
    """Different positions give different vectors (page test
    test_rope_different_positions_differ), with the tail past dims untouched."""
    rng = _rng(32)
    x = _randn_f16(rng, (1, 80))
    a = orc.rope(x, 5, dims=64)
    b = orc.rope(x, 6, dims=64)
    assert np.abs(a[:, :64] - b[:, :64]).max() > 1e-3
    assert np.array_equal(a[:, 64:], x[:, 64:].astype(np.float64))
    assert np.array_equal(b[:, 64:], x[:, 64:].astype(np.float64))


def pin_rope_single_pair_closed_form(orc):
    """dims = 2: one pair with frequency 1, so e_0 -> (cos p, sin p) and
    e_1 -> (-sin p, cos p), for small and very large positions (decimal
    reference, so the large angles check the fp64 reduction too)."""
    for pos in [1, 2, 3, 1000, 20000, 131071]:
        c, s, t = _dec_angle_cos_sin(pos, 0, 2, 10000)
        tol = 1e-13 + 4e-16 * t
        for trad in (False, True):
            o0 = orc.rope(_unit(2, 0)[None], pos, dims=2, traditional=trad)[0]
            o1 = orc.rope(_unit(2, 1)[None], pos, dims=2, traditional=trad)[0]
            assert abs(o0[0] - c) < tol and abs(o0[1] - s) < tol, (pos, o0, c, s)
            assert abs(o1[0] + s) < tol and abs(o1[1] - c) < tol, (pos, o1, c, s)


def pin_rope_frequencies_and_pairing(orc):
    """head_dim 6, dims 4: pair i turns by pos * base^(-2i/dims).  Half-split
    pairs are (0, 2) and (1, 3); traditional pairs are (0, 1) and (2, 3);
    elements 4 and 5 pass through.  Unit vectors show every entry."""
    D, dims = 6, 4
    for base, pos in [(10000.0, 100), (100.0, 10), (500000.0, 777)]:
        for trad in (False, True):
            pairs = [(0, 1), (2, 3)] if trad else [(0, 2), (1, 3)]
            for i, (ia, ib) in enumerate(pairs):
                c, s, t = _dec_angle_cos_sin(pos, i, dims, base)
                tol = 1e-13 + 4e-16 * t
                oa = orc.rope(_unit(D, ia)[None], pos, dims=dims, base=base, traditional=trad)[0]
                ob = orc.rope(_unit(D, ib)[None], pos, dims=dims, base=base, traditional=trad)[0]
                want_a = np.zeros(D)
                want_a[ia], want_a[ib] = c, s
                want_b = np.zeros(D)
                want_b[ia], want_b[ib] = -s, c
                assert np.abs(oa - want_a).max() < tol, (base, pos, trad, i, oa, want_a)
                assert np.abs(ob - want_b).max() < tol, (base, pos, trad, i, ob, want_b)
            for j in (4, 5):
                o = orc.rope(_unit(D, j)[None], pos, dims=dims, base=base, traditional=trad)[0]
                assert np.array_equal(o, _unit(D, j).astype(np.float64))


def pin_rope_preserves_pair_norms(orc):
    """A rotation keeps the length of every pair."""
    rng = _rng(33)
    D, dims = 128, 96
    x = _randn_f16(rng, (64, D), 3.0)
    pos = rng.integers(0, 200000, 64)
    for trad in (False, True):
        out = orc.rope(x, pos, dims=dims, traditional=trad)
        xd = x.astype(np.float64)
        if trad:
            n_in = xd[:, 0:dims:2] ** 2 + xd[:, 1:dims:2] ** 2
            n_out = out[:, 0:dims:2] ** 2 + out[:, 1:dims:2] ** 2
        else:
            h = dims // 2
            n_in = xd[:, :h] ** 2 + xd[:, h:dims] ** 2
            n_out = out[:, :h] ** 2 + out[:, h:dims] ** 2
        assert np.allclose(n_out, n_in, rtol=1e-12, atol=1e-12)


def pin_rope_scores_depend_on_relative_position(orc):
    """<R(m) q, R(n) k> = <R(m - n) q, k>: the rotated dot product depends
    only on the distance between the two positions."""
    rng = _rng(34)
    for D, dims, trad in [(128, 128, False), (64, 32, True)]:
        q = _randn_f16(rng, (1, D))
        k = _randn_f16(rng, (1, D))
        scale = np.linalg.norm(q.astype(np.float64)) * np.linalg.norm(k.astype(np.float64))
        for m, n in [(5, 0), (100, 37), (4096, 4000), (131071, 131000), (70000, 12)]:
            lhs = float(orc.rope(q, m, dims=dims, traditional=trad)[0]
                        @ orc.rope(k, n, dims=dims, traditional=trad)[0])
            rhs = float(orc.rope(q, m - n, dims=dims, traditional=trad)[0] @ k[0].astype(np.float64))
            assert abs(lhs - rhs) < 1e-10 * scale * (1 + m / 1000.0), (D, m, n, lhs, rhs)


def pin_rope_traditional_is_interleaved_half_split(orc):
    """Traditional pairing is the half-split pairing applied to the vector
    with its even elements moved to the front and its odd ones after them."""
    rng = _rng(35)
    D, dims = 64, 48
    x = _randn_f16(rng, (8, D))
    pos = rng.integers(0, 50000, 8)
    perm = np.concatenate([np.arange(0, dims, 2), np.arange(1, dims, 2), np.arange(dims, D)])
    trad = orc.rope(x, pos, dims=dims, traditional=True)
    split = orc.rope(np.ascontiguousarray(x[:, perm]), pos, dims=dims, traditional=False)
    assert np.array_equal(trad[:, perm], split)


def pin_decode_step_first_position(orc):
    """A step at position 0 attends to its own row only: the output is v_new
    exactly, and the appended key is k_new (angle 0)."""
    rng = _rng(36)
    S, H, D = 8, 3, 32
    kc = _randn_f16(rng, (S, H, D)).view(np.uint16).copy()
    vc = _randn_f16(rng, (S, H, D)).view(np.uint16).copy()
    q, kn, vn = (_randn_f16(rng, (H, D)) for _ in range(3))
    r = orc.decode_step(q, kn, vn, kc, vc, 0, dims=D)
    assert np.array_equal(r["out"], vn.astype(np.float64))
    assert np.array_equal(kc[0], kn.view(np.uint16)) and np.array_equal(vc[0], vn.view(np.uint16))


def pin_decode_step_against_torch(orc):
    """The step is rotate (at pos), round to fp16, write row pos, attend over
    0..pos: rebuilt here with torch float64 for the rotation and torch's
    scaled-dot-product attention, rows after pos filled with garbage."""
    rng = _rng(37)
    for S, H, D, dims, cp, trad in [(40, 4, 64, 64, 17, False), (33, 2, 128, 96, 32, True),
                                    (16, 3, 32, 32, 99, False)]:
        kc = _randn_f16(rng, (S, H, D)).view(np.uint16).copy()
        vc = _randn_f16(rng, (S, H, D)).view(np.uint16).copy()
        q, kn, vn = (_randn_f16(rng, (H, D)) for _ in range(3))
        kc0, vc0 = kc.copy(), vc.copy()
        r = orc.decode_step(q, kn, vn, kc, vc, cp, dims=dims, traditional=trad)
        pos = min(cp, S - 1)

        def t_rope(x):
            x = torch.from_numpy(x.astype(np.float64))
            i = torch.arange(dims // 2, dtype=torch.float64)
            ang = pos * torch.pow(torch.tensor(10000.0, dtype=torch.float64), -2.0 * i / dims)
            c, s = torch.cos(ang), torch.sin(ang)
            y = x.clone()
            ia = torch.arange(0, dims, 2) if trad else torch.arange(dims // 2)
            ib = ia + 1 if trad else ia + dims // 2
            a, b = x[:, ia], x[:, ib]
            y[:, ia] = a * c - b * s
            y[:, ib] = a * s + b * c
            return y.numpy().astype(np.float16)

        q16, k16 = t_rope(q), t_rope(kn)
        assert np.array_equal(r["q16"], q16.view(np.uint16))
        assert np.array_equal(r["k16"], k16.view(np.uint16))
        want_k, want_v = kc0.copy(), vc0.copy()
        want_k[pos], want_v[pos] = k16.view(np.uint16), vn.view(np.uint16)
        assert np.array_equal(kc, want_k) and np.array_equal(vc, want_v)
        kt = torch.from_numpy(want_k[: pos + 1].view(np.float16).astype(np.float64)).transpose(0, 1)
        vt = torch.from_numpy(want_v[: pos + 1].view(np.float16).astype(np.float64)).transpose(0, 1)
        qt = torch.from_numpy(q16.astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous())
        assert np.allclose(r["out"], ref[:, 0, :].numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- row softmax
# The Foundry notes' fm_softmax (section "API Reference": x [rows, cols] ->
# out [rows, cols]), in the max-shifted form of the page "Developing Apple
# Metal Kernels in Rust - A Deep Dive Through Attention" ("The MSL, briefly").


def pin_softmax_rows_sum_to_one_and_match_torch(orc):
    """Rows sum to 1, and every value equals torch's own float64 softmax."""
    rng = _rng(40)
    for rows, cols, sigma in [(1, 1, 1.0), (3, 7, 1.0), (16, 1000, 3.0), (4, 5000, 8.0)]:
        x = (rng.standard_normal((rows, cols)) * sigma).astype(np.float32)
        out = orc.softmax_rows(x)
        assert np.allclose(out.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        ref = torch.softmax(torch.from_numpy(x.astype(np.float64)), dim=1).numpy()
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-300), (rows, cols)


def pin_softmax_two_values_closed_form(orc):
    """[a, b] -> [1/(1+e^(b-a)), 1/(1+e^(a-b))]; [x, x] -> [1/2, 1/2] exactly."""
    for a, b in [(0.0, 0.0), (1.0, 3.0), (-20.0, 5.5), (100.0, 100.25)]:
        out = orc.softmax_rows(np.array([[a, b]], np.float32))[0]
        w0 = 1.0 / (1.0 + math.exp(b - a))
        assert abs(out[0] - w0) < 1e-15 and abs(out[1] - (1.0 - w0)) < 1e-15, (a, b, out)
    assert np.array_equal(orc.softmax_rows(np.full((1, 2), 7.5, np.float32))[0], [0.5, 0.5])


def pin_softmax_uniform_row(orc):
    """Equal values give exactly 1/cols for power-of-two lengths."""
    for cols in (1, 2, 64, 4096):
        out = orc.softmax_rows(np.full((2, cols), -3.25, np.float32))
        assert np.all(out == 1.0 / cols), cols


def pin_softmax_shift_invariant_exactly(orc):
    """Adding the same integer to every entry of an integer-valued row leaves
    x - max unchanged, so the output is bitwise unchanged."""
    rng = _rng(41)
    x = rng.integers(-40, 40, (5, 300)).astype(np.float32)
    base = orc.softmax_rows(x)
    for c in (1.0, -1000.0, 65536.0):
        assert np.array_equal(orc.softmax_rows(x + np.float32(c)), base), c


def pin_softmax_large_values_stay_finite(orc):
    """Entries in the thousands: the max shift is there (exp(1000) overflows)."""
    x = np.array([[1000.0, 999.0, 998.0], [3e4, 3e4, -3e4]], np.float32)
    out = orc.softmax_rows(x)
    assert np.all(np.isfinite(out))
    e = np.exp([0.0, -1.0, -2.0])
    assert np.allclose(out[0], e / e.sum(), rtol=1e-15, atol=0)
    assert np.array_equal(out[1], [0.5, 0.5, 0.0])


def pin_softmax_masked_entries(orc):
    """-inf entries weigh exactly 0 and leave the rest as the shorter row;
    a row of -inf only is NaN (the plain definition: m = -inf)."""
    rng = _rng(42)
    x = rng.standard_normal((3, 50)).astype(np.float32)
    xm = x.copy()
    xm[:, 30:] = -np.inf
    out = orc.softmax_rows(xm)
    assert np.all(out[:, 30:] == 0.0)
    assert np.array_equal(out[:, :30], orc.softmax_rows(np.ascontiguousarray(x[:, :30])))
    nan_row = orc.softmax_rows(np.full((1, 4), -np.inf, np.float32))
    assert np.all(np.isnan(nan_row))


def pin_softmax_rows_are_independent_and_row_major(orc):
    """Row r of the output depends on row r of x only, laid out row-major."""
    rng = _rng(43)
    x = rng.standard_normal((6, 37)).astype(np.float32)
    whole = orc.softmax_rows(x)
    for r in range(6):
        assert np.array_equal(whole[r], orc.softmax_rows(np.ascontiguousarray(x[r:r + 1]))[0])
    col = orc.softmax_rows(np.ascontiguousarray(x[:, :1]))
    assert np.all(col == 1.0)


def pin_softmax_equals_decode_weights(orc):
    """The decode oracle's softmax weights are the row softmax of its scores
    (two separately written routines): scores rounded to fp32 first, so they
    agree to the fp32 rounding of the scores (|ds| <= 2^-24 |s|)."""
    rng = _rng(44)
    S, H, D, cp = 200, 3, 64, 150
    q, k, v = _randn_f16(rng, (H, D)), _randn_f16(rng, (S, H, D)), _randn_f16(rng, (S, H, D))
    _, s, w = orc.decode(q, k, v, cp, want_scores=True, want_weights=True)
    out = orc.softmax_rows(s.astype(np.float32))
    bound = w * (2.0 ** -23) * (np.abs(s[:, : cp + 1]).max() + 1) * 4
    assert np.all(out[:, cp + 1:] == 0.0)
    assert np.all(np.abs(out[:, : cp + 1] - w[:, : cp + 1]) <= bound[:, : cp + 1] + 1e-300)


# ---------------------------------------------------------------- batch and host threads
# The pages define one sequence; a batch is read as independent sequences of
# one cache capacity, each with its own current_pos (the oracle's batched form
# loops over single-sequence calls).  Host threads only split heads or rows.


def _sdpa_f64(q, k, v, L):
    """torch float64 attention of one sequence: q [H, D], k/v [S, H, D], the
    first L positions visible (boolean mask)."""
    S, H, D = k.shape
    qt = torch.from_numpy(q.astype(np.float64)).view(H, 1, D)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).contiguous()
    mask = (torch.arange(S) < L).view(1, 1, S).expand(H, 1, S)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return ref.view(H, D).numpy()


def pin_batched_is_independent_sequences(orc):
    """Five sequences with distinct queries, caches and lengths (current_pos
    0, the last slot, past the cache, two in between): each output equals
    torch's float64 attention under that sequence's own mask, and the
    single-sequence oracle on that sequence bitwise; each score row is -inf
    exactly after that sequence's current_pos."""
    rng = _rng(40)
    B, S, H, D = 5, 23, 3, 16
    cps = [0, S - 1, S + 4, 7, 12]
    q = _randn_f16(rng, (B, H, D), 1.5)
    k = _randn_f16(rng, (B, S, H, D))
    v = _randn_f16(rng, (B, S, H, D))
    for threads in (1, 2):
        out, sc = orc.decode_batched(q, k, v, np.array(cps, dtype=np.int64), want_scores=True,
                                     threads=threads)
        assert out.shape == (B, H, D) and sc.shape == (B, H, S)
        for b, cp in enumerate(cps):
            L = min(cp, S - 1) + 1
            assert np.allclose(out[b], _sdpa_f64(q[b], k[b], v[b], L), rtol=1e-12, atol=1e-13), b
            one, s1, _ = orc.decode(q[b], k[b], v[b], cp, want_scores=True)
            assert np.array_equal(out[b], one), b
            assert np.array_equal(sc[b], s1), b
            assert np.all(sc[b][:, L:] == -np.inf), b
            assert np.all(np.isfinite(sc[b][:, :L])), b


def pin_host_threads_split_heads_exactly(orc):
    """Heads split over host threads, thread counts that do not divide the
    head count among them: every head is computed once, by the same routine,
    so outputs, scores and weights are bitwise those of one thread, and match
    torch's float64 attention."""
    rng = _rng(41)
    S, H, D, cp = 19, 7, 24, 15
    q = _randn_f16(rng, (H, D), 1.5)
    k = _randn_f16(rng, (S, H, D))
    v = _randn_f16(rng, (S, H, D))
    base, s1, w1 = orc.decode(q, k, v, cp, want_scores=True, want_weights=True)
    ref = _sdpa_f64(q, k, v, cp + 1)
    for t in (2, 3, 5, 6, 7, 9):
        out, s, w = orc.decode(q, k, v, cp, want_scores=True, want_weights=True, threads=t)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-13), t
        assert np.array_equal(out, base), t
        assert np.array_equal(s, s1), t
        assert np.array_equal(w, w1), t


def pin_softmax_host_threads_split_rows_exactly(orc):
    """Rows split over host threads (counts that do not divide the row count):
    bitwise the one-thread result, and torch's float64 softmax."""
    rng = _rng(42)
    x = (rng.standard_normal((11, 37)) * 3).astype(np.float32)
    base = orc.softmax_rows(x)
    ref = torch.softmax(torch.from_numpy(x.astype(np.float64)), dim=1).numpy()
    for t in (2, 3, 4, 10, 11, 16):
        out = orc.softmax_rows(x, threads=t)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-15), t
        assert np.array_equal(out, base), t


ALL_PINS = [
    pin_half_decoder_all_patterns,
    pin_one_hot_query_scores,
    pin_all_ones_score,
    pin_page_cases_exact_scores,
    pin_weights_sum_to_one,
    pin_two_positions_closed_form,
    pin_large_scores_stay_finite,
    pin_identical_keys_give_mean_of_values,
    pin_dominant_score_returns_its_row,
    pin_first_position_only,
    pin_masked_rows_never_matter,
    pin_current_pos_beyond_cache_masks_nothing,
    pin_direct_formula_bruteforce,
    pin_torch_sdpa_float64,
    pin_position_permutation_invariance,
    pin_linear_in_values,
    pin_output_within_value_range,
    pin_heads_are_independent,
    pin_pv_equals_decode_on_representable_scores,
    pin_pv_two_positions_closed_form,
    pin_pv_neg_inf_scores_have_zero_weight,
    pin_pv_direct_formula,
    pin_double_to_half_matches_numpy,
    pin_double_to_half_hand_cases,
    pin_rope_position_zero_is_identity,
    pin_rope_positions_differ,
    pin_rope_single_pair_closed_form,
    pin_rope_frequencies_and_pairing,
    pin_rope_preserves_pair_norms,
    pin_rope_scores_depend_on_relative_position,
    pin_rope_traditional_is_interleaved_half_split,
    pin_decode_step_first_position,
    pin_decode_step_against_torch,
    pin_softmax_rows_sum_to_one_and_match_torch,
    pin_softmax_two_values_closed_form,
    pin_softmax_uniform_row,
    pin_softmax_shift_invariant_exactly,
    pin_softmax_large_values_stay_finite,
    pin_softmax_masked_entries,
    pin_softmax_rows_are_independent_and_row_major,
    pin_softmax_equals_decode_weights,
    pin_batched_is_independent_sequences,
    pin_host_threads_split_heads_exactly,
    pin_softmax_host_threads_split_rows_exactly,
]
