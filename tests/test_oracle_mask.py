"""Pins for oracle.block_mask: closed forms, numpy's quantile, pure-Python enumeration and invariants."""
import math
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import block_mask as M


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------------------------------------------ stats (step 1-2)
def test_single_key_block_closed_form():
    """All keys of a block zero except one key x: centroid x/b, radius (b-1)/b * |x| (the other keys sit at
    |x|/b, closer), and a query block of identical rows has that row as its mean."""
    b, D = 8, 5
    x = np.array([3.0, -4.0, 0.0, 12.0, 0.0])          # |x| = 13
    k = np.zeros((1, 1, 2 * b, D))
    k[0, 0, 3] = x
    k[0, 0, b:] = 1.0                                    # second block: identical keys -> radius 0
    q = np.zeros((1, 2, 2 * b, D))
    q[0, 1, :b] = x
    qbar, kbar, r = M.block_stats(q, k, b)
    np.testing.assert_allclose(kbar[0, 0, 0], x / b, atol=1e-15)
    assert abs(r[0, 0, 0] - (b - 1) / b * 13.0) < 1e-13
    assert r[0, 0, 1] == 0.0
    np.testing.assert_allclose(kbar[0, 0, 1], 1.0)
    np.testing.assert_allclose(qbar[0, 1, 0], x, atol=1e-15)
    np.testing.assert_allclose(qbar[0, 0], 0.0)


def test_stats_equal_explicit_loops():
    b = 4
    q, k = rnd(1, 1, 4, 12, 3), rnd(2, 1, 2, 12, 3)
    qbar, kbar, r = M.block_stats(q, k, b)
    for h in range(4):
        for i in range(3):
            for d in range(3):
                assert abs(qbar[0, h, i, d] - sum(q[0, h, i * b + t, d] for t in range(b)) / b) < 1e-14
    for g in range(2):
        for j in range(3):
            c = [sum(k[0, g, j * b + t, d] for t in range(b)) / b for d in range(3)]
            far = max(math.sqrt(sum((k[0, g, j * b + t, d] - c[d]) ** 2 for d in range(3))) for t in range(b))
            assert abs(r[0, g, j] - far) < 1e-13


# ---------------------------------------------------------------------------------------------- quantiles (step 3)
@pytest.mark.parametrize("n", [1, 2, 3, 10, 11, 512, 1024, 1000])
@pytest.mark.parametrize("pct", [0, 10, 50, 90, 100, 37])
def test_quantile_matches_numpy_linear(n, pct):
    x = np.sort(np.random.default_rng(n * 101 + pct).random(n) * 10)
    mine = M.quantile_type7(x, pct)
    ref = float(np.quantile(x, pct / 100.0, method="linear"))
    assert abs(mine - ref) <= 1e-12 * max(1.0, abs(ref))


@pytest.mark.parametrize("n,expected", [(512, 52), (1024, 103), (100, 10)])
def test_flag_count_with_alpha_one(n, expected):
    """With alpha = 1 the threshold is the interpolated 90th percentile, which sits strictly between the two
    order statistics around (n-1)*0.9 when that position is not an integer; the count above it is
    n-1-floor(0.9(n-1))."""
    x = np.random.default_rng(n).permutation(np.arange(n, dtype=np.float64) * 0.37 + 1.0)
    med, p90, tau = M.rescue_threshold(x, 1.0)
    assert int((x > tau).sum()) == n - 1 - (9 * (n - 1)) // 10 == expected
    assert abs(med - float(np.median(x))) < 1e-12


def test_threshold_moves_with_alpha_in_the_right_direction():
    x = np.random.default_rng(3).random(200)
    _, _, t0 = M.rescue_threshold(x, 0.0)
    _, _, t1 = M.rescue_threshold(x, 1.0)
    _, _, t2 = M.rescue_threshold(x, 2.0)
    assert abs(t0 - np.median(x)) < 1e-15 and t0 < t1 < t2
    assert abs(t2 - (2 * np.quantile(x, 0.9) - np.median(x))) < 1e-12
    assert M.rescue_threshold(x, math.inf)[2] == math.inf


# -------------------------------------------------------------------------------------------- select (steps 4-7)
def brute_mask(qbar, kbar, rad, scale, keep, alpha, G, lo=50, hi=90):
    """Pure-Python statement of the rule for tiny sizes (sorted() with an explicit key, Fraction ceilings)."""
    B, Hq, nb, D = qbar.shape
    out = np.zeros((B, Hq, nb, nb), dtype=np.uint8)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            xs = sorted(float(r) for r in rad[b, g])
            def qt(p):
                pos = Fraction((len(xs) - 1) * p, 100)
                lo_i = math.floor(pos)
                f = float(pos - lo_i)
                return xs[lo_i] if lo_i + 1 >= len(xs) or f == 0 else xs[lo_i] + f * (xs[lo_i + 1] - xs[lo_i])
            tau = math.inf if math.isinf(alpha) else qt(lo) + alpha * (qt(hi) - qt(lo))
            for i in range(nb):
                score = {j: scale * sum(qbar[b, h, i, d] * kbar[b, g, j, d] for d in range(D)) for j in range(i + 1)}
                budget = math.ceil(Fraction((i + 1) * keep, 1000))
                ranked = sorted(range(i + 1), key=lambda j: (-score[j], j))
                for j in range(i + 1):
                    if j in ranked[:budget] or rad[b, g, j] > tau or j == i:
                        out[b, h, i, j] = 1
    return out


@pytest.mark.parametrize("keep,alpha", [(100, 1.0), (300, 0.5), (0, math.inf), (1000, math.inf), (250, math.inf),
                                        (0, 0.0)])
def test_mask_equals_enumeration(keep, alpha):
    b, nb = 4, 8
    q, k = rnd(40, 1, 4, b * nb, 3), rnd(41, 1, 2, b * nb, 3)
    res = M.build_mask(q, k, 0.7, b, keep, alpha)
    qbar, kbar, rad = M.block_stats(q, k, b)
    np.testing.assert_array_equal(res.mask, brute_mask(qbar, kbar, rad, 0.7, keep, alpha, 2))


def test_ties_go_to_the_smaller_block_index():
    """Integer centroids make exact score ties; the budget must take the earlier blocks."""
    b, nb, D = 2, 6, 2
    q = np.zeros((1, 1, b * nb, D)); q[..., 0] = 1.0
    k = np.zeros((1, 1, b * nb, D))
    k[0, 0, :, 0] = np.repeat([1.0, 3.0, 3.0, 1.0, 3.0, 0.0], b)       # blocks 1, 2, 4 tie at the top
    res = M.build_mask(q, k, 1.0, b, keep_permille=400, alpha=math.inf)   # row 5: ceil(6*0.4) = 3 picks
    assert res.centroid[0, 0, 5].nonzero()[0].tolist() == [1, 2, 4]
    res2 = M.build_mask(q, k, 1.0, b, keep_permille=200, alpha=math.inf)  # row 5: 2 picks -> the first two ties
    assert res2.centroid[0, 0, 5].nonzero()[0].tolist() == [1, 2]
    assert res2.mask[0, 0, 5].nonzero()[0].tolist() == [1, 2, 5]


def test_mask_invariants():
    b, nb = 8, 16
    q, k = rnd(50, 2, 4, b * nb, 6), rnd(51, 2, 2, b * nb, 6)
    res = M.build_mask(q, k, 0.5, b, keep_permille=200, alpha=1.0)
    m = res.mask.astype(bool)
    assert not np.triu(m, 1).any()
    assert all(m[..., i, i].all() for i in range(nb))
    for i in range(nb):
        assert (res.centroid[..., i, :].sum(-1) == M.centroid_budget(i, 200)).all()
    np.testing.assert_array_equal(res.kv_count, m.sum(-1))
    for bb in range(2):
        for h in range(4):
            for i in range(nb):
                c = res.kv_count[bb, h, i]
                idx = res.kv_index[bb, h, i]
                assert (np.diff(idx[:c]) > 0).all() and idx[c - 1] == i and (idx[c:] == -1).all()
                np.testing.assert_array_equal(idx[:c], np.nonzero(m[bb, h, i])[0])
    full = M.build_mask(q, k, 0.5, b, 1000, 1.0).mask
    np.testing.assert_array_equal(full, np.broadcast_to(np.tril(np.ones((nb, nb), np.uint8)), full.shape))
    cen_only = M.build_mask(q, k, 0.5, b, 200, math.inf)
    eye = np.eye(nb, dtype=bool)
    np.testing.assert_array_equal(cen_only.mask.astype(bool), cen_only.centroid | eye)
    diag = M.build_mask(q, k, 0.5, b, 0, math.inf).mask
    np.testing.assert_array_equal(diag.astype(bool), np.broadcast_to(eye, diag.shape))
    # rescue flags are shared across the query heads of a kv-head group
    G = 2
    for h in range(4):
        resc = res.rescue[:, h // G]
        lower = np.tril(np.ones((nb, nb), bool))
        assert ((m[:, h] | ~(resc[:, None, :] & lower)).all())


def test_rescue_catches_every_planted_block():
    """The planted 6x query keys widen their block's radius far beyond the 90th percentile, so the rescue branch
    flags every planted block, which the centroid branch alone often misses (mean dilution)."""
    inp = W.planted_inputs(3, 1, 8, 2, 64 * 64, 64, block=64, planted_per_mille=100)
    q, k, _ = inp.as_f64()
    res = M.build_mask(q, k, inp.scale, 64, keep_permille=100, alpha=1.0)
    for (b, g, j, u, h, t) in inp.planted:
        assert res.rescue[b, g, j]
        assert res.mask[b, h, t // 64, j] == 1
    # and the planted keys do draw the attention of their query row
    O, _ = A.causal_attention(q[:, :1], k[:, :1], inp.as_f64()[2][:, :1], inp.scale, rows=np.array([0]))
    assert np.isfinite(O).all()


def test_rescue_comparison_is_strict():
    """alpha = 0 with an odd block count puts tau exactly on the median radius; that block is not flagged."""
    b, nb, D = 4, 5, 3
    k = np.zeros((1, 1, b * nb, D))
    for j, mag in enumerate([4.0, 8.0, 2.0, 16.0, 1.0]):       # radii (b-1)/b * mag, median from mag 4
        k[0, 0, j * b, 0] = mag
    q = np.zeros((1, 1, b * nb, D))
    res = M.build_mask(q, k, 1.0, b, keep_permille=0, alpha=0.0)
    assert res.tau[0, 0] == res.radius[0, 0, 0]
    assert res.rescue[0, 0].tolist() == [False, True, False, True, False]
    assert res.mask[0, 0, 4].nonzero()[0].tolist() == [1, 3, 4]


# -------------------------------------------------------------------------------- query-aware rescue (mode 1)
def _two_axis_keys(radii, xs, b=2):
    """Key block j holds (x_j, +r_j) and (x_j, -r_j) (b = 2): centroid (x_j, 0), radius exactly r_j."""
    nb = len(radii)
    k = np.zeros((1, 1, b * nb, 2))
    for j, (r, x) in enumerate(zip(radii, xs)):
        k[0, 0, b * j] = (x, r)
        k[0, 0, b * j + 1] = (x, -r)
    return k


def test_rescue_coefficient_closed_forms():
    assert M.rescue_coefficient(4.0, 12.0) == 8.0 / 12.0
    assert M.rescue_coefficient(3.0, 3.0) == 0.0           # no spread between the reference points
    assert M.rescue_coefficient(0.0, 0.0) == 0.0           # degenerate: p90 = 0
    assert M.rescue_coefficient(0.0, 5.0) == 1.0


def test_query_aware_rescue_hand_case():
    """Six key blocks of two keys in 2-D with radii 15, 5, 9, 1, 2, 3 (sorted 1 2 3 5 9 15: median 4, 90th
    percentile 12, lambda = 2/3). Head 0's last query block has mean (0.9, 1.2), norm 1.5, so its allowance per
    unit of excess radius is lambda * 1.5 = 1; its centroid scores 0.9 * x_j are, per block,
    -13, -0.85, -5.2, 0, -0.3, +1 and keep_permille 300 keeps two (blocks 5 and 3, cutoff 0).
    alpha = 0 makes blocks 0, 1, 2 (radius > 4) candidates with excess 11, 1, 5:
      U = -13 + 11 = -2 (no), -0.85 + 1 = 0.15 (rescued), -5.2 + 5 = -0.2 (no).
    Every other query block is zero (all scores tie at 0, cutoff 0, allowance 0: nothing is rescued, the centroid
    branch keeps the first k_i blocks). A dropped or squared query norm, the full radius instead of the excess, a
    coefficient of 1 or (p90 - med) / med, the wrong rank for the cutoff, a flipped sign or a missing candidate
    filter each change head 0's last row."""
    radii = [15.0, 5.0, 9.0, 1.0, 2.0, 3.0]
    target = [-13.0, -0.85, -5.2, 0.0, -0.3, 1.0]
    k = _two_axis_keys(radii, [t / 0.9 for t in target])
    q = np.zeros((1, 2, 12, 2))
    q[0, 0, 10:12] = (0.9, 1.2)
    res = M.build_mask(q, k, 1.0, 2, keep_permille=300, alpha=0.0, rescue_mode=1)
    assert (res.med[0, 0], res.p90[0, 0]) == (4.0, 12.0)
    assert abs(res.qnorm[0, 0, 5] - 1.5) < 1e-15
    rows = lambda h: [res.mask[0, h, i].nonzero()[0].tolist() for i in range(6)]
    first = [[0], [0, 1], [0, 2], [0, 1, 3], [0, 1, 4]]
    assert rows(0) == first + [[1, 3, 5]]
    assert rows(1) == first + [[0, 1, 5]]
    # the query-blind rule rescues all three candidates in every row that sees them
    blind = M.build_mask(q, k, 1.0, 2, keep_permille=300, alpha=0.0, rescue_mode=0)
    assert blind.mask[0, 0, 5].nonzero()[0].tolist() == [0, 1, 2, 3, 5]
    # alpha = 0.5 raises tau to 8: block 1 (radius 5) is no longer a candidate
    half = M.build_mask(q, k, 1.0, 2, keep_permille=300, alpha=0.5, rescue_mode=1)
    assert half.mask[0, 0, 5].nonzero()[0].tolist() == [3, 5]


def test_query_aware_rescue_is_strict():
    """Exactly representable case: radii 5 3 3 1 1 1 (median 2, 90th percentile 4, lambda 1/2), query mean (2, 0)
    (allowance 1 per unit of excess), scores 2 * x_j = -1, 1, 1.5, 2, 0, 4, cutoff 2 (blocks 5 and 3). Blocks 0
    and 1 land exactly on the cutoff (U = -1 + 3 = 2, 1 + 1 = 2) and are not rescued; block 2 (U = 2.5) is."""
    k = _two_axis_keys([5.0, 3.0, 3.0, 1.0, 1.0, 1.0], [-0.5, 0.5, 0.75, 1.0, 0.0, 2.0])
    q = np.zeros((1, 1, 12, 2))
    q[0, 0, 10:12] = (2.0, 0.0)
    res = M.build_mask(q, k, 1.0, 2, keep_permille=300, alpha=0.0, rescue_mode=1)
    assert res.lam[0, 0] == 0.5
    assert res.mask[0, 0, 5].nonzero()[0].tolist() == [2, 3, 5]
    assert res.rescue_gap[0, 0, 5] == 0.0


def brute_mask_query_aware(qbar, kbar, rad, scale, keep, alpha, G):
    """Pure-Python statement of the mode-1 rule for tiny sizes."""
    B, Hq, nb, D = qbar.shape
    out = np.zeros((B, Hq, nb, nb), dtype=np.uint8)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            xs = sorted(float(r) for r in rad[b, g])
            med = float(np.quantile(xs, 0.5))
            hi = float(np.quantile(xs, 0.9))
            tau = math.inf if math.isinf(alpha) else med + alpha * (hi - med)
            lam = 0.0 if hi == 0 else (hi - med) / hi
            for i in range(nb):
                qn = math.sqrt(sum(v * v for v in qbar[b, h, i]))
                score = {j: scale * sum(qbar[b, h, i, d] * kbar[b, g, j, d] for d in range(D)) for j in range(i + 1)}
                budget = math.ceil(Fraction((i + 1) * keep, 1000))
                ranked = sorted(range(i + 1), key=lambda j: (-score[j], j))
                cut = score[ranked[budget - 1]] if budget > 0 else math.inf
                for j in range(i + 1):
                    rescued = rad[b, g, j] > tau and score[j] + lam * scale * qn * (rad[b, g, j] - med) > cut
                    if j in ranked[:budget] or rescued or j == i:
                        out[b, h, i, j] = 1
    return out


@pytest.mark.parametrize("keep,alpha", [(100, 1.0), (300, 0.5), (200, 0.0), (0, 0.0), (250, math.inf)])
def test_query_aware_mask_equals_enumeration(keep, alpha):
    b, nb = 4, 10
    q, k = rnd(60, 1, 4, b * nb, 3), rnd(61, 1, 2, b * nb, 3)
    res = M.build_mask(q, k, 0.7, b, keep, alpha, rescue_mode=1)
    qbar, kbar, rad = M.block_stats(q, k, b)
    assert np.isfinite(res.rescue_gap[np.isfinite(res.rescue_gap)]).all()
    np.testing.assert_array_equal(res.mask, brute_mask_query_aware(qbar, kbar, rad, 0.7, keep, alpha, 2))


def test_query_aware_rescue_lies_between_centroid_and_blind():
    b, nb = 8, 24
    q, k = rnd(70, 2, 4, b * nb, 6), rnd(71, 2, 2, b * nb, 6)
    for alpha in (0.0, 0.5, 1.0):
        aware = M.build_mask(q, k, 0.5, b, 150, alpha, rescue_mode=1)
        blind = M.build_mask(q, k, 0.5, b, 150, alpha, rescue_mode=0)
        floor = M.build_mask(q, k, 0.5, b, 150, math.inf, rescue_mode=1)
        assert (aware.mask <= blind.mask).all() and (floor.mask <= aware.mask).all()
        np.testing.assert_array_equal(floor.mask, M.build_mask(q, k, 0.5, b, 150, math.inf).mask)
        assert (aware.rescued <= blind.rescued).all()
        # the coefficient is in [0, 1], so the allowance never exceeds the Cauchy-Schwarz bound
        assert ((aware.lam >= 0) & (aware.lam <= 1)).all()
    # equal radii: nothing is a candidate and the modes agree with the centroid branch
    kk = np.zeros((1, 1, b * nb, 6))
    kk[0, 0, ::b, 0] = 1.0                                         # every block: one key at e0, radius (b-1)/b
    qq = rnd(72, 1, 2, b * nb, 6)
    eq = M.build_mask(qq, kk, 0.5, b, 150, 0.0, rescue_mode=1)
    assert eq.lam[0, 0] == 0.0 and not eq.rescued.any()


def test_query_aware_rescue_keeps_every_planted_block():
    """The planted keys sit in the direction of one query row, so their block's excess radius earns an allowance
    far above the centroid cutoff of the row that holds that query; mode 1 keeps every planted block there while
    rescuing fewer blocks overall than the query-blind rule."""
    inp = W.planted_inputs(3, 1, 8, 2, 64 * 64, 64, block=64, planted_per_mille=100)
    q, k, _ = inp.as_f64()
    aware = M.build_mask(q, k, inp.scale, 64, keep_permille=100, alpha=1.0, rescue_mode=1)
    blind = M.build_mask(q, k, inp.scale, 64, keep_permille=100, alpha=1.0, rescue_mode=0)
    for (b, g, j, u, h, t) in inp.planted:
        assert aware.mask[b, h, t // 64, j] == 1
    assert aware.mask.sum() < blind.mask.sum()


def _radius_quintile_share(inp, block):
    """Share of the top-5% attention blocks whose key block lies in its kv head's top radius quintile. A pair
    (query block i, key block j <= i) is weighed by the exact softmax mass the query rows of block i (all query
    heads of the kv head) put on block j, relative to a uniform spread over the i+1 visible blocks."""
    q, k, _ = inp.as_f64()
    _, Hq, N, D = q.shape
    Hkv = k.shape[1]
    G, nb = Hq // Hkv, N // block
    _, _, rad = M.block_stats(q, k, block)
    rel, top_q = [], []
    for g in range(Hkv):
        mass = np.zeros((nb, nb))
        for h in range(g * G, (g + 1) * G):
            S = inp.scale * (q[0, h] @ k[0, g].T)
            S[np.triu_indices(N, 1)] = -np.inf
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            mass += P.reshape(N, nb, block).sum(axis=2).reshape(nb, block, nb).sum(axis=1)
        top = rad[0, g] >= np.quantile(rad[0, g], 0.8)
        for i in range(1, nb):
            rel.extend(mass[i, :i + 1] * (i + 1) / (G * block))
            top_q.extend(top[:i + 1])
    rel, top_q = np.array(rel), np.array(top_q)
    sel = rel >= np.quantile(rel, 0.95)
    return float(top_q[sel].mean())


def test_radius_quintile_diagnostic_synthetic_analogue():
    """Synthetic analogue of the mean-dilution diagnostic ("Your 128K Context Is 6x Slower Than It Needs to Be",
    section "Why block-sparse attention underperforms": the highest-radius quintile of key blocks held 39.5% of
    the top-5% attention blocks). On the planted workload every one of the top-5% attention blocks is in the top
    radius quintile: a planted key is 6x one query, so it scores ~6 sigma against every query aligned with that
    one and draws attention from many rows. Without the plants the share is chance (one fifth)."""
    planted = _radius_quintile_share(W.planted_inputs(3, 1, 8, 2, 64 * 64, 64, 64), 64)
    plain = _radius_quintile_share(W.dense_inputs(3, 1, 8, 2, 64 * 64, 64, "bf16"), 64)
    assert planted >= 0.9
    assert 0.1 <= plain <= 0.3


# ------------------------------------------------------------------------------------------------- fp8 keys
def test_fp8_key_mask_is_the_mask_of_the_dequantised_keys():
    """Keys that are E4M3 values times a power of two: the fp8-key mask must equal build_mask on those exact keys
    (scale applied once, to the key, not to the radius or the score)."""
    from oracle import attention as A
    rng = np.random.default_rng(80)
    codes = rng.integers(0, 0x7F, size=(1, 2, 64 * 12, 16), dtype=np.uint8)   # finite, non-negative codes
    codes[..., ::2] |= 0x80                                                    # and negative ones
    kscale = 2.0 ** -5
    k = A.e4m3_value(codes) * kscale
    q = rnd(81, 1, 4, 64 * 12, 16)
    for mode in (0, 1):
        a = M.build_mask_fp8_keys(q, codes, kscale, 0.25, 64, 150, 1.0, rescue_mode=mode)
        b = M.build_mask(q, k, 0.25, 64, 150, 1.0, rescue_mode=mode)
        np.testing.assert_array_equal(a.mask, b.mask)
        np.testing.assert_array_equal(a.radius, b.radius)
    # a different scale moves the radii and the scores by the same factor: the quantile-based flags and the
    # centroid ranking are scale-free, so the mask is unchanged while the radii scale
    c = M.build_mask_fp8_keys(q, codes, 4 * kscale, 0.25, 64, 150, 1.0)
    np.testing.assert_array_equal(c.mask, M.build_mask_fp8_keys(q, codes, kscale, 0.25, 64, 150, 1.0).mask)
    np.testing.assert_allclose(c.radius, 4 * b.radius, rtol=1e-15)


def test_e4m3_keys_calibration():
    inp = W.planted_inputs(3, 1, 4, 2, 64 * 8, 32, 64)
    codes, sc = W.e4m3_keys(inp.k)
    from oracle import attention as A
    k = W.f64_from_bf16_bits(inp.k)
    kq = A.e4m3_value(codes) * sc
    assert np.abs(A.e4m3_value(codes)).max() <= 448 and (codes & 0x7F).max() <= 0x7E
    # E4M3 keeps 3 mantissa bits: within 2^-4 relative in the normal range, a subnormal quantum below it
    assert np.all(np.abs(kq - k) <= np.abs(k) * 2.0 ** -4 + sc * 2.0 ** -10)
