"""The tie-band mask checker used by the GPU mask tests, pinned on constructed inputs (no GPU).

Two constructions put decisions exactly on their thresholds, where two correct float64 evaluations in different
orders may disagree:
  - every key block has the same centroid, so every centroid score of a row ties and any k_i of the row's
    candidates is a valid centroid pick;
  - radii with a repeated median and alpha = 0, so two blocks' radii equal tau exactly and their (strict) rescue
    flags may go either way.
The checker must accept the oracle's answer and the other valid answers there, and reject answers that break a
rule outside the band.
"""
import numpy as np
import pytest

from oracle import block_mask as M
from tests import mask_check as C


def tied_centroids(nb=10, block=64, D=64, seed=3):
    """Key block j = c + (-1)^row * d_j: every block's centroid is exactly c."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, nb * block, D))
    c = np.round(rng.standard_normal(D) * 4) / 4
    k = np.empty((1, 1, nb * block, D))
    sign = np.where(np.arange(block) % 2 == 0, 1.0, -1.0)[:, None]
    for j in range(nb):
        d = np.round(rng.standard_normal(D) * 4) / 4
        k[0, 0, j * block:(j + 1) * block] = c + sign * d
    return q, k


def radii_at_tau(block=64, D=64, seed=4):
    """Ten key blocks with radii 1,2,3,4,5,5,7,8,9,10 (distance from c_j along e_0), distinct centroids."""
    rng = np.random.default_rng(seed)
    radii = [1.0, 2.0, 3.0, 4.0, 5.0, 5.0, 7.0, 8.0, 9.0, 10.0]
    nb = len(radii)
    q = rng.standard_normal((1, 2, nb * block, D))
    k = np.empty((1, 1, nb * block, D))
    sign = np.where(np.arange(block) % 2 == 0, 1.0, -1.0)
    for j, r in enumerate(radii):
        cj = np.round(rng.standard_normal(D) * 4) / 4
        kb = np.tile(cj, (block, 1))
        kb[:, 0] += sign * r
        k[0, 0, j * block:(j + 1) * block] = kb
    return q, k


def status(q, k, scale, block, keep, alpha, mode):
    ref = M.build_mask(q, k, scale, block, keep, alpha, rescue_mode=mode)
    qbar, kbar, _ = M.block_stats(q, k, block)
    return ref, C.entry_status(ref, qbar, kbar, scale, keep, mode)


def csr(mask):
    cnt = mask.sum(axis=-1).astype(np.int32)
    nb = mask.shape[-1]
    idx = np.full(mask.shape, -1, np.int32)
    for pos in np.ndindex(mask.shape[:-1]):
        nz = np.nonzero(mask[pos])[0]
        idx[pos][:len(nz)] = nz
    return cnt, idx


def check(mask, st, max_free):
    cnt, idx = csr(mask)
    return C.check_mask(mask, cnt, idx, st, max_free=max_free)


def test_oracle_mask_passes_with_no_free_entries_on_random_inputs():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 64 * 12, 64))
    k = rng.standard_normal((1, 2, 64 * 12, 64))
    for mode in (0, 1):
        ref, st = status(q, k, 0.125, 64, 250, 1.0, mode)
        assert int(st.free.sum()) == 0
        check(ref.mask, st, 0)


def test_exact_centroid_ties_accept_any_valid_pick():
    q, k = tied_centroids()
    ref, st = status(q, k, 0.125, 64, 300, np.inf, 0)
    nb = ref.mask.shape[-1]
    # every candidate of a row with 0 < k_i < i + 1 lies in the band
    assert st.free_cen.any()
    with pytest.raises(AssertionError, match="tie band"):
        check(ref.mask, st, 0)            # free entries exist, and the count is asserted
    check(ref.mask, st, st.free.sum())
    # the other valid answer: the k_i LARGEST candidate indices instead of the smallest
    alt = np.zeros_like(ref.mask)
    for h in range(2):
        for i in range(nb):
            kk = M.centroid_budget(i, 300)
            alt[0, h, i, i + 1 - kk:i + 1] = 1
            alt[0, h, i, i] = 1
    assert not np.array_equal(alt, ref.mask)
    check(alt, st, st.free.sum())
    # the diagonal may itself be one of the k_i picks, so a tied row may set k_i or k_i - 1 of its other
    # candidates: both pass, k_i + 1 and k_i - 2 do not
    i = 7
    kk = M.centroid_budget(i, 300)
    ok_max = alt.copy()
    ok_max[0, 0, i, 0] = 1
    assert ok_max[0, 0, i, :i].sum() == kk
    check(ok_max, st, st.free.sum())
    too_many = ok_max.copy()
    too_many[0, 0, i, 1] = 1
    with pytest.raises(AssertionError, match="tie-band centroid"):
        check(too_many, st, st.free.sum())
    ok_min = ref.mask.copy()
    off = np.nonzero(ok_min[0, 1, i, :i])[0]
    assert len(off) == kk
    ok_min[0, 1, i, off[0]] = 0
    check(ok_min, st, st.free.sum())
    too_few = ok_min.copy()
    too_few[0, 1, i, off[1]] = 0
    with pytest.raises(AssertionError, match="tie-band centroid"):
        check(too_few, st, st.free.sum())


def test_radius_exactly_at_tau_frees_only_its_column():
    q, k = radii_at_tau()
    ref, st = status(q, k, 0.125, 64, 0, 0.0, 0)   # no centroid budget: rescue and diagonal only
    assert ref.med[0, 0] == 5.0 and ref.tau[0, 0] == 5.0
    # blocks 4 and 5 sit exactly on tau: not flagged by the oracle (strict), free for the library
    assert not ref.rescue[0, 0, 4] and not ref.rescue[0, 0, 5] and ref.rescue[0, 0, 6]
    assert st.free_res[0, :, 6:, 4].all() and st.free_res[0, :, 6:, 5].all()
    assert not st.free_res[0, :, :, [0, 1, 2, 3, 6, 7, 8, 9]].any()
    # flagging them is a valid answer too
    alt = ref.mask.copy()
    alt[0, :, 5:, 4] = 1
    alt[0, :, 6:, 5] = 1
    check(alt, st, st.free.sum())
    # a clearly flagged block dropped from a row fails
    bad = ref.mask.copy()
    bad[0, 0, 8, 7] = 0
    with pytest.raises(AssertionError, match="must-be-1"):
        check(bad, st, st.free.sum())
    # a clearly unflagged block set fails
    bad = ref.mask.copy()
    bad[0, 1, 8, 2] = 1
    with pytest.raises(AssertionError, match="must-be-0"):
        check(bad, st, st.free.sum())


def test_query_aware_band_uses_the_same_columns():
    q, k = radii_at_tau()
    ref, st = status(q, k, 0.125, 64, 200, 0.0, 1)
    # mode 1 rescues a subset of mode 0, and nothing clearly unflagged is free
    assert not (st.free_res[0, :, :, [0, 1, 2, 3]]).any()
    check(ref.mask, st, st.free.sum())


def test_csr_consistency_is_checked():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 64 * 8, 64))
    k = rng.standard_normal((1, 1, 64 * 8, 64))
    ref, st = status(q, k, 0.125, 64, 300, 1.0, 0)
    cnt, idx = csr(ref.mask)
    cnt_bad = cnt.copy()
    cnt_bad[0, 1, 5] += 1
    with pytest.raises(AssertionError, match="kv_count"):
        C.check_mask(ref.mask, cnt_bad, idx, st)
    idx_bad = idx.copy()
    row = idx_bad[0, 0, 7]
    c = cnt[0, 0, 7]
    assert c >= 2
    row[0], row[1] = row[1], row[0]   # not ascending
    with pytest.raises(AssertionError, match="kv_index"):
        C.check_mask(ref.mask, cnt, idx_bad, st)
    C.check_mask(ref.mask, cnt, idx, st)
