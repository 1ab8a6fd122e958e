"""Entry-by-entry check of a block mask against the oracle's, with the documented fp64 tie band.

The library and the oracle both compute the block-selection rule in float64, but in different summation orders, so
a decision that sits within rounding of its threshold may legitimately go either way. This module decides, for every
mask entry, whether it is fixed by the rule whatever the rounding ("must be 1", "must be 0") or falls in the tie
band ("free"), and checks a candidate mask against that:

  - j > i                                              must be 0 (causal)
  - j == i                                             must be 1 (diagonal)
  - centroid score above the row's cut by more than the band    must be 1
  - rescued, with the decision clear of its threshold           must be 1
  - centroid score inside the band around the cut      free (centroid)
  - rescue decision inside its band                    free (rescue)
  - anything else                                      must be 0

The band around the cut is 1e-12 * (1 + max |score| of the row); a radius is in the band when it lies within
1e-12 relative of tau; a query-aware rescue score when it lies within 1e-12 relative (to 1 + |S| + |allowance| +
|cut|) of the cut. A near-tau radius therefore frees only its own column's rescue decisions, not whole rows.

Each row keeps exactly k_i centroid picks, so the free centroid entries of a row hold exactly k_i - |picks clear of
the band| picks. Picks that are also set for another reason (diagonal, clear rescue) cannot be seen in the mask, so
the check is the bound that follows: the count of set free-centroid entries lies in
[k_i - |clear picks| - |band entries set for another reason|, k_i - |clear picks| + |band entries that are also
free rescue decisions|].

The library's kv_count and kv_index must also be the CSR form of its own mask on every row (count = row sum,
indices = the set columns in ascending order).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import block_mask as M


@dataclass
class EntryStatus:
    must1: np.ndarray       # bool [B,Hq,nb,nb]
    must0: np.ndarray       # bool [B,Hq,nb,nb]
    free_cen: np.ndarray    # bool [B,Hq,nb,nb]: centroid decision inside the band
    free_res: np.ndarray    # bool [B,Hq,nb,nb]: rescue decision inside the band
    lo: np.ndarray          # int [B,Hq,nb]: bounds on the set free-centroid entries (see the module text)
    hi: np.ndarray          # int [B,Hq,nb]

    @property
    def free(self) -> np.ndarray:
        return (self.free_cen | self.free_res) & ~self.must1


def entry_status(ref: M.MaskResult, qbar: np.ndarray, kbar: np.ndarray, scale: float, keep_permille: int,
                 rescue_mode: int) -> EntryStatus:
    """Classify every entry of the oracle's mask. qbar/kbar are the oracle's block means for the same inputs."""
    B, Hq, nb, _ = ref.mask.shape
    Hkv = ref.radius.shape[1]
    G = Hq // Hkv
    must1 = np.zeros(ref.mask.shape, bool)
    must0 = np.zeros(ref.mask.shape, bool)
    free_cen = np.zeros(ref.mask.shape, bool)
    free_res = np.zeros(ref.mask.shape, bool)
    lo = np.zeros((B, Hq, nb), np.int64)
    hi = np.zeros((B, Hq, nb), np.int64)
    tau = ref.tau
    near_tau = np.isfinite(tau)[:, :, None] & (np.abs(ref.radius - tau[:, :, None])
                                              <= 1e-12 * np.abs(tau)[:, :, None])
    flag_clear = ref.rescue & ~near_tau
    for b in range(B):
        for h in range(Hq):
            g = h // G
            S = scale * (qbar[b, h] @ kbar[b, g].T)
            for i in range(nb):
                n = i + 1
                s = S[i, :n]
                j = np.arange(n)
                k = min(M.centroid_budget(i, keep_permille), n)
                eps = 1e-12 * (1.0 + np.abs(s).max())
                order = np.lexsort((j, -s))
                if k == 0:
                    clear_pick = np.zeros(n, bool)
                    band = np.zeros(n, bool)
                    cut = np.inf
                elif k == n:
                    clear_pick = np.ones(n, bool)
                    band = np.zeros(n, bool)
                    cut = s[order[k - 1]]
                else:
                    c1, c2 = s[order[k - 1]], s[order[k]]
                    cut = c1
                    if c1 - c2 >= eps:
                        clear_pick = s >= c1
                        band = np.zeros(n, bool)
                    else:
                        clear_pick = s > c1 + eps
                        band = (s >= c2 - eps) & ~clear_pick
                # rescue decisions of this row
                if rescue_mode == 0:
                    res_clear = flag_clear[b, g, :n].copy()
                    fr = near_tau[b, g, :n].copy()
                else:
                    allow = ref.lam[b, g] * scale * ref.qnorm[b, h, i] * (ref.radius[b, g, :n] - ref.med[b, g])
                    u = s + allow
                    if np.isfinite(cut):
                        rel = np.abs(u - cut) / (1.0 + np.abs(s) + np.abs(allow) + abs(cut))
                        near_u = rel <= 1e-12
                        # the cut itself may be any score of the band when the row has one
                        if band.any():
                            near_u |= (u >= s[band].min() - eps) & (u <= s[band].max() + eps)
                    else:
                        near_u = np.zeros(n, bool)
                    # a flag in the band matters only where the score test could pass
                    res_clear = flag_clear[b, g, :n] & (u > cut) & ~near_u
                    fr = (near_tau[b, g, :n] & ((u > cut) | near_u)) | (ref.rescue[b, g, :n] & near_u)
                m1 = clear_pick | res_clear
                m1[i] = True
                fc = band & ~m1
                fr &= ~m1
                must1[b, h, i, :n] = m1
                must0[b, h, i, :n] = ~m1 & ~fc & ~fr
                must0[b, h, i, n:] = True
                free_cen[b, h, i, :n] = fc
                free_res[b, h, i, :n] = fr
                picks_free = k - int(clear_pick.sum())
                lo[b, h, i] = picks_free - int((band & m1).sum())
                hi[b, h, i] = picks_free + int((fc & fr).sum())
    return EntryStatus(must1, must0, free_cen, free_res, lo, hi)


def check_mask(mask: np.ndarray, kv_count: np.ndarray, kv_index: np.ndarray, st: EntryStatus,
               max_free: int = 0) -> dict:
    """Assert that (mask, kv_count, kv_index) is a valid answer under `st`; returns counts for the log. Raises
    AssertionError naming the first offending (b, h, i)."""
    m = mask.astype(bool)
    bad1 = st.must1 & ~m
    bad0 = st.must0 & m
    for name, bad in (("a must-be-1 entry is 0", bad1), ("a must-be-0 entry is 1", bad0)):
        if bad.any():
            b, h, i, j = (int(x) for x in np.argwhere(bad)[0])
            raise AssertionError(f"{name} at (b={b}, h={h}, i={i}, j={j}); {int(bad.sum())} such entries")
    setc = (m & st.free_cen).sum(axis=-1)
    rows_with_band = st.free_cen.any(axis=-1)
    viol = rows_with_band & ((setc < st.lo) | (setc > st.hi))
    if viol.any():
        b, h, i = (int(x) for x in np.argwhere(viol)[0])
        raise AssertionError(f"row (b={b}, h={h}, i={i}) sets {int(setc[b, h, i])} of its tie-band centroid "
                             f"entries, outside [{int(st.lo[b, h, i])}, {int(st.hi[b, h, i])}]")
    # CSR of the library's own mask, on every row
    rowsum = m.sum(axis=-1)
    if not np.array_equal(kv_count, rowsum):
        b, h, i = (int(x) for x in np.argwhere(kv_count != rowsum)[0])
        raise AssertionError(f"kv_count {int(kv_count[b, h, i])} != mask row sum {int(rowsum[b, h, i])} at "
                             f"(b={b}, h={h}, i={i})")
    nb = m.shape[-1]
    cols = np.broadcast_to(np.arange(nb), m.shape)
    # ascending set columns of each row, padded with nb, against the first kv_count entries of kv_index
    want = np.sort(np.where(m, cols, nb), axis=-1)
    valid = cols < kv_count[..., None]
    if not np.array_equal(np.where(valid, kv_index, nb), np.where(valid, want, nb)):
        b, h, i = (int(x) for x in np.argwhere((np.where(valid, kv_index, nb) != np.where(valid, want, nb))
                                               .any(axis=-1))[0])
        raise AssertionError(f"kv_index is not the ascending list of the mask's set blocks at (b={b}, h={h}, i={i})")
    nfree = int(st.free.sum())
    if nfree > max_free:
        raise AssertionError(f"{nfree} mask entries fall in the fp64 tie band (allowed {max_free})")
    return {"free_entries": nfree, "free_rows": int(st.free.any(axis=-1).sum())}
