"""The block-selection pre-pass in float64 (oracle; test infrastructure only).

Source: "Your 128K Context Is 6x Slower Than It Needs to Be", sections "Why block-sparse attention
underperforms: the mean-dilution trap" and "The rescue branch: two selection paths, one mask". The page gives
the method in outline; the steps below are its order, with the open points fixed as follows:

 1. Queries and keys are cut into blocks of `block` rows. A key block's centroid is the mean of its keys; the
    query side of the centroid score is the mean of the query block's rows, taken per query head. (By linearity
    the mean query's score against a key centroid equals the mean of the block's token-to-centroid scores, so
    the two readings of the query side agree.)
 2. A key block's radius is the largest Euclidean distance from one of its keys to the block centroid.
 3. Per (batch, kv-head), over all key blocks: the median and the 90th percentile of the radii, as type-7
    linear-interpolated quantiles (numpy's default method) at integer percentages, evaluated with exact integer
    index arithmetic; then the rescue threshold tau = med + alpha * (p90 - med).
 4. Rescue branch: key block j is flagged when r_j > tau (strict), for every query head of the kv-head's group
    (rescue_mode 0; the query-aware form, rescue_mode 1, follows below).
 5. Centroid branch: for query block i of head h, the candidates are the causally visible key blocks j <= i;
    their score is scale * <mean q-block, key centroid>; the k_i = ceil((i+1) * keep_permille / 1000) best are
    kept (integer ceiling), ties broken towards the smaller j.
 6. Each branch applies its own threshold, the two results are OR-ed, and the diagonal block is always kept:
    M[h,i,j] = 1 iff j <= i and (centroid-kept or rescued or j == i).
 7. The kept list of each (h, i) row, ascending in j, is the CSR form the sparse kernel walks.

Step 4 has two forms. rescue_mode 0 is the query-blind test above: every flagged block is rescued for every row
that can see it. rescue_mode 1 reads the section's last step -- the radius distribution yields a coefficient,
and the rescue candidates are then scored against the base path with it -- as follows:
 4a. coefficient lambda = (p90 - med) / p90 per (batch, kv-head), the spread of the radii between the two
     reference points relative to the upper one (0 when p90 is 0); it lies in [0, 1];
 4b. the candidates of row (h, i) are the blocks j <= i flagged by the radius test of step 4;
 4c. a candidate's rescue score is its centroid score plus lambda times the Cauchy-Schwarz allowance of the
     part of its radius above the median, U_ij = S_ij + lambda * scale * |qbar_i| * (r_j - med): with lambda = 1
     and med = 0 this is the upper bound of <qbar_i, key> * scale over the block's keys;
 4d. the candidate is rescued for that row when U_ij > the base branch's cutoff in the same row (the k_i-th
     largest centroid score; no cutoff, so no rescue, when k_i = 0).
 Mode 1 therefore rescues a subset of what mode 0 rescues, row by row, and a query block whose mean is far from
 a wide block's outlier direction no longer pays for it.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Tuple

import numpy as np


def block_stats(q: np.ndarray, k: np.ndarray, block: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Step 1-2: q-block means [B,Hq,nQB,D], key-block centroids [B,Hkv,nKB,D], radii [B,Hkv,nKB] (float64).

    q [B,Hq,N,D], k [B,Hkv,N,D] float64 (the widened bf16 inputs)."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if N % block:
        raise ValueError("N must be a multiple of block")
    nb = N // block
    qbar = np.empty((B, Hq, nb, D), dtype=np.float64)
    kbar = np.empty((B, Hkv, nb, D), dtype=np.float64)
    rad = np.empty((B, Hkv, nb), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            qbar[b, h] = q[b, h].reshape(nb, block, D).mean(axis=1)
        for g in range(Hkv):
            kb = k[b, g].reshape(nb, block, D)
            c = kb.mean(axis=1)
            kbar[b, g] = c
            dist = np.sqrt(((kb - c[:, None, :]) ** 2).sum(axis=2))
            rad[b, g] = dist.max(axis=1)
    return qbar, kbar, rad


def quantile_type7(sorted_x: np.ndarray, pct: int) -> float:
    """Linear-interpolation quantile of ascending data at integer percentage pct in [0, 100]:
    position (n-1)*pct/100, split exactly into an integer index lo and fraction f = ((n-1)*pct mod 100)/100,
    value x[lo] + f * (x[lo+1] - x[lo])."""
    n = len(sorted_x)
    if n == 0:
        raise ValueError("empty")
    num = (n - 1) * int(pct)
    lo = num // 100
    f = (num % 100) / 100.0
    if lo + 1 >= n or f == 0.0:
        return float(sorted_x[lo])
    return float(sorted_x[lo] + f * (sorted_x[lo + 1] - sorted_x[lo]))


def rescue_threshold(radii: np.ndarray, alpha: float, lo_pct: int = 50, hi_pct: int = 90
                     ) -> Tuple[float, float, float]:
    """Step 3 for one (batch, kv-head): (med, p90, tau) with tau = med + alpha * (p90 - med).
    alpha = +inf disables the rescue branch (tau = +inf)."""
    xs = np.sort(np.asarray(radii, dtype=np.float64))
    med = quantile_type7(xs, lo_pct)
    hi = quantile_type7(xs, hi_pct)
    tau = np.inf if np.isinf(alpha) else med + alpha * (hi - med)
    return med, hi, float(tau)


def rescue_coefficient(med: float, hi: float) -> float:
    """Step 4a: lambda = (p90 - med) / p90, and 0 when p90 is 0 (then at least the upper tenth of the radii are
    zero, every block above the median is a single point, and no allowance is owed)."""
    return 0.0 if hi == 0.0 else (hi - med) / hi


def centroid_budget(i: int, keep_permille: int) -> int:
    """k_i = ceil((i+1) * keep_permille / 1000) in integer arithmetic."""
    return ((i + 1) * int(keep_permille) + 999) // 1000


@dataclass
class MaskResult:
    mask: np.ndarray         # uint8 [B,Hq,nQB,nKB]
    kv_count: np.ndarray     # int32 [B,Hq,nQB]
    kv_index: np.ndarray     # int32 [B,Hq,nQB,nKB]; entries past kv_count are -1
    radius: np.ndarray       # float64 [B,Hkv,nKB]
    med: np.ndarray          # float64 [B,Hkv]
    p90: np.ndarray          # float64 [B,Hkv]
    tau: np.ndarray          # float64 [B,Hkv]
    rescue: np.ndarray       # bool [B,Hkv,nKB]
    centroid: np.ndarray     # bool [B,Hq,nQB,nKB]: the centroid branch alone (before the OR)
    cut_gap: np.ndarray      # float64 [B,Hq,nQB]: score of the last kept minus the best dropped (inf if none)
    score_absmax: np.ndarray  # float64 [B,Hq,nQB]: max |score| over the row's candidates
    rescued: np.ndarray      # bool [B,Hq,nQB,nKB]: the rescue branch alone, per row (mode 0: rescue broadcast)
    lam: np.ndarray          # float64 [B,Hkv]: step 4a coefficient (computed in both modes)
    qnorm: np.ndarray        # float64 [B,Hq,nQB]: |qbar_i|
    rescue_gap: np.ndarray   # float64 [B,Hq,nQB]: mode 1, min over deciding candidates of |U - cut| relative to
                             # 1 + |S| + |allowance| + |cut| (inf if none, and always inf in mode 0)


def build_mask(q: np.ndarray, k: np.ndarray, scale: float, block: int, keep_permille: int, alpha: float,
               lo_pct: int = 50, hi_pct: int = 90, rescue_mode: int = 0) -> MaskResult:
    """Steps 1-7 on float64 inputs q [B,Hq,N,D], k [B,Hkv,N,D]; rescue_mode 0 or 1 selects step 4's form."""
    if rescue_mode not in (0, 1):
        raise ValueError("rescue_mode must be 0 or 1")
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    G = Hq // Hkv
    nb = N // block
    qbar, kbar, rad = block_stats(q, k, block)
    med = np.empty((B, Hkv))
    p90 = np.empty((B, Hkv))
    tau = np.empty((B, Hkv))
    for b in range(B):
        for g in range(Hkv):
            med[b, g], p90[b, g], tau[b, g] = rescue_threshold(rad[b, g], alpha, lo_pct, hi_pct)
    rescue = rad > tau[:, :, None]
    lam = np.array([[rescue_coefficient(med[b, g], p90[b, g]) for g in range(Hkv)] for b in range(B)])
    qnorm = np.sqrt((qbar * qbar).sum(axis=3))
    mask = np.zeros((B, Hq, nb, nb), dtype=np.uint8)
    cen = np.zeros((B, Hq, nb, nb), dtype=bool)
    resc = np.zeros((B, Hq, nb, nb), dtype=bool)
    gap = np.full((B, Hq, nb), np.inf)
    rgap = np.full((B, Hq, nb), np.inf)
    amax = np.zeros((B, Hq, nb))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            S = scale * (qbar[b, h] @ kbar[b, g].T)       # [nQB, nKB]
            for i in range(nb):
                j = np.arange(i + 1)
                s = S[i, :i + 1]
                amax[b, h, i] = np.abs(s).max()
                kk = min(centroid_budget(i, keep_permille), i + 1)
                order = np.lexsort((j, -s))                # score descending, then smaller j
                kept = order[:kk]
                cen[b, h, i, kept] = True
                if 0 < kk < i + 1:
                    gap[b, h, i] = s[order[kk - 1]] - s[order[kk]]
                cand = rescue[b, g, :i + 1]
                if rescue_mode == 0:
                    r_row = cand.copy()
                else:
                    cut = s[order[kk - 1]] if kk > 0 else np.inf
                    coef = lam[b, g] * scale * qnorm[b, h, i]
                    allow = coef * (rad[b, g, :i + 1] - med[b, g])
                    u = s + allow
                    r_row = cand & (u > cut)
                    # decisions that can change the mask: candidates outside the centroid pick, off the diagonal
                    deciding = cand & ~cen[b, h, i, :i + 1] & (j != i)
                    if np.isfinite(cut) and deciding.any():
                        rel = np.abs(u - cut) / (1.0 + np.abs(s) + np.abs(allow) + abs(cut))
                        rgap[b, h, i] = rel[deciding].min()
                resc[b, h, i, :i + 1] = r_row
                row = cen[b, h, i, :i + 1] | r_row
                row[i] = True
                mask[b, h, i, :i + 1] = row
    kv_count = mask.sum(axis=3, dtype=np.int64).astype(np.int32)
    kv_index = np.full((B, Hq, nb, nb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hq):
            for i in range(nb):
                idx = np.nonzero(mask[b, h, i])[0]
                kv_index[b, h, i, :len(idx)] = idx
    return MaskResult(mask=mask, kv_count=kv_count, kv_index=kv_index, radius=rad, med=med, p90=p90, tau=tau,
                      rescue=rescue, centroid=cen, cut_gap=gap, score_absmax=amax, rescued=resc, lam=lam,
                      qnorm=qnorm, rescue_gap=rgap)


def build_mask_fp8_keys(q: np.ndarray, k_codes: np.ndarray, k_scale: float, scale: float, block: int,
                        keep_permille: int, alpha: float, lo_pct: int = 50, hi_pct: int = 90,
                        rescue_mode: int = 0) -> MaskResult:
    """build_mask with the keys given as 8-bit E4M3 codes and one scale per tensor: every key is its code's value
    times k_scale, in float64, and the rule is then applied unchanged ("Your 128K Context Is 6x Slower Than It
    Needs to Be", section "The numbers, stated honestly", reports the rescue signal holding with FP8 keys)."""
    from oracle.attention import e4m3_value
    k = e4m3_value(k_codes) * float(k_scale)
    return build_mask(q, k, scale, block, keep_permille, alpha, lo_pct, hi_pct, rescue_mode)
