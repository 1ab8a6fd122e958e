"""Exact causal attention in float64 (oracle; test infrastructure only).

The tiled, online-softmax method ("attention-kernel-optimization", section "FlashAttention (1 -> 2 -> 3)")
streams Q/K/V tiles on chip and keeps the softmax normalisation exact by rescaling as it goes, so it reaches the
plain softmax-attention result up to rounding order. The oracle is therefore that plain definition, evaluated
row-chunked with a library matmul and a max-subtracted exponential:

    O[b,h,i] = sum_{j<=i} softmax_j(scale * q[b,h,i] . k[b,g(h),j]) v[b,g(h),j]
    lse[b,h,i] = ln sum_{j<=i} exp(scale * q[b,h,i] . k[b,g(h),j])        (natural log)

Causal means square and top-left aligned (query i sees keys 0..i); the pages take causality as the subject and
never spell the alignment out. GQA maps query head h to key/value head g(h) = h // (Hq/Hkv): contiguous groups
("Your 128K Context Is 6x Slower Than It Needs to Be", section "The rescue branch", gives 32 query heads against 4
key-value heads and no order, so the plainest grouping is taken).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _group(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return hq // hkv


def _rows_for_head(rows: Optional[np.ndarray], h: int, n: int) -> np.ndarray:
    if rows is None:
        return np.arange(n, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    return rows[h] if rows.ndim == 2 else rows


def _softmax_rows(s: np.ndarray, allowed: np.ndarray, vv: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax over the allowed entries of each score row, then the weighted sum of value rows.

    Rows with no allowed entry give O = 0 and lse = -inf."""
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.where(allowed, np.exp(s - m_safe), 0.0)
    l = e.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l > 0, (e @ vv) / np.where(l > 0, l, 1.0), 0.0)
        lse = np.where(l[:, 0] > 0, m_safe[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)), -np.inf)
    return o, lse


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     rows: Optional[np.ndarray] = None, max_elems: int = 1 << 24
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Dense causal GQA attention.

    q [B,Hq,N,D], k/v [B,Hkv,N,D] (float64). `rows` optionally restricts the query rows: an int array [R]
    (same rows for every head) or [Hq,R]. Returns O [B,Hq,R,D] and lse [B,Hq,R] in float64."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    G = _group(Hq, Hkv)
    R = N if rows is None else np.asarray(rows).shape[-1]
    out = np.zeros((B, Hq, R, D), dtype=np.float64)
    lse = np.full((B, Hq, R), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            rr = _rows_for_head(rows, h, N)
            for s0 in range(0, len(rr), max(1, max_elems // max(N, 1))):
                sel = rr[s0:s0 + max(1, max_elems // max(N, 1))]
                top = int(sel.max()) + 1
                kk = k[b, g, :top]
                s = scale * (q[b, h, sel] @ kk.T)
                allowed = np.arange(top)[None, :] <= sel[:, None]
                o, l = _softmax_rows(s, allowed, v[b, g, :top])
                out[b, h, s0:s0 + len(sel)] = o
                lse[b, h, s0:s0 + len(sel)] = l
    return out, lse


def masked_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, mask: np.ndarray, block: int,
                     rows: Optional[np.ndarray] = None, max_elems: int = 1 << 24
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """Causal attention restricted to the key blocks a block mask keeps.

    Block-sparse attention groups keys into blocks and attends only to the kept ones ("Your 128K Context Is 6x
    Slower Than It Needs to Be", section "Why block-sparse attention underperforms"), and the combined mask runs
    as ordinary block-sparse tiled attention (same page, section "The rescue branch"). So query row t of query
    block i = t // block attends exactly the keys u <= t whose key block u // block has mask[b,h,i,u//block] = 1.
    mask is [B,Hq,nQB,nKB] (nonzero = kept); q/k/v as in causal_attention."""
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    G = _group(Hq, Hkv)
    if N % block:
        raise ValueError("N must be a multiple of block")
    R = N if rows is None else np.asarray(rows).shape[-1]
    out = np.zeros((B, Hq, R, D), dtype=np.float64)
    lse = np.full((B, Hq, R), -np.inf, dtype=np.float64)
    key_block = np.arange(N) // block
    for b in range(B):
        for h in range(Hq):
            g = h // G
            rr = _rows_for_head(rows, h, N)
            step = max(1, max_elems // max(N, 1))
            for s0 in range(0, len(rr), step):
                sel = rr[s0:s0 + step]
                top = int(sel.max()) + 1
                s = scale * (q[b, h, sel] @ k[b, g, :top].T)
                kept = mask[b, h, sel // block][:, key_block[:top]] != 0
                allowed = kept & (np.arange(top)[None, :] <= sel[:, None])
                o, l = _softmax_rows(s, allowed, v[b, g, :top])
                out[b, h, s0:s0 + len(sel)] = o
                lse[b, h, s0:s0 + len(sel)] = l
    return out, lse


def gather_paged(cache: np.ndarray, block_table: np.ndarray, b: int, length: int) -> np.ndarray:
    """Logical token t of sequence b lives in slot t % page of physical page block_table[b, t // page]
    ("attention-kernel-optimization", section "PagedAttention"). Returns [length, Hkv, D]."""
    page = cache.shape[2]
    t = np.arange(length)
    pid = block_table[b, t // page]
    return cache[pid, :, t % page, :]


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Values of 8-bit E4M3 codes as float64, per the OCP 8-bit floating point specification (OFP8): sign bit,
    4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals M/8 * 2^-6; there are no
    infinities and S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448. The pages ask for an
    fp8 KV cache ("Your Context Length Decides What a Kernel Is Worth": the --kv-cache-dtype fp8 setting cuts the
    bytes decode has to read) without naming the encoding; E4M3 is read as that encoding."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def paged_decode_fp8(q: np.ndarray, k_codes: np.ndarray, v_codes_t: np.ndarray, k_scale: float, v_scale: float,
                     block_table: np.ndarray, seq_lens: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Single-token decode over an fp8 paged cache: the keys and values are the E4M3 code values times one
    scale per tensor, and the attention is then paged_decode's.

    k_codes [num_pages, Hkv, page, D] (token-major, as the bf16 cache); v_codes_t [num_pages, Hkv, D, page]: the
    value cache holds each page transposed, the page's tokens contiguous for every head dimension. Only the
    tokens a sequence reaches are dequantised, so codes past its end (NaN included) play no part."""
    B, Hq, D = q.shape
    Hkv = k_codes.shape[1]
    page = k_codes.shape[2]
    G = _group(Hq, Hkv)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        t = np.arange(L)
        pid, slot = block_table[b, t // page], t % page
        K = e4m3_value(k_codes[pid, :, slot, :]) * float(k_scale)      # [L, Hkv, D]
        V = e4m3_value(v_codes_t[pid, :, :, slot]) * float(v_scale)    # [L, Hkv, D]
        for h in range(Hq):
            g = h // G
            s = scale * (K[:, g, :] @ q[b, h])
            o, l = _softmax_rows(s[None, :], np.ones((1, L), dtype=bool), V[:, g, :])
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Single-token decode over a paged cache, unsplit.

    The query of sequence b is the token at position L_b - 1 and attends all L_b cached tokens (its own K/V are
    already in the cache). q [B,Hq,D]; caches [num_pages,Hkv,page,D] (float64); returns O [B,Hq,D] and
    lse [B,Hq]. L_b = 0 gives O = 0 and lse = -inf."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K = gather_paged(k_cache, block_table, b, L)
        V = gather_paged(v_cache, block_table, b, L)
        for h in range(Hq):
            g = h // G
            s = scale * (K[:, g, :] @ q[b, h])
            o, l = _softmax_rows(s[None, :], np.ones((1, L), dtype=bool), V[:, g, :])
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def paged_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                  seq_lens: np.ndarray, scale: float, window: int = 0,
                  rows: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Chunked prefill over a paged cache: sequence b holds L_b = seq_lens[b] cached tokens, the last Nq of which
    are the chunk whose queries q[b, :, r] (r < Nq) sit at positions P_b + r, P_b = L_b - Nq (their own K/V are
    already in the cache). Query position p sees key t when t <= p and, with a sliding window W > 0, when
    t > p - W (its W latest keys, itself included; "Your Context Length Decides What a Kernel Is Worth" names
    sliding-window attention on half of a model's layers; "attention-kernel-optimization", section
    "PagedAttention", gives the paged layout). q [B,Hq,Nq,D]; caches [num_pages,Hkv,page,D] float64.
    Returns O [B,Hq,R,D] and natural-log lse [B,Hq,R] for the chunk rows `rows` (all Nq when None)."""
    B, Hq, Nq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    rr = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, Hq, len(rr), D), dtype=np.float64)
    lse = np.full((B, Hq, len(rr)), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L < Nq:
            raise ValueError("every sequence must hold at least the chunk's tokens")
        K = gather_paged(k_cache, block_table, b, L)
        V = gather_paged(v_cache, block_table, b, L)
        pos = (L - Nq) + rr
        t = np.arange(L)
        allowed = t[None, :] <= pos[:, None]
        if window > 0:
            allowed &= t[None, :] > pos[:, None] - window
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, h, rr] @ K[:, g, :].T)
            out[b, h], lse[b, h] = _softmax_rows(s, allowed, V[:, g, :])
    return out, lse


def split_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, scale: float, chunk: int) -> Tuple[np.ndarray, np.ndarray]:
    """The split-KV form: each sequence's keys are cut into chunks of `chunk` tokens and every chunk is attended
    on its own ("attention-kernel-optimization", section "Inference-specific: Flash-Decoding and FlashInfer").
    Returns per-chunk normalised outputs o [B,Hq,C,D] and their log-sum-exps lse [B,Hq,C] (-inf for chunks past
    the sequence), C = ceil(max L / chunk)."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = _group(Hq, Hkv)
    C = max(1, -(-int(np.max(seq_lens)) // chunk)) if len(seq_lens) else 1
    o = np.zeros((B, Hq, C, D), dtype=np.float64)
    lse = np.full((B, Hq, C), -np.inf, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K = gather_paged(k_cache, block_table, b, L)
        V = gather_paged(v_cache, block_table, b, L)
        for c in range(-(-L // chunk)):
            lo, hi = c * chunk, min(L, (c + 1) * chunk)
            for h in range(Hq):
                g = h // G
                s = scale * (K[lo:hi, g, :] @ q[b, h])
                oc, lc = _softmax_rows(s[None, :], np.ones((1, hi - lo), dtype=bool), V[lo:hi, g, :])
                o[b, h, c] = oc[0]
                lse[b, h, c] = lc[0]
    return o, lse


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The reduce after the split: with M = max_c lse_c and w_c = exp(lse_c - M), the full output is
    sum_c w_c o_c / sum_c w_c and the full lse is M + ln sum_c w_c. Chunks with lse = -inf carry no weight; if
    every chunk is empty the output is 0 and lse is -inf. o_parts [...,C,D], lse_parts [...,C]."""
    M = lse_parts.max(axis=-1, keepdims=True)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms), 0.0)
    sw = w.sum(axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(sw > 0, (w[..., None] * o_parts).sum(axis=-2) / np.where(sw > 0, sw, 1.0), 0.0)
        lse = np.where(sw[..., 0] > 0, Ms[..., 0] + np.log(np.where(sw[..., 0] > 0, sw[..., 0], 1.0)), -np.inf)
    return o, lse
