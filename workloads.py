"""Seeded synthetic inputs for the long-context causal attention workloads.

This module is shared by the CPU oracle tests and by the HIP-path tests and benchmark. It holds none of the
attention arithmetic: only random draws (numpy PCG64, one spawned stream per purpose), round-to-nearest-even
conversion of the drawn fp32 values to bf16 bit patterns, and index bookkeeping (planted outlier positions,
the paged KV layout and block table, sampled query rows).

Workload shapes follow the pages:
  * 32 query heads sharing 4 key/value heads with head_dim 128 and a 128K context, the model shape in
    "Your 128K Context Is 6x Slower Than It Needs to Be" (section "The rescue branch: two selection paths,
    one mask"), and the 32K / 128K pair that page measures (sections "The rescue branch" and "What to do
    today").
  * A paged KV cache of fixed-size pages that need not be contiguous, walked through a block table
    ("attention-kernel-optimization", section "PagedAttention (the vLLM revolution)"), for q_len = 1 decode
    (same page, section "Inference-specific: Flash-Decoding and FlashInfer").
The pages measure on real prompts and checkpoints that are not available here; these generators stand in for
them with i.i.d. N(0,1) activations of the same shapes, plus one planted high-attention key per chosen block to
reproduce the mean-dilution geometry described in "Your 128K Context Is 6x Slower Than It Needs to Be",
section "Why block-sparse attention underperforms: the mean-dilution trap".
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


# --------------------------------------------------------------------------------------------------------------
# bit-level helpers (input preparation only)
# --------------------------------------------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns the uint16 bit patterns.

    Inputs are assumed finite (the generators only produce finite values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_from_bf16_bits(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    return f32_from_bf16_bits(u).astype(np.float64)


def e4m3_codes_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to 8-bit E4M3 codes (OCP OFP8: bias 7, 3 mantissa bits, subnormals below 2^-6, largest
    finite 448) with round-to-nearest-even, saturating at +-448; returns uint8 codes. Inputs are assumed finite.

    Normal range: the fp32 pattern is rounded to its top 3 mantissa bits in integer arithmetic (a carry moves into
    the exponent) and the exponent is rebased from 127 to 7. Below 2^-6 the code is the magnitude in units of
    2^-9, rounded half to even."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    u = a.view(np.uint32)
    code = (u >> np.uint32(20)) & np.uint32(1)
    code += u
    code += np.uint32(0x7FFFF)
    code >>= np.uint32(20)
    code -= np.uint32(120 << 3)                                  # wraps below 2^-6; replaced next
    small = a < np.float32(2.0 ** -6)
    if small.any():
        code[small] = np.rint(a[small] * np.float32(512.0)).astype(np.uint32)   # exact scaling, ties to even
    code |= (x.view(np.uint32) >> np.uint32(24)) & np.uint32(0x80)   # the sign bit
    return code.astype(np.uint8)


def e4m3_keys(k_bits: np.ndarray) -> Tuple[np.ndarray, float]:
    """Per-tensor E4M3 codes of bf16 keys: the scale maps the largest |key| onto 448 (computed in fp32), and each
    code is the E4M3 rounding of key / scale. Returns (codes uint8 like k_bits, scale)."""
    k32 = f32_from_bf16_bits(k_bits)
    scale = float(np.float32(np.abs(k32).max()) / np.float32(448.0))
    if scale == 0.0:
        scale = 1.0
    return e4m3_codes_from_f32(k32 / np.float32(scale)), scale


def streams(seed: int, names: List[str]) -> Dict[str, np.random.Generator]:
    """Independent PCG64 generators, one per purpose, spawned from one SeedSequence."""
    children = np.random.SeedSequence(seed).spawn(len(names))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(names, children)}


def _normal_bf16(rng: np.random.Generator, shape: Tuple[int, ...], chunk_elems: int = 1 << 26) -> np.ndarray:
    """i.i.d. N(0,1) fp32 draws rounded to bf16 bits, generated in chunks to bound host memory."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    for s in range(0, total, chunk_elems):
        e = min(total, s + chunk_elems)
        out[s:e] = bf16_bits_from_f32(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


# --------------------------------------------------------------------------------------------------------------
# prefill inputs
# --------------------------------------------------------------------------------------------------------------
@dataclass
class PrefillInputs:
    """Q [B,Hq,N,D], K/V [B,Hkv,N,D]; bf16 bit patterns (uint16) or fp32 values, D contiguous."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str                      # "bf16" | "fp32"
    scale: float
    block: Optional[int] = None     # q-block == k-block size for the block-sparse path
    # planted outliers: tuples (b, kv_head, key_block, slot, q_head, q_row)
    planted: List[Tuple[int, int, int, int, int, int]] = field(default_factory=list)

    @property
    def shape(self) -> Tuple[int, int, int, int, int]:
        B, Hq, N, D = self.q.shape
        return B, Hq, self.k.shape[1], N, D

    def as_f64(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Exact widening of the very values the GPU receives."""
        if self.dtype == "bf16":
            return f64_from_bf16_bits(self.q), f64_from_bf16_bits(self.k), f64_from_bf16_bits(self.v)
        return self.q.astype(np.float64), self.k.astype(np.float64), self.v.astype(np.float64)


def dense_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, D: int, dtype: str = "bf16",
                 scale: Optional[float] = None) -> PrefillInputs:
    """i.i.d. N(0,1) Q/K/V. bf16 inputs are fp32 draws rounded to nearest even."""
    r = streams(seed, ["q", "k", "v", "planted", "rows"])
    sc = float(1.0 / np.sqrt(D)) if scale is None else float(scale)
    if dtype == "fp32":
        q = r["q"].standard_normal((B, Hq, N, D), dtype=np.float32)
        k = r["k"].standard_normal((B, Hkv, N, D), dtype=np.float32)
        v = r["v"].standard_normal((B, Hkv, N, D), dtype=np.float32)
    elif dtype == "bf16":
        q = _normal_bf16(r["q"], (B, Hq, N, D))
        k = _normal_bf16(r["k"], (B, Hkv, N, D))
        v = _normal_bf16(r["v"], (B, Hkv, N, D))
    else:
        raise ValueError(dtype)
    return PrefillInputs(q=q, k=k, v=v, dtype=dtype, scale=sc)


def planted_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, D: int, block: int,
                   planted_per_mille: int = 50) -> PrefillInputs:
    """Dense bf16 inputs plus planted high-attention keys (plant_outliers)."""
    if N % block:
        raise ValueError("N must be a multiple of block")
    inp = dense_inputs(seed, B, Hq, Hkv, N, D, "bf16")
    plant_outliers(inp, seed, block, planted_per_mille)
    return inp


def plant_outliers(inp: PrefillInputs, seed: int, block: int, planted_per_mille: int = 50) -> PrefillInputs:
    """Overwrite keys of bf16 inputs in place with planted high-attention keys, for blocks of `block` rows.

    Per (batch, kv-head g): choose nKB*planted_per_mille//1000 key blocks j without replacement from
    [0, nKB-2]. For each: a slot u in [0, block), a later query block i in [j+1, nQB-1], a query row t in block i
    and a query head h of g's group are drawn, and key row j*block+u of kv-head g is overwritten with
    bf16(6.0 * q[b, h, t]). The key then scores far above its neighbours for that query while the block's mean
    barely moves, which is the geometry the mean-dilution section describes. The draws come from the seed's own
    "planted" stream, so the same seed and block give the same plants whatever was drawn before."""
    B, Hq, N, D = inp.q.shape
    Hkv = inp.k.shape[1]
    if N % block:
        raise ValueError("N must be a multiple of block")
    inp.block = block
    inp.planted = []
    rng = streams(seed, ["q", "k", "v", "planted", "rows"])["planted"]
    nb = N // block
    G = Hq // Hkv
    count = nb * planted_per_mille // 1000
    for b in range(B):
        for g in range(Hkv):
            js = rng.choice(nb - 1, size=count, replace=False)
            for j in sorted(int(x) for x in js):
                u = int(rng.integers(0, block))
                i = int(rng.integers(j + 1, nb))
                t = int(rng.integers(i * block, (i + 1) * block))
                h = g * G + int(rng.integers(0, G))
                qv = f32_from_bf16_bits(inp.q[b, h, t])
                inp.k[b, g, j * block + u] = bf16_bits_from_f32(np.float32(6.0) * qv)
                inp.planted.append((b, g, j, u, h, t))
    return inp


# --------------------------------------------------------------------------------------------------------------
# decode inputs
# --------------------------------------------------------------------------------------------------------------
@dataclass
class DecodeInputs:
    """q [B,Hq,D]; k_cache/v_cache [num_pages,Hkv,page,D] (bf16 bits); block_table [B,max_pages] int32 (-1 pad);
    seq_lens [B] int32. Slots at or past seq_lens[b] in a sequence's last page hold NaN bit patterns."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    page: int
    scale: float

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        B, Hq, D = self.q.shape
        return B, Hq, self.k_cache.shape[1], D


def decode_inputs(seed: int, B: int, Hq: int, Hkv: int, D: int, page: int, len_lo: int, len_hi: int,
                  poison_tail: bool = True, seq_lens: Optional[np.ndarray] = None) -> DecodeInputs:
    """Paged KV cache with per-sequence lengths uniform on [len_lo, len_hi] (both ends inclusive).

    Physical pages number exactly sum(ceil(L_b / page)); they are handed out from one seeded permutation in
    sequence order, so logical page p of sequence b lives at block_table[b, p]. Entries past a sequence's last
    page are -1 and are never meant to be read."""
    r = streams(seed, ["q", "k", "v", "lens", "perm", "rows"])
    if seq_lens is None:
        lens = r["lens"].integers(len_lo, len_hi, size=B, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, dtype=np.int32)
    pages_per = (lens.astype(np.int64) + page - 1) // page
    num_pages = int(pages_per.sum())
    max_pages = max(1, -(-int(len_hi) // page))
    perm = r["perm"].permutation(num_pages).astype(np.int32)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    kc = _normal_bf16(r["k"], (max(num_pages, 1), Hkv, page, D))
    vc = _normal_bf16(r["v"], (max(num_pages, 1), Hkv, page, D))
    if poison_tail:
        for b in range(B):
            L = int(lens[b])
            if L % page:
                pid = bt[b, L // page]
                kc[pid, :, L % page:, :] = BF16_NAN_BITS
                vc[pid, :, L % page:, :] = BF16_NAN_BITS
    q = _normal_bf16(r["q"], (B, Hq, D))
    return DecodeInputs(q=q, k_cache=kc, v_cache=vc, block_table=bt, seq_lens=lens, page=page,
                        scale=float(1.0 / np.sqrt(D)))


@dataclass
class DecodeInputsFP8:
    """q [B,Hq,D] bf16 bits; k_cache [num_pages,Hkv,page,D] and v_cache_t [num_pages,Hkv,D,page] E4M3 codes
    (uint8; the value cache holds each page transposed); one scale per cache; block_table, seq_lens as in
    DecodeInputs. Slots at or past seq_lens[b] in a sequence's last page hold the NaN code 0x7F."""
    q: np.ndarray
    k_cache: np.ndarray
    v_cache_t: np.ndarray
    k_scale: float
    v_scale: float
    block_table: np.ndarray
    seq_lens: np.ndarray
    page: int
    scale: float


E4M3_NAN_CODE = np.uint8(0x7F)


def _normal_e4m3(rng: np.random.Generator, shape: Tuple[int, ...], inv_scale: float,
                 chunk_elems: int = 1 << 26) -> np.ndarray:
    """i.i.d. N(0,1) fp32 draws (the same draws as _normal_bf16 on the same stream) times inv_scale, rounded to
    E4M3 codes."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint8)
    for s in range(0, total, chunk_elems):
        e = min(total, s + chunk_elems)
        out[s:e] = e4m3_codes_from_f32(rng.standard_normal(e - s, dtype=np.float32) * np.float32(inv_scale))
    return out.reshape(shape)


def decode_inputs_fp8(seed: int, B: int, Hq: int, Hkv: int, D: int, page: int, len_lo: int, len_hi: int,
                      k_scale: float = 2.0 ** -6, v_scale: float = 2.0 ** -6, poison_tail: bool = True,
                      seq_lens: Optional[np.ndarray] = None) -> DecodeInputsFP8:
    """The paged decode workload of decode_inputs (same lengths, page permutation, block table and activation
    draws) with K and V stored as E4M3 codes of value / scale, one scale per cache. The default scale 2^-6 maps
    the N(0,1) activations onto the format's range (7 sigma saturates at 448) and is exact to apply. The value
    cache is written transposed within each page: [page id, kv head, head dim, slot]."""
    r = streams(seed, ["q", "k", "v", "lens", "perm", "rows"])
    if seq_lens is None:
        lens = r["lens"].integers(len_lo, len_hi, size=B, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, dtype=np.int32)
    pages_per = (lens.astype(np.int64) + page - 1) // page
    num_pages = int(pages_per.sum())
    max_pages = max(1, -(-int(len_hi) // page))
    perm = r["perm"].permutation(num_pages).astype(np.int32)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    P = max(num_pages, 1)
    kc = _normal_e4m3(r["k"], (P, Hkv, page, D), 1.0 / k_scale)
    vc = _normal_e4m3(r["v"], (P, Hkv, page, D), 1.0 / v_scale)
    if poison_tail:
        for b in range(B):
            L = int(lens[b])
            if L % page:
                pid = bt[b, L // page]
                kc[pid, :, L % page:, :] = E4M3_NAN_CODE
                vc[pid, :, L % page:, :] = E4M3_NAN_CODE
    vt = np.ascontiguousarray(vc.transpose(0, 1, 3, 2))
    q = _normal_bf16(r["q"], (B, Hq, D))
    return DecodeInputsFP8(q=q, k_cache=kc, v_cache_t=vt, k_scale=float(k_scale), v_scale=float(v_scale),
                           block_table=bt, seq_lens=lens, page=page, scale=float(1.0 / np.sqrt(D)))


@dataclass
class PagedPrefillInputs:
    """A chunk of Nq new tokens per sequence over a paged bf16 cache that already holds them: q [B,Hq,Nq,D]
    (bf16 bits), the cache, block table and lengths of DecodeInputs (seq_lens[b] >= Nq), and a sliding window
    (0 = none)."""
    q: np.ndarray
    cache: DecodeInputs
    window: int

    @property
    def scale(self) -> float:
        return self.cache.scale


def paged_prefill_inputs(seed: int, B: int, Hq: int, Hkv: int, D: int, Nq: int, page: int, len_lo: int,
                         len_hi: int, window: int = 0, seq_lens: Optional[np.ndarray] = None) -> PagedPrefillInputs:
    """The paged cache of decode_inputs (lengths uniform on [len_lo, len_hi], len_lo >= Nq, NaN past each end)
    plus Nq query rows per sequence and head from a stream of their own."""
    if len_lo < Nq and seq_lens is None:
        raise ValueError("every sequence must hold the chunk: len_lo >= Nq")
    cache = decode_inputs(seed, B, Hq, Hkv, D, page, len_lo, len_hi, seq_lens=seq_lens)
    rq = streams(seed, ["q", "k", "v", "lens", "perm", "rows", "chunk_q"])["chunk_q"]
    q = _normal_bf16(rq, (B, Hq, Nq, D))
    return PagedPrefillInputs(q=q, cache=cache, window=int(window))


# --------------------------------------------------------------------------------------------------------------
# sampled query rows for large configurations
# --------------------------------------------------------------------------------------------------------------
def sample_rows(seed: int, N: int, Hq: int, per_head: int, block: Optional[int] = None,
                planted: Optional[List[Tuple[int, int, int, int, int, int]]] = None) -> np.ndarray:
    """Sorted query-row indices per head, int64 [Hq, R] (same R for every head).

    Every head's sample holds row 0, row N-1, the first and last row of a middle block (or of the middle 64
    rows) and, for planted inputs, the planted query rows of that head; the rest is drawn without
    replacement."""
    rng = streams(seed, ["q", "k", "v", "planted", "rows"])["rows"]
    b = block or 64
    mid = (N // b // 2) * b
    fixed = {0, N - 1, min(mid, N - 1), min(mid + b - 1, N - 1)}
    per_head_fixed = [set(fixed) for _ in range(Hq)]
    if planted:
        for (_, _, _, _, h, t) in planted:
            per_head_fixed[h].add(int(t))
    R = max(per_head, max(len(s) for s in per_head_fixed))
    R = min(R, N)
    out = np.empty((Hq, R), dtype=np.int64)
    for h in range(Hq):
        base = sorted(per_head_fixed[h])[:R]
        need = R - len(base)
        pool = np.setdiff1d(np.arange(N, dtype=np.int64), np.asarray(base, dtype=np.int64), assume_unique=True) \
            if N <= (1 << 22) else None
        if need > 0:
            if pool is not None:
                extra = rng.choice(pool, size=need, replace=False)
            else:
                extra = set()
                while len(extra) < need:
                    for x in rng.integers(0, N, size=need * 2):
                        if int(x) not in per_head_fixed[h] and len(extra) < need:
                            extra.add(int(x))
                extra = np.fromiter(extra, dtype=np.int64)
            rows = np.concatenate([np.asarray(base, dtype=np.int64), np.asarray(extra, dtype=np.int64)])
        else:
            rows = np.asarray(base, dtype=np.int64)
        out[h] = np.sort(rows)
    return out


# --------------------------------------------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------------------------------------------
WORKLOADS = {
    "c1_dense_fp32_n256": dict(kind="dense", seed=1, B=1, Hq=1, Hkv=1, N=256, D=64, dtype="fp32"),
    "c2_dense_bf16_n4k": dict(kind="dense", seed=2, B=1, Hq=32, Hkv=4, N=4096, D=128, dtype="bf16"),
    # dense causal GQA prefill at 32K on plain N(0,1) inputs: the rescue page's model shape at the shorter of the
    # two context lengths it compares
    "dense_bf16_n32k": dict(kind="dense", seed=32, B=1, Hq=32, Hkv=4, N=32768, D=128, dtype="bf16"),
    "c3_sparse_bf16_n32k": dict(kind="sparse", seed=3, B=1, Hq=32, Hkv=4, N=32768, D=128, block=64,
                                keep_permille=100, alpha=1.0, q_lo_pct=50, q_hi_pct=90),
    "c4_sparse_bf16_n128k": dict(kind="sparse", seed=4, B=1, Hq=32, Hkv=4, N=131072, D=128, block=128,
                                 keep_permille=50, alpha=1.0, q_lo_pct=50, q_hi_pct=90),
    "c5_decode_paged_bf16": dict(kind="decode", seed=5, B=32, Hq=64, Hkv=8, D=64, page=16, len_lo=1024,
                                 len_hi=32768, chunk=512),
    # chunked prefill: the last 4096 tokens of a 32768-token sequence in a paged cache, the model shape above
    "c6_paged_prefill_chunk": dict(kind="paged_prefill", seed=6, B=1, Hq=32, Hkv=4, D=128, Nq=4096, page=16,
                                   len_lo=32768, len_hi=32768, window=0),
    # sliding-window chunked prefill, the grouped-query, windowed layer shape (64 query heads, 8 kv heads,
    # head_dim 64, window 128) over 8 sequences of 8K-16K tokens, 2048 new tokens each
    "c7_paged_prefill_window": dict(kind="paged_prefill", seed=7, B=8, Hq=64, Hkv=8, D=64, Nq=2048, page=16,
                                    len_lo=8192, len_hi=16384, window=128),
    # the same decode workload over an E4M3 KV cache (per-tensor scales 2^-6)
    "c5_decode_paged_fp8": dict(kind="decode_fp8", seed=5, B=32, Hq=64, Hkv=8, D=64, page=16, len_lo=1024,
                                len_hi=32768, chunk=512, k_scale=2.0 ** -6, v_scale=2.0 ** -6),
}


def make(name: str):
    """Generate the named workload's inputs."""
    w = WORKLOADS[name]
    if w["kind"] == "dense":
        return dense_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["dtype"])
    if w["kind"] == "sparse":
        return planted_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["block"])
    if w["kind"] == "decode":
        return decode_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["D"], w["page"], w["len_lo"], w["len_hi"])
    if w["kind"] == "paged_prefill":
        return paged_prefill_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["D"], w["Nq"], w["page"], w["len_lo"],
                                    w["len_hi"], w["window"])
    if w["kind"] == "decode_fp8":
        return decode_inputs_fp8(w["seed"], w["B"], w["Hq"], w["Hkv"], w["D"], w["page"], w["len_lo"], w["len_hi"],
                                 w["k_scale"], w["v_scale"])
    raise KeyError(name)
