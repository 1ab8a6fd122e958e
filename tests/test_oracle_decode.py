"""Pins for oracle.attention.paged_decode, split_decode and lse_combine."""
import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_decode(seed=5, B=5, Hq=8, Hkv=2, D=16, page=16, lo=1, hi=300, lens=None):
    d = W.decode_inputs(seed, B, Hq, Hkv, D, page, lo, hi, seq_lens=lens)
    q = W.f64_from_bf16_bits(d.q)
    kc = W.f64_from_bf16_bits(d.k_cache)
    vc = W.f64_from_bf16_bits(d.v_cache)
    return d, q, kc, vc


@pytest.mark.parametrize("chunk", [16, 48, 512, 1 << 20])
def test_split_then_combine_equals_unsplit(chunk):
    d, q, kc, vc = small_decode(lens=np.array([1, 15, 16, 17, 300], dtype=np.int32))
    O, L = A.paged_decode(q, kc, vc, d.block_table, d.seq_lens, d.scale)
    op, lp = A.split_decode(q, kc, vc, d.block_table, d.seq_lens, d.scale, chunk)
    Oc, Lc = A.lse_combine(op, lp)
    np.testing.assert_allclose(Oc, O, atol=1e-12)
    np.testing.assert_allclose(Lc, L, atol=1e-12)


def test_decode_equals_dense_prefill_last_row():
    """Cross-variant pin: decoding at length L is row L-1 of causal prefill over the same tokens."""
    d, q, kc, vc = small_decode(seed=9, B=3, lens=np.array([37, 64, 129], dtype=np.int32))
    O, L = A.paged_decode(q, kc, vc, d.block_table, d.seq_lens, d.scale)
    for b in range(3):
        n = int(d.seq_lens[b])
        K = A.gather_paged(kc, d.block_table, b, n).transpose(1, 0, 2)[None]     # [1,Hkv,n,D]
        V = A.gather_paged(vc, d.block_table, b, n).transpose(1, 0, 2)[None]
        Qp = np.zeros((1, q.shape[1], n, q.shape[2]))
        Qp[0, :, n - 1] = q[b]
        Od, Ld = A.causal_attention(Qp, K, V, d.scale, rows=np.array([n - 1]))
        np.testing.assert_allclose(O[b], Od[0, :, 0], atol=1e-12)
        np.testing.assert_allclose(L[b], Ld[0, :, 0], atol=1e-12)


def test_gather_follows_the_block_table_not_memory_order():
    d, q, kc, vc = small_decode(seed=11, B=2, lens=np.array([40, 70], dtype=np.int32))
    # build the contiguous cache by hand and an identity block table over it
    for b in range(2):
        n = int(d.seq_lens[b])
        pages = -(-n // 16)
        contig = np.stack([kc[d.block_table[b, p]] for p in range(pages)])   # [pages,Hkv,16,D]
        ident = np.arange(pages, dtype=np.int32)[None]
        g1 = A.gather_paged(contig, ident, 0, n)
        g2 = A.gather_paged(kc, d.block_table, b, n)
        np.testing.assert_array_equal(g1, g2)
        # token t of the gather is slot t % 16 of page t // 16, spelled out element by element
        for t in (0, 15, 16, n - 1):
            np.testing.assert_array_equal(g2[t], kc[d.block_table[b, t // 16], :, t % 16, :])


def test_needle_returns_the_needle_value():
    B, Hq, Hkv, D = 1, 4, 1, 8
    n = 100
    d, q, kc, vc = small_decode(seed=13, B=B, Hq=Hq, Hkv=Hkv, D=D, lens=np.array([n], dtype=np.int32))
    kc[:] = 0.0
    tstar = 77
    pid = d.block_table[0, tstar // 16]
    qq = np.zeros_like(q)
    qq[0, :, 0] = 1.0
    kc[pid, 0, tstar % 16, 0] = 200.0 / d.scale        # score gap 200 against every other key
    O, L = A.paged_decode(qq, kc, vc, d.block_table, d.seq_lens, d.scale)
    want = vc[pid, 0, tstar % 16]
    bound = (n - 1) * math.exp(-200.0) * np.nanmax(np.abs(vc)) * 2
    assert np.abs(O[0] - want).max() <= bound
    assert abs(L[0, 0] - 200.0) < 1e-9


def test_zero_length_and_nan_tails():
    d, q, kc, vc = small_decode(seed=17, B=3, lens=np.array([0, 5, 33], dtype=np.int32))
    O, L = A.paged_decode(q, kc, vc, d.block_table, d.seq_lens, d.scale)
    assert (O[0] == 0).all() and np.isneginf(L[0]).all()
    assert np.isfinite(O[1:]).all() and np.isfinite(L[1:]).all()
    assert np.isnan(kc).any()        # the poisoned tails exist and are never gathered
    o, l = A.lse_combine(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert (o == 0).all() and np.isneginf(l).all()


def test_decode_intensity_matches_the_page():
    """The page on context length puts decode attention at an arithmetic intensity of about 8 flop/byte; for
    grouped-query attention with a 16-bit KV cache that is the group size, which the decode workload has."""
    gold = json.load(open(os.path.join(GOLDEN, "decode_intensity.json")))
    w = W.WORKLOADS["c5_decode_paged_bf16"]
    G = w["Hq"] // w["Hkv"]
    flops_per_token = 4 * w["D"] * w["Hq"]                 # q.k and p.v for every query head
    bytes_per_token = 2 * 2 * w["D"] * w["Hkv"]            # one K and one V row per kv head, 2 bytes each
    ai = flops_per_token / bytes_per_token
    assert ai == G
    assert abs(ai - gold["arithmetic_intensity_flop_per_byte"]) <= gold["tolerance"]
