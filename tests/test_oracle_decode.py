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


# ------------------------------------------------------------------------------------------------- fp8 KV cache
def test_e4m3_values_follow_the_format_definition():
    """Anchors from the OFP8 E4M3 definition (bias 7, 3 mantissa bits, subnormals, NaN only at S.1111.111) and the
    whole code table against PyTorch's float8_e4m3fn, an independent implementation of the same format."""
    import torch
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
               0x40: 2.0, 0xC0: -2.0, 0x7E: 448.0, 0xFE: -448.0, 0x77: 240.0, 0x80: 0.0}
    for c, v in anchors.items():
        assert A.e4m3_value(np.array([c]))[0] == v, hex(c)
    assert np.isnan(A.e4m3_value(np.array([0x7F, 0xFF]))).all()
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    mine = A.e4m3_value(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_e4m3_encoder_rounds_to_nearest_even_and_saturates():
    """The generator's encoder against PyTorch's float8_e4m3fn conversion (round to nearest even) on random
    values over the whole range, exact midpoints and the subnormal range; beyond 448 it saturates."""
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 64, rng.standard_normal(5000) * 2.0 ** -7,
                        (np.arange(-40, 40) + 0.5) * 2.0 ** -9, np.array([1.0625, 1.1875, 17.0, 19.0, 0.0]),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    mine = W.e4m3_codes_from_f32(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)
    assert W.e4m3_codes_from_f32(np.array([1000.0, -500.0], np.float32)).tolist() == [0x7E, 0xFE]


def test_fp8_decode_is_decode_over_the_dequantised_cache():
    """Every E4M3 value times a power-of-two scale is a bf16 number, so decoding the fp8 cache must equal the bf16
    oracle decoding a cache that holds those numbers (with V transposed back to token-major)."""
    d = W.decode_inputs_fp8(7, 4, 8, 2, 16, 16, 1, 200, k_scale=2.0 ** -5, v_scale=2.0 ** -7,
                            seq_lens=np.array([1, 16, 33, 200], np.int32))
    q = W.f64_from_bf16_bits(d.q)
    O8, L8 = A.paged_decode_fp8(q, d.k_cache, d.v_cache_t, d.k_scale, d.v_scale, d.block_table, d.seq_lens, d.scale)
    kf = np.nan_to_num(A.e4m3_value(d.k_cache)) * d.k_scale
    vf = np.nan_to_num(A.e4m3_value(d.v_cache_t.transpose(0, 1, 3, 2))) * d.v_scale
    O, L = A.paged_decode(q, kf, vf, d.block_table, d.seq_lens, d.scale)
    assert np.isfinite(O8).all()
    np.testing.assert_array_equal(O8, O)
    np.testing.assert_array_equal(L8, L)


def test_fp8_needle_reads_the_transposed_value_page():
    """One sequence of 20 tokens over two pages, head_dim 4. Keys are zero except token 17, whose key makes its
    score 448 * 2 * scale larger than every other; the output is then token 17's value row, which sits in page
    table[1], slot 1, spread over the page's head-dim rows: V^T[page][g][d][1]. Codes: 0x38 = 1, 0x40 = 2,
    0x48 = 4, 0x30 = 0.5. With v_scale 2 the value row is (2, 4, 8, 1)."""
    D, page, Hkv = 4, 16, 1
    bt = np.array([[3, 0]], np.int32)
    kc = np.zeros((4, Hkv, page, D), np.uint8)
    vt = np.full((4, Hkv, D, page), 0x38, np.uint8)     # every other value 1.0
    kc[0, 0, 1, :] = 0x7E                                # token 17 = page bt[0,1] = 0, slot 1: key 448 * (1,1,1,1)
    vt[0, 0, :, 1] = [0x38, 0x40, 0x48, 0x30]
    kc[0, 0, 4:, :] = 0x7F                               # NaN past the end (tokens 20..31)
    vt[0, 0, :, 4:] = 0x7F
    q = np.full((1, 1, D), 1.0)
    O, L = A.paged_decode_fp8(q, kc, vt, 1.0, 2.0, bt, np.array([20], np.int32), 1.0)
    np.testing.assert_allclose(O[0, 0], [2.0, 4.0, 8.0, 1.0], atol=1e-300)
    assert abs(L[0, 0] - 4 * 448.0) < 1e-9
