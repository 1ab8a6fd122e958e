"""Pins for oracle.attention.causal_attention and masked_attention.

Each check comes from outside the oracle's own code: a pure-Python brute force (math.exp, explicit loops),
closed forms of softmax attention, textbook reductions (GQA with repeated K/V is multi-head attention) and a
library routine (torch's scaled-dot-product attention on CPU in float64)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A


def brute_attention(q, k, v, scale, allowed):
    """Pure Python: allowed(b, h, i, j) -> bool. Returns O and natural-log lse as nested lists."""
    B, Hq, N, D = q.shape
    G = Hq // k.shape[1]
    O = np.zeros((B, Hq, N, D))
    L = np.full((B, Hq, N), -math.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(N):
                js = [j for j in range(N) if allowed(b, h, i, j)]
                if not js:
                    continue
                sc = [scale * sum(float(q[b, h, i, d]) * float(k[b, g, j, d]) for d in range(D)) for j in js]
                m = max(sc)
                w = [math.exp(s - m) for s in sc]
                tot = sum(w)
                for d in range(D):
                    O[b, h, i, d] = sum(wj * float(v[b, g, j, d]) for wj, j in zip(w, js)) / tot
                L[b, h, i] = m + math.log(tot)
    return O, L


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("N", [1, 2, 7, 13])
def test_dense_equals_brute_force(N):
    q, k, v = rnd(1, 2, 4, N, 5), rnd(2, 2, 2, N, 5), rnd(3, 2, 2, N, 5)
    scale = 0.37
    O, L = A.causal_attention(q, k, v, scale)
    Ob, Lb = brute_attention(q, k, v, scale, lambda b, h, i, j: j <= i)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_closed_form_three_keys():
    # one query row 2 sees keys 0..2 with scores ln1, ln2, ln3 -> weights 1/6, 2/6, 3/6 and lse = ln 6
    D = 2
    q = np.zeros((1, 1, 3, D)); q[0, 0, 2] = [1.0, 0.0]
    k = np.zeros((1, 1, 3, D)); k[0, 0, :, 0] = [math.log(1), math.log(2), math.log(3)]
    v = np.zeros((1, 1, 3, D)); v[0, 0, :, 1] = [6.0, 12.0, 18.0]
    O, L = A.causal_attention(q, k, v, 1.0)
    assert abs(O[0, 0, 2, 1] - (6 * 1 + 12 * 2 + 18 * 3) / 6.0) < 1e-12
    assert abs(L[0, 0, 2] - math.log(6.0)) < 1e-12
    # row 1 sees keys 0, 1 with q = 0 -> equal weights
    assert abs(O[0, 0, 1, 1] - 9.0) < 1e-12 and abs(L[0, 0, 1] - math.log(2.0)) < 1e-12


def test_uniform_values_return_the_value_and_weights_sum_to_one():
    q, k = rnd(4, 1, 4, 33, 8), rnd(5, 1, 2, 33, 8)
    vrow = rnd(6, 8)
    v = np.broadcast_to(vrow, (1, 2, 33, 8)).copy()
    O, _ = A.causal_attention(q, k, v, 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(vrow, O.shape), atol=1e-13)
    ones = np.ones((1, 2, 33, 1))
    O1, _ = A.causal_attention(q, k, ones, 0.5)
    np.testing.assert_allclose(O1, 1.0, atol=1e-13)


def test_row_zero_and_single_token():
    q, k, v = rnd(7, 1, 2, 9, 4), rnd(8, 1, 1, 9, 4), rnd(9, 1, 1, 9, 4)
    O, L = A.causal_attention(q, k, v, 1.3)
    for h in range(2):
        np.testing.assert_array_equal(O[0, h, 0], v[0, 0, 0])
        assert abs(L[0, h, 0] - 1.3 * float(q[0, h, 0] @ k[0, 0, 0])) < 1e-13
    O1, _ = A.causal_attention(q[:, :, :1], k[:, :, :1], v[:, :, :1], 1.3)
    np.testing.assert_array_equal(O1[0, :, 0], np.broadcast_to(v[0, 0, 0], (2, 4)))


def test_zero_query_gives_prefix_means():
    N = 17
    q = np.zeros((1, 2, N, 3))
    k, v = rnd(10, 1, 1, N, 3), rnd(11, 1, 1, N, 3)
    O, L = A.causal_attention(q, k, v, 0.9)
    pref = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    for h in range(2):
        np.testing.assert_allclose(O[0, h], pref, atol=1e-13)
        np.testing.assert_allclose(L[0, h], np.log(np.arange(1, N + 1)), atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = rnd(12, 2, 8, 20, 6), rnd(13, 2, 2, 20, 6), rnd(14, 2, 2, 20, 6)
    O, L = A.causal_attention(q, k, v, 0.4)
    Om, Lm = A.causal_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.4)
    np.testing.assert_allclose(O, Om, atol=1e-13)
    np.testing.assert_allclose(L, Lm, atol=1e-13)
    # and a head-map slip (h % Hkv instead of h // G) would differ
    Ow, _ = A.causal_attention(q, np.tile(k, (1, 4, 1, 1)), np.tile(v, (1, 4, 1, 1)), 0.4)
    assert np.abs(Ow - O).max() > 1e-3


def test_matches_torch_sdpa_cpu_float64():
    q, k, v = rnd(15, 1, 3, 50, 16), rnd(16, 1, 3, 50, 16), rnd(17, 1, 3, 50, 16)
    O, _ = A.causal_attention(q, k, v, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.25).numpy()
    np.testing.assert_allclose(O, ref, atol=1e-12)


def test_row_subset_equals_full():
    q, k, v = rnd(18, 1, 4, 70, 8), rnd(19, 1, 2, 70, 8), rnd(20, 1, 2, 70, 8)
    O, L = A.causal_attention(q, k, v, 0.3)
    rows = np.array([[0, 5, 69], [1, 2, 3], [10, 40, 68], [0, 1, 69]])
    Os, Ls = A.causal_attention(q, k, v, 0.3, rows=rows, max_elems=100)
    for h in range(4):
        np.testing.assert_allclose(Os[0, h], O[0, h, rows[h]], atol=1e-14)
        np.testing.assert_allclose(Ls[0, h], L[0, h, rows[h]], atol=1e-14)


# ---------------------------------------------------------------------------------------------- masked attention
def test_all_ones_mask_equals_dense():
    q, k, v = rnd(21, 1, 4, 64, 8), rnd(22, 1, 2, 64, 8), rnd(23, 1, 2, 64, 8)
    mask = np.ones((1, 4, 8, 8), dtype=np.uint8)
    O, L = A.masked_attention(q, k, v, 0.3, mask, 8)
    Od, Ld = A.causal_attention(q, k, v, 0.3)
    np.testing.assert_allclose(O, Od, atol=1e-14)
    np.testing.assert_allclose(L, Ld, atol=1e-14)


def test_diagonal_mask_equals_blockwise_dense():
    b = 8
    q, k, v = rnd(24, 1, 2, 48, 4), rnd(25, 1, 1, 48, 4), rnd(26, 1, 1, 48, 4)
    mask = np.zeros((1, 2, 6, 6), dtype=np.uint8)
    for i in range(6):
        mask[0, :, i, i] = 1
    O, L = A.masked_attention(q, k, v, 0.7, mask, b)
    for i in range(6):
        sl = slice(i * b, (i + 1) * b)
        Od, Ld = A.causal_attention(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.7)
        np.testing.assert_allclose(O[:, :, sl], Od, atol=1e-14)
        np.testing.assert_allclose(L[:, :, sl], Ld, atol=1e-14)


def test_random_mask_equals_brute_force():
    b, nb = 4, 5
    N = b * nb
    q, k, v = rnd(27, 1, 4, N, 3), rnd(28, 1, 2, N, 3), rnd(29, 1, 2, N, 3)
    rng = np.random.default_rng(30)
    mask = (rng.random((1, 4, nb, nb)) < 0.5).astype(np.uint8)
    for i in range(nb):
        mask[0, :, i, i] = 1
    O, L = A.masked_attention(q, k, v, 0.6, mask, b)
    Ob, Lb = brute_attention(q, k, v, 0.6, lambda bb, h, i, j: j <= i and mask[bb, h, i // b, j // b] == 1)
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    np.testing.assert_allclose(L, Lb, atol=1e-12)
