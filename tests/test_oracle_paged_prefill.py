"""Pins for oracle.attention.paged_prefill (chunked prefill over a paged cache, optional sliding window)."""
import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as A


def f64(p: W.PagedPrefillInputs):
    c = p.cache
    return (W.f64_from_bf16_bits(p.q), W.f64_from_bf16_bits(c.k_cache), W.f64_from_bf16_bits(c.v_cache),
            c.block_table, c.seq_lens)


def test_whole_sequence_chunk_is_causal_attention():
    """Nq = L (no prefix) and no window: dense causal attention over the gathered contiguous keys."""
    p = W.paged_prefill_inputs(1, 2, 8, 2, 16, 50, 16, 50, 50)
    q, kc, vc, bt, L = f64(p)
    O, lse = A.paged_prefill(q, kc, vc, bt, L, p.scale)
    for b in range(2):
        K = A.gather_paged(kc, bt, b, 50).transpose(1, 0, 2)[None]
        V = A.gather_paged(vc, bt, b, 50).transpose(1, 0, 2)[None]
        Or, Lr = A.causal_attention(q[b:b + 1], K, V, p.scale)
        np.testing.assert_allclose(O[b], Or[0], atol=1e-12)
        np.testing.assert_allclose(lse[b], Lr[0], atol=1e-12)


def test_one_token_chunk_is_decode():
    p = W.paged_prefill_inputs(2, 4, 8, 2, 16, 1, 16, 1, 300, seq_lens=np.array([1, 16, 17, 300]))
    q, kc, vc, bt, L = f64(p)
    O, lse = A.paged_prefill(q, kc, vc, bt, L, p.scale)
    Od, Ld = A.paged_decode(q[:, :, 0], kc, vc, bt, L, p.scale)
    np.testing.assert_allclose(O[:, :, 0], Od, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, 0], Ld, atol=1e-12)


def test_window_one_returns_own_value_and_wide_window_changes_nothing():
    p = W.paged_prefill_inputs(3, 2, 4, 2, 16, 20, 16, 40, 70)
    q, kc, vc, bt, L = f64(p)
    O1, l1 = A.paged_prefill(q, kc, vc, bt, L, p.scale, window=1)
    for b in range(2):
        n = int(L[b])
        K = A.gather_paged(kc, bt, b, n)
        V = A.gather_paged(vc, bt, b, n)
        for h in range(4):
            g = h // 2
            np.testing.assert_array_equal(O1[b, h], V[n - 20:, g, :])
            np.testing.assert_allclose(l1[b, h], p.scale * (q[b, h] * K[n - 20:, g, :]).sum(-1), atol=1e-12)
    O0, l0 = A.paged_prefill(q, kc, vc, bt, L, p.scale)
    Ow, lw = A.paged_prefill(q, kc, vc, bt, L, p.scale, window=int(L.max()))
    np.testing.assert_array_equal(Ow, O0)
    np.testing.assert_array_equal(lw, l0)


@pytest.mark.parametrize("window", [0, 3, 7])
def test_equals_pure_python_loops(window):
    p = W.paged_prefill_inputs(4, 2, 4, 1, 3, 5, 16, 5, 37, window=window)
    q, kc, vc, bt, L = f64(p)
    O, lse = A.paged_prefill(q, kc, vc, bt, L, p.scale, window=window)
    for b in range(2):
        n = int(L[b])
        for h in range(4):
            for r in range(5):
                pos = n - 5 + r
                keys = [t for t in range(n) if t <= pos and (window == 0 or pos - t < window)]
                sc = {}
                for t in keys:
                    pid, slot = bt[b, t // 16], t % 16
                    sc[t] = p.scale * sum(q[b, h, r, d] * kc[pid, 0, slot, d] for d in range(3))
                mx = max(sc.values())
                w = {t: math.exp(sc[t] - mx) for t in keys}
                tot = sum(w.values())
                for d in range(3):
                    want = sum(w[t] * vc[bt[b, t // 16], 0, t % 16, d] for t in keys) / tot
                    assert abs(O[b, h, r, d] - want) < 1e-12
                assert abs(lse[b, h, r] - (mx + math.log(tot))) < 1e-12


def test_row_subset_equals_full_rows():
    p = W.paged_prefill_inputs(5, 2, 4, 2, 16, 40, 16, 40, 90, window=9)
    q, kc, vc, bt, L = f64(p)
    O, lse = A.paged_prefill(q, kc, vc, bt, L, p.scale, window=9)
    rows = np.array([0, 7, 31, 39])
    Os, ls = A.paged_prefill(q, kc, vc, bt, L, p.scale, window=9, rows=rows)
    np.testing.assert_array_equal(Os, O[:, :, rows])
    np.testing.assert_array_equal(ls, lse[:, :, rows])
