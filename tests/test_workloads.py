"""Generator checks: rounding, reproducibility, planted positions, paged layout."""
import numpy as np
import torch

import workloads as W


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.float32([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 65504.0, 1e-30])])
    mine = W.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> 1.0
    assert W.f32_from_bf16_bits(W.bf16_bits_from_f32(np.float32([1.0 + 2 ** -8])))[0] == 1.0
    np.testing.assert_array_equal(W.f32_from_bf16_bits(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeds_reproduce_bitwise():
    a = W.dense_inputs(7, 1, 4, 2, 128, 64, "bf16")
    b = W.dense_inputs(7, 1, 4, 2, 128, 64, "bf16")
    c = W.dense_inputs(8, 1, 4, 2, 128, 64, "bf16")
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, c.q)
    # streams are independent: q differs from k
    assert not np.array_equal(a.q[:, :2], a.k)


def test_planted_outliers_land_where_recorded():
    inp = W.planted_inputs(3, 1, 8, 2, 64 * 40, 64, block=64)
    nb = 40
    assert len(inp.planted) == 2 * (nb * 50 // 1000)
    base = W.dense_inputs(3, 1, 8, 2, 64 * 40, 64, "bf16")
    changed = np.argwhere((inp.k != base.k).any(axis=-1))
    rec = {(b, g, j * 64 + u) for (b, g, j, u, h, t) in inp.planted}
    assert {tuple(int(x) for x in c) for c in changed} <= rec
    for (b, g, j, u, h, t) in inp.planted:
        assert h // 4 == g and t // 64 > j and j <= nb - 2
        want = W.bf16_bits_from_f32(np.float32(6.0) * W.f32_from_bf16_bits(inp.q[b, h, t]))
        np.testing.assert_array_equal(inp.k[b, g, j * 64 + u], want)


def test_decode_layout_is_a_permutation_with_poisoned_tails():
    d = W.decode_inputs(5, 6, 8, 2, 64, 16, 20, 200)
    lens = d.seq_lens
    assert lens.min() >= 20 and lens.max() <= 200
    pages = (lens + 15) // 16
    used = np.concatenate([d.block_table[b, :pages[b]] for b in range(6)])
    np.testing.assert_array_equal(np.sort(used), np.arange(pages.sum()))
    for b in range(6):
        assert (d.block_table[b, pages[b]:] == -1).all()
        L = int(lens[b])
        last = d.block_table[b, (L - 1) // 16]
        tail = d.k_cache[last, :, (L - 1) % 16 + 1:, :]
        assert (tail == W.BF16_NAN_BITS).all()
        assert not (d.k_cache[last, :, :(L - 1) % 16 + 1, :] == W.BF16_NAN_BITS).any()


def test_sample_rows_hold_the_fixed_rows():
    inp = W.planted_inputs(3, 1, 8, 2, 64 * 40, 64, block=64)
    rows = W.sample_rows(3, 64 * 40, 8, 32, block=64, planted=inp.planted)
    assert rows.shape[0] == 8 and rows.shape[1] >= 32
    for h in range(8):
        r = set(rows[h].tolist())
        assert {0, 64 * 40 - 1} <= r
        assert len(r) == rows.shape[1]
    for (b, g, j, u, h, t) in inp.planted:
        assert t in set(rows[h].tolist())


def test_fp8_decode_inputs_match_the_bf16_workload():
    """Same lengths, block table and activation draws as the bf16 decode workload; codes are the E4M3 rounding of
    value / scale (within half a quantum of the bf16 values), the value cache is transposed within each page, and
    slots past each sequence hold the NaN code."""
    import torch
    d = W.decode_inputs(9, 3, 8, 2, 16, 16, 1, 100)
    f = W.decode_inputs_fp8(9, 3, 8, 2, 16, 16, 1, 100, k_scale=2.0 ** -6, v_scale=2.0 ** -6)
    assert np.array_equal(d.seq_lens, f.seq_lens) and np.array_equal(d.block_table, f.block_table)
    assert np.array_equal(d.q, f.q)
    assert f.v_cache_t.shape == (f.k_cache.shape[0], 2, 16, 16)
    kv = torch.from_numpy(f.k_cache).view(torch.float8_e4m3fn).double().numpy() * f.k_scale
    vv = torch.from_numpy(np.ascontiguousarray(f.v_cache_t.transpose(0, 1, 3, 2))).view(
        torch.float8_e4m3fn).double().numpy() * f.v_scale
    kb, vb = W.f64_from_bf16_bits(d.k_cache), W.f64_from_bf16_bits(d.v_cache)
    for b in range(3):
        L = int(d.seq_lens[b])
        t = np.arange(L)
        pid, slot = d.block_table[b, t // 16], t % 16
        for a, ref in ((kv, kb), (vv, vb)):
            x, y = a[pid, :, slot, :], ref[pid, :, slot, :]
            # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 (normal range); bf16 adds 2^-8 more
            assert np.all(np.abs(x - y) <= np.abs(y) * (2.0 ** -4 + 2.0 ** -8) + 2.0 ** -10 * f.k_scale)
        if L % 16:
            assert (f.k_cache[d.block_table[b, L // 16], :, L % 16:, :] == 0x7F).all()
            assert (f.v_cache_t[d.block_table[b, L // 16], :, :, L % 16:] == 0x7F).all()
