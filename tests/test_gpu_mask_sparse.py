"""GPU parity of attn_block_mask_build (bit-exact masks) and attn_prefill_block_sparse (against the oracle's
masked attention, fed the oracle's own mask so the two checks stay separate)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import block_mask as M
from tests import mask_check
from tests.gpu_util import BF16_TOL, LSE_TOL, dev_i32, host64, max_err, prefill_to_device, say, take_rows

pytestmark = pytest.mark.gpu


def gpu_mask(lib, inp, keep, alpha, lo=50, hi=90, mode=0):
    q, k, _ = prefill_to_device(inp)
    m = lib.block_mask_build(q, k, inp.block, keep, alpha, lo, hi, scale=inp.scale, rescue_mode=mode)
    torch.cuda.synchronize()
    return m


def check_against_oracle(m, ref, qf, kf, scale, keep, mode, label, tag="mask"):
    """Every entry of the library's mask against the oracle's: entries fixed by the rule must match, entries in the
    documented fp64 tie band may take either value within the row's pick count, and kv_count/kv_index must be the
    CSR form of the library's own mask. The seeded workloads have no entry in the band, which is asserted."""
    qbar, kbar, _ = M.block_stats(qf, kf, qf.shape[2] // ref.mask.shape[-1])
    st = mask_check.entry_status(ref, qbar, kbar, scale, keep, mode)
    mask = m.mask.cpu().numpy()
    cnt = m.kv_count.cpu().numpy()
    idx = m.kv_index.cpu().numpy()
    nb = ref.mask.shape[-1]
    diff = int((mask != ref.mask).sum())
    say(f"[{tag}] {label} mode {mode}: rows={cnt.size} differing entries={diff} free entries="
        f"{int(st.free.sum())} density={ref.mask.sum() / (cnt.size * (nb + 1) / 2):.4f}")
    mask_check.check_mask(mask, cnt, idx, st, max_free=0)
    # with no entry in the band the answer is unique
    np.testing.assert_array_equal(mask, ref.mask)
    np.testing.assert_array_equal(cnt, ref.kv_count)


def compare_mask(lib, inp, keep, alpha, label, lo=50, hi=90, mode=0):
    say(f"[mask] {label} mode {mode}: gpu")
    m = gpu_mask(lib, inp, keep, alpha, lo, hi, mode)
    q, k, _ = inp.as_f64()
    say(f"[mask] {label} mode {mode}: oracle")
    # the library takes the scale as float32
    sc = float(np.float32(inp.scale))
    ref = M.build_mask(q, k, sc, inp.block, keep, alpha, lo, hi, rescue_mode=mode)
    rs = m.radius_stats.cpu().numpy()
    nb = ref.mask.shape[-1]
    # radii and thresholds: the same fp64 quantities up to summation order
    np.testing.assert_allclose(rs[..., :nb], ref.radius, rtol=1e-12, atol=0)
    if not math.isinf(alpha):
        np.testing.assert_allclose(rs[..., nb + 2], ref.tau, rtol=1e-12, atol=0)
    np.testing.assert_allclose(rs[..., nb], ref.med, rtol=1e-12, atol=0)
    np.testing.assert_allclose(rs[..., nb + 1], ref.p90, rtol=1e-12, atol=0)
    check_against_oracle(m, ref, q, k, sc, keep, mode, label)
    return m, ref


def compare_mask_fp8_keys(lib, inp, keep, alpha, label, lo=50, hi=90, mode=0):
    """The mask from E4M3 key codes (per-tensor scale) against the oracle applied to the dequantised keys."""
    codes, ksc = W.e4m3_keys(inp.k)
    ksc32 = float(np.float32(ksc))
    q, _, _ = prefill_to_device(inp)
    say(f"[mask fp8k] {label} mode {mode}: gpu")
    m = lib.block_mask_build(q, torch.from_numpy(codes).cuda(), inp.block, keep, alpha, lo, hi, scale=inp.scale,
                             rescue_mode=mode, k_scale=ksc32)
    torch.cuda.synchronize()
    del q
    qf, _, _ = inp.as_f64()
    sc = float(np.float32(inp.scale))
    say(f"[mask fp8k] {label} mode {mode}: oracle")
    ref = M.build_mask_fp8_keys(qf, codes, ksc32, sc, inp.block, keep, alpha, lo, hi, rescue_mode=mode)
    nb = ref.mask.shape[-1]
    rs = m.radius_stats.cpu().numpy()
    np.testing.assert_allclose(rs[..., :nb], ref.radius, rtol=1e-12, atol=0)
    np.testing.assert_allclose(rs[..., nb], ref.med, rtol=1e-12, atol=0)
    np.testing.assert_allclose(rs[..., nb + 1], ref.p90, rtol=1e-12, atol=0)
    if not math.isinf(alpha):
        np.testing.assert_allclose(rs[..., nb + 2], ref.tau, rtol=1e-12, atol=0)
    kf = A.e4m3_value(codes) * ksc32
    check_against_oracle(m, ref, qf, kf, sc, keep, mode, label, tag="mask fp8k")
    return m, ref


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("B,Hq,Hkv,N,D,block,keep,alpha", [
    (2, 8, 2, 64 * 40, 128, 64, 100, 1.0),
    (1, 4, 4, 128 * 20, 64, 128, 50, 1.0),
])
def test_mask_fp8_keys_small(lib, B, Hq, Hkv, N, D, block, keep, alpha, mode):
    inp = W.planted_inputs(46, B, Hq, Hkv, N, D, block)
    compare_mask_fp8_keys(lib, inp, keep, alpha, f"small {B},{Hq},{Hkv},{N},{D},b{block}", mode=mode)


@pytest.mark.parametrize("mode", [0, 1])
def test_mask_fp8_keys_c3(lib, mode):
    """The 32K workload's mask from fp8 keys: bit-exact with the oracle, and every planted block still kept in the row
    of its query (the rescue signal survives eight-bit keys on this workload)."""
    w = W.WORKLOADS["c3_sparse_bf16_n32k"]
    inp = W.planted_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["block"])
    m, ref = compare_mask_fp8_keys(lib, inp, w["keep_permille"], w["alpha"], "c3", w["q_lo_pct"], w["q_hi_pct"],
                                   mode)
    mask = m.mask.cpu().numpy()
    for (b, g, j, u, h, t) in inp.planted:
        assert mask[b, h, t // w["block"], j] == 1


@pytest.mark.parametrize("mode", [0, 1])
def test_mask_fp8_keys_c4(lib, mode):
    """The 128K workload's mask from fp8 keys: bit-exact with the oracle (mask, kv_count, kv_index), and every
    planted block still kept in the row of its query."""
    w = W.WORKLOADS["c4_sparse_bf16_n128k"]
    say("[mask fp8k] c4: generating inputs")
    inp = W.planted_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["block"])
    m, ref = compare_mask_fp8_keys(lib, inp, w["keep_permille"], w["alpha"], "c4", w["q_lo_pct"], w["q_hi_pct"],
                                   mode)
    mask = m.mask.cpu().numpy()
    for (b, g, j, u, h, t) in inp.planted:
        assert mask[b, h, t // w["block"], j] == 1
    del m
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", [0, 1])
def test_mask_exact_ties_go_to_the_smaller_block(lib, mode):
    """Every key block with the same centroid: each row's centroid scores tie exactly, on the GPU as in the oracle
    (identical columns give identical fp64 products), and the rule's tie-break (the smaller block) decides. The radii
    differ, so the rescue branch still flags blocks; the mask must be the oracle's bit for bit."""
    B, Hq, Hkv, nb, blk, D = 1, 4, 2, 24, 64, 64
    rng = np.random.default_rng(48)
    q = rng.standard_normal((B, Hq, nb * blk, D)).astype(np.float32)
    k = np.empty((B, Hkv, nb * blk, D), np.float32)
    sign = np.where(np.arange(blk) % 2 == 0, 1.0, -1.0).astype(np.float32)[:, None]
    for g in range(Hkv):
        c = np.round(rng.standard_normal(D) * 4) / 4      # quarters: exact in bf16, exact block means
        for j in range(nb):
            d = np.round(rng.standard_normal(D) * 4 * (1 + j % 5)) / 4
            k[0, g, j * blk:(j + 1) * blk] = c + sign * d
    inp = W.PrefillInputs(q=W.bf16_bits_from_f32(q), k=W.bf16_bits_from_f32(k),
                          v=W.bf16_bits_from_f32(np.zeros_like(k)), dtype="bf16", scale=1.0 / 8.0, block=blk)
    assert np.array_equal(W.f64_from_bf16_bits(inp.k), k.astype(np.float64))
    m = gpu_mask(lib, inp, 250, 1.0, mode=mode)
    qf, kf, _ = inp.as_f64()
    ref = M.build_mask(qf, kf, 0.125, blk, 250, 1.0, rescue_mode=mode)
    say(f"[mask ties] mode {mode}: rows with a zero cut gap = {int((ref.cut_gap == 0).sum())}")
    assert (ref.cut_gap == 0).sum() > 0
    np.testing.assert_array_equal(m.mask.cpu().numpy(), ref.mask)
    np.testing.assert_array_equal(m.kv_count.cpu().numpy(), ref.kv_count)
    cnt = ref.kv_count
    idx = m.kv_index.cpu().numpy()
    for pos in np.ndindex(cnt.shape):
        assert np.array_equal(idx[pos][:cnt[pos]], ref.kv_index[pos][:cnt[pos]])


@pytest.mark.parametrize("B,Hq,Hkv,N,D,block,keep,alpha", [
    (2, 8, 2, 64 * 40, 128, 64, 100, 1.0),
    (1, 4, 4, 128 * 20, 64, 128, 50, 1.0),
    (1, 8, 1, 64 * 70, 128, 64, 300, 0.5),
    (1, 2, 1, 64 * 3, 128, 64, 100, 2.0),
    (1, 4, 2, 256 * 9, 128, 256, 200, 1.0),
])
@pytest.mark.parametrize("mode", [0, 1])
def test_mask_small(lib, B, Hq, Hkv, N, D, block, keep, alpha, mode):
    inp = W.planted_inputs(41, B, Hq, Hkv, N, D, block)
    compare_mask(lib, inp, keep, alpha, f"small {B},{Hq},{Hkv},{N},{D},b{block},k{keep},a{alpha}", mode=mode)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("N", [131072, 262144])
def test_mask_largest_block_counts(lib, N, mode):
    """The select kernel's two widest instantiations: 2048 and 4096 (the library's maximum) key blocks per row,
    64-row blocks, one kv head shared by two query heads."""
    inp = W.planted_inputs(47, 1, 2, 1, N, 64, 64)
    m, _ = compare_mask(lib, inp, 60, 1.0, f"largest nb={N // 64}", mode=mode)
    del m
    torch.cuda.empty_cache()


def test_mask_special_rules(lib):
    inp = W.planted_inputs(42, 1, 8, 2, 64 * 30, 128, 64)
    nb = 30
    full = gpu_mask(lib, inp, 1000, 1.0).mask.cpu().numpy()
    assert (full == np.tril(np.ones((nb, nb), np.uint8))).all()
    diag = gpu_mask(lib, inp, 0, math.inf).mask.cpu().numpy()
    assert (diag == np.eye(nb, dtype=np.uint8)).all()
    compare_mask(lib, inp, 150, math.inf, "centroid only")
    compare_mask(lib, inp, 0, 0.0, "rescue only, alpha 0")
    # query-aware: alpha = inf is the centroid branch alone; no budget means no cutoff, so nothing is rescued
    cen = compare_mask(lib, inp, 150, math.inf, "centroid only", mode=1)[0].mask.cpu().numpy()
    assert (cen == gpu_mask(lib, inp, 150, math.inf).mask.cpu().numpy()).all()
    diag1 = gpu_mask(lib, inp, 0, 0.0, mode=1).mask.cpu().numpy()
    assert (diag1 == np.eye(nb, dtype=np.uint8)).all()
    # alpha = 0 widens the candidates to every block above the median radius; the query-aware mask stays inside
    # the query-blind one
    aware, _ = compare_mask(lib, inp, 150, 0.0, "alpha 0", mode=1)
    blind = gpu_mask(lib, inp, 150, 0.0).mask.cpu().numpy()
    assert (aware.mask.cpu().numpy() <= blind).all()


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("name", ["c3_sparse_bf16_n32k", "c4_sparse_bf16_n128k"])
def test_mask_full_size(lib, name, mode):
    w = W.WORKLOADS[name]
    say(f"[mask] {name}: generating inputs")
    inp = W.planted_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["block"])
    m, ref = compare_mask(lib, inp, w["keep_permille"], w["alpha"], name, w["q_lo_pct"], w["q_hi_pct"], mode)
    # every planted block is kept in the row of the query it was planted for (mean dilution would hide many from
    # the centroids; the query-aware rescue still reaches them through the radius allowance)
    mask = m.mask.cpu().numpy()
    for (b, g, j, u, h, t) in inp.planted:
        assert mask[b, h, t // w["block"], j] == 1


# ------------------------------------------------------------------------------------------------ sparse prefill
def run_sparse(lib, inp, kv_count, kv_index):
    q, k, v = prefill_to_device(inp)
    o, lse = lib.prefill_block_sparse(q, k, v, dev_i32(kv_count), dev_i32(kv_index), inp.block, scale=inp.scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,N,D,block,keep,alpha", [
    (1, 8, 2, 64 * 20, 128, 64, 150, 1.0),
    (1, 4, 1, 128 * 12, 128, 128, 100, 1.0),
    (1, 8, 4, 64 * 11, 64, 64, 200, 0.5),
    (1, 4, 2, 256 * 6, 128, 256, 300, 1.0),
    (1, 8, 2, 64 * 20, 128, 64, 0, math.inf),  # diagonal blocks only
    (2, 8, 2, 64 * 12, 128, 64, 150, 1.0),     # two sequences: the head order spans the batch
    (1, 24, 3, 128 * 6, 128, 128, 100, 1.0),   # 24 heads: three per XCD in kv-group order
    (1, 16, 1, 64 * 10, 64, 64, 200, 1.0),     # G = 16, head_dim 64
    (1, 8, 2, 256 * 5, 64, 256, 250, 1.0),     # 256-row blocks at head_dim 64: each block over two work-groups
    (2, 4, 1, 256 * 3, 128, 256, 400, 0.5),    # 256-row blocks, two sequences
])
def test_sparse_small_full(lib, B, Hq, Hkv, N, D, block, keep, alpha):
    inp = W.planted_inputs(43, B, Hq, Hkv, N, D, block)
    q, k, v = inp.as_f64()
    ref = M.build_mask(q, k, inp.scale, block, keep, alpha)
    o, lse = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    Oref, Lref = A.masked_attention(q, k, v, inp.scale, ref.mask, block)
    eo, el = max_err(host64(o), Oref), max_err(host64(lse), Lref)
    say(f"[sparse] small {B},{Hq},{Hkv},{N},{D},b{block} max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= BF16_TOL and el <= LSE_TOL


@pytest.mark.parametrize("block", [64, 128, 256])
def test_sparse_all_blocks_equals_dense(lib, block):
    inp = W.planted_inputs(44, 1, 8, 2, block * 10, 128, block)
    nb = 10
    cnt = np.broadcast_to(np.arange(1, nb + 1, dtype=np.int32), (1, 8, nb)).copy()
    idx = np.full((1, 8, nb, nb), -1, np.int32)
    for i in range(nb):
        idx[..., i, :i + 1] = np.arange(i + 1)
    o, lse = run_sparse(lib, inp, cnt, idx)
    q, k, v = prefill_to_device(inp)
    od, ld = lib.prefill_dense(q, k, v, scale=inp.scale)
    torch.cuda.synchronize()
    Oref, _ = A.causal_attention(*inp.as_f64(), inp.scale)
    assert max_err(host64(o), Oref) <= BF16_TOL
    assert (o.float() - od.float()).abs().max().item() <= BF16_TOL
    # 128- and 256-row blocks walk the dense kernel's 64-key tiles, so both paths round the same probabilities;
    # 64-row blocks walk 32-key tiles, whose running maxima (hence the bf16 roundings in the row sums) can differ
    # from the dense walk's: two independently rounded sums, each within 2^-8 relative, agree in ln l to 2 * 2^-8
    assert (lse - ld).abs().max().item() <= (2 * 2.0 ** -8 if block == 64 else 1e-3)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("name", ["c3_sparse_bf16_n32k", "c4_sparse_bf16_n128k"])
def test_sparse_full_size_sampled(lib, name, mode):
    """The sparse kernel over the oracle's lists at full size, for the query-blind and the query-aware rescue."""
    w = W.WORKLOADS[name]
    say(f"[sparse] {name} mode {mode}: generating inputs")
    inp = W.planted_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["block"])
    q, k, v = inp.as_f64()
    say(f"[sparse] {name} mode {mode}: oracle mask")
    ref = M.build_mask(q, k, inp.scale, w["block"], w["keep_permille"], w["alpha"], w["q_lo_pct"], w["q_hi_pct"],
                       rescue_mode=mode)
    del q
    say(f"[sparse] {name}: gpu")
    o, lse = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    per = 512 if name.startswith("c3") else 256
    rows = W.sample_rows(w["seed"], w["N"], w["Hq"], per, block=w["block"], planted=inp.planted)
    og, lg = take_rows(o, rows), take_rows(lse.unsqueeze(-1), rows)[..., 0]
    del o, lse
    say(f"[sparse] {name}: oracle rows {rows.size}")
    B, Hq, N, D = inp.q.shape
    G = Hq // inp.k.shape[1]
    Oref = np.zeros_like(og)
    Lref = np.zeros_like(lg)
    for h in range(Hq):
        g = h // G
        qh = np.zeros((B, 1, N, D))
        qh[:, 0, rows[h]] = W.f64_from_bf16_bits(inp.q[:, h, rows[h]])
        o_h, l_h = A.masked_attention(qh, k[:, g:g + 1], v[:, g:g + 1], inp.scale, ref.mask[:, h:h + 1], w["block"],
                                      rows=rows[h])
        Oref[:, h], Lref[:, h] = o_h[:, 0], l_h[:, 0]
    eo, el = max_err(og, Oref), max_err(lg, Lref)
    say(f"[sparse] {name} mode {mode}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= BF16_TOL and el <= LSE_TOL


def test_sparse_largest_block_count(lib):
    """The sparse kernel at the library's largest block count: 4096 key blocks of 64 rows (N = 262144), so each
    row's kept list takes 16 KiB of LDS beside the tiles. Sampled rows against the oracle over the oracle's lists,
    the last row of the sequence included."""
    N, blk = 262144, 64
    inp = W.planted_inputs(49, 1, 2, 1, N, 64, blk)
    q, k, v = inp.as_f64()
    say("[sparse] largest nb=4096: oracle mask")
    ref = M.build_mask(q, k, inp.scale, blk, 30, 1.0)
    del q
    o, lse = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    rows = W.sample_rows(49, N, 2, 48, block=blk, planted=inp.planted)
    og, lg = take_rows(o, rows), take_rows(lse.unsqueeze(-1), rows)[..., 0]
    del o, lse
    Oref = np.zeros_like(og)
    Lref = np.zeros_like(lg)
    for h in range(2):
        qh = np.zeros((1, 1, N, 64))
        qh[:, 0, rows[h]] = W.f64_from_bf16_bits(inp.q[:, h, rows[h]])
        o_h, l_h = A.masked_attention(qh, k, v, inp.scale, ref.mask[:, h:h + 1], blk, rows=rows[h])
        Oref[:, h], Lref[:, h] = o_h[:, 0], l_h[:, 0]
    eo, el = max_err(og, Oref), max_err(lg, Lref)
    say(f"[sparse] largest nb=4096: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= BF16_TOL and el <= LSE_TOL
    torch.cuda.empty_cache()


def test_sparse_deterministic(lib):
    inp = W.planted_inputs(45, 1, 8, 2, 64 * 16, 128, 64)
    q, k, v = inp.as_f64()
    ref = M.build_mask(q, k, inp.scale, 64, 200, 1.0)
    o1, l1 = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    o2, l2 = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
