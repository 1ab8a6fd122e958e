"""GPU parity of attn_block_mask_build (bit-exact masks) and attn_prefill_block_sparse (against the oracle's
masked attention, fed the oracle's own mask so the two checks stay separate)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from oracle import block_mask as M
from tests.gpu_util import BF16_TOL, LSE_TOL, dev_i32, host64, max_err, prefill_to_device, say, take_rows

pytestmark = pytest.mark.gpu


def gpu_mask(lib, inp, keep, alpha, lo=50, hi=90, mode=0):
    q, k, _ = prefill_to_device(inp)
    m = lib.block_mask_build(q, k, inp.block, keep, alpha, lo, hi, scale=inp.scale, rescue_mode=mode)
    torch.cuda.synchronize()
    return m


def ambiguous_rows(ref: M.MaskResult, G: int) -> np.ndarray:
    """Rows whose result may legitimately differ between two correct fp64 evaluations: the centroid cut falls on
    a score gap below 1e-12 relative, a radius lies within 1e-12 relative of its threshold, or (query-aware
    rescue) a candidate's rescue score lies within 1e-12 relative of the row's cutoff."""
    amb = (ref.cut_gap < 1e-12 * (1.0 + ref.score_absmax)) | (ref.rescue_gap < 1e-12)
    tau = ref.tau[:, :, None]
    near = np.isfinite(tau) & (np.abs(ref.radius - tau) <= 1e-12 * np.abs(tau))   # tau = inf flags nothing
    B, Hq, nb = ref.kv_count.shape
    for h in range(Hq):
        touched = near[:, h // G, :]                      # [B, nb] key blocks
        # a near-threshold key block j affects every row i >= j
        first = np.where(touched.any(axis=1), touched.argmax(axis=1), nb)
        for b in range(B):
            amb[b, h, first[b]:] = True
    return amb


def compare_mask(lib, inp, keep, alpha, label, lo=50, hi=90, mode=0):
    say(f"[mask] {label} mode {mode}: gpu")
    m = gpu_mask(lib, inp, keep, alpha, lo, hi, mode)
    q, k, _ = inp.as_f64()
    say(f"[mask] {label} mode {mode}: oracle")
    # the library takes the scale as float32
    ref = M.build_mask(q, k, float(np.float32(inp.scale)), inp.block, keep, alpha, lo, hi, rescue_mode=mode)
    G = inp.q.shape[1] // inp.k.shape[1]
    mask = m.mask.cpu().numpy()
    cnt = m.kv_count.cpu().numpy()
    idx = m.kv_index.cpu().numpy()
    rs = m.radius_stats.cpu().numpy()
    nb = ref.mask.shape[-1]
    # radii and thresholds: the same fp64 quantities up to summation order
    np.testing.assert_allclose(rs[..., :nb], ref.radius, rtol=1e-12, atol=0)
    if not math.isinf(alpha):
        np.testing.assert_allclose(rs[..., nb + 2], ref.tau, rtol=1e-12, atol=0)
    np.testing.assert_allclose(rs[..., nb], ref.med, rtol=1e-12, atol=0)
    np.testing.assert_allclose(rs[..., nb + 1], ref.p90, rtol=1e-12, atol=0)
    amb = ambiguous_rows(ref, G)
    bad = (mask != ref.mask).any(axis=-1)
    say(f"[mask] {label}: rows={bad.size} mismatched={int(bad.sum())} ambiguous={int(amb.sum())} "
        f"density={ref.mask.sum() / (bad.size * (nb + 1) / 2):.4f}")
    assert not (bad & ~amb).any(), "mask differs outside the documented tie band"
    ok = ~amb
    np.testing.assert_array_equal(cnt[ok], ref.kv_count[ok])
    B, Hq = cnt.shape[:2]
    for b in range(B):
        for h in range(Hq):
            for i in np.nonzero(ok[b, h])[0]:
                c = cnt[b, h, i]
                if not np.array_equal(idx[b, h, i, :c], ref.kv_index[b, h, i, :c]):
                    raise AssertionError(f"kv_index differs at {(b, h, i)}")
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
    qf, _, _ = inp.as_f64()
    ref = M.build_mask_fp8_keys(qf, codes, ksc32, float(np.float32(inp.scale)), inp.block, keep, alpha, lo, hi,
                                rescue_mode=mode)
    G = inp.q.shape[1] // inp.k.shape[1]
    nb = ref.mask.shape[-1]
    rs = m.radius_stats.cpu().numpy()
    np.testing.assert_allclose(rs[..., :nb], ref.radius, rtol=1e-12, atol=0)
    amb = ambiguous_rows(ref, G)
    mask = m.mask.cpu().numpy()
    bad = (mask != ref.mask).any(axis=-1)
    say(f"[mask fp8k] {label} mode {mode}: rows={bad.size} mismatched={int(bad.sum())} ambiguous={int(amb.sum())}")
    assert not (bad & ~amb).any(), "fp8-key mask differs outside the documented tie band"
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


@pytest.mark.parametrize("block", [64, 128])
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
    assert (lse - ld).abs().max().item() <= 1e-3


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


def test_sparse_deterministic(lib):
    inp = W.planted_inputs(45, 1, 8, 2, 64 * 16, 128, 64)
    q, k, v = inp.as_f64()
    ref = M.build_mask(q, k, inp.scale, 64, 200, 1.0)
    o1, l1 = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    o2, l2 = run_sparse(lib, inp, ref.kv_count, ref.kv_index)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
