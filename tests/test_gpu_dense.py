"""GPU parity of attn_prefill_dense against the fp64 oracle (element-wise, or on seeded row samples at the
32K / 128K workload sizes)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_util import (BF16_TOL, FP32_TOL, LSE_TOL, host64, max_err, prefill_to_device, say, take_rows)

pytestmark = pytest.mark.gpu


def sampled_oracle(inp, rows):
    """Oracle outputs for rows [Hq,R] of every head; only the needed query rows are widened."""
    B, Hq, N, D = inp.q.shape
    G = Hq // inp.k.shape[1]
    kf = W.f64_from_bf16_bits(inp.k)
    vf = W.f64_from_bf16_bits(inp.v)
    Oref = np.zeros((B, Hq, rows.shape[1], D))
    Lref = np.zeros((B, Hq, rows.shape[1]))
    for h in range(Hq):
        g = h // G
        qh = np.zeros((B, 1, N, D))
        qh[:, 0, rows[h]] = W.f64_from_bf16_bits(inp.q[:, h, rows[h]])
        o_h, l_h = A.causal_attention(qh, kf[:, g:g + 1], vf[:, g:g + 1], inp.scale, rows=rows[h])
        Oref[:, h], Lref[:, h] = o_h[:, 0], l_h[:, 0]
    return Oref, Lref


def run_dense(lib, inp):
    q, k, v = prefill_to_device(inp)
    o, lse = lib.prefill_dense(q, k, v, scale=inp.scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


def check_full(lib, inp, tol, lse_tol, label):
    say(f"[dense] {label} shape={inp.shape} dtype={inp.dtype}")
    _, _, _, o, lse = run_dense(lib, inp)
    q, k, v = inp.as_f64()
    Oref, Lref = A.causal_attention(q, k, v, inp.scale)
    eo, el = max_err(host64(o), Oref), max_err(host64(lse), Lref)
    say(f"[dense] {label} max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert np.isfinite(host64(o)).all()
    assert eo <= tol and el <= lse_tol


def test_c1_fp32_n256(lib):
    w = W.WORKLOADS["c1_dense_fp32_n256"]
    inp = W.dense_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], "fp32")
    check_full(lib, inp, FP32_TOL, FP32_TOL, "c1")


@pytest.mark.parametrize("B,Hq,Hkv,N,D", [(2, 4, 2, 77, 128), (1, 3, 1, 130, 64), (1, 2, 2, 1, 64)])
def test_fp32_ragged(lib, B, Hq, Hkv, N, D):
    check_full(lib, W.dense_inputs(11, B, Hq, Hkv, N, D, "fp32"), FP32_TOL, FP32_TOL, f"fp32 N={N} D={D}")


@pytest.mark.parametrize("B,Hq,Hkv,N,D", [
    (1, 8, 1, 300, 128),     # G = 8: one work-group holds all heads of the group; ragged last tile
    (2, 8, 2, 257, 128),     # G = 4
    (1, 2, 2, 200, 128),     # MHA: 256 positions per work-group
    (1, 6, 2, 129, 64),      # G = 3, head_dim 64
    (1, 4, 4, 1, 128),       # a single token
    (1, 8, 8, 64, 64),       # exactly one tile
    (1, 16, 2, 1000, 128),   # G = 8 with several position tiles
    (1, 16, 1, 500, 128),    # G = 16: two work-groups per position block
    (2, 8, 1, 700, 64),      # head_dim 64, G = 8, two sequences
])
def test_bf16_small(lib, B, Hq, Hkv, N, D):
    check_full(lib, W.dense_inputs(21, B, Hq, Hkv, N, D, "bf16"), BF16_TOL, LSE_TOL, f"bf16 {B},{Hq},{Hkv},{N},{D}")


def test_c2_bf16_n4096_full(lib):
    w = W.WORKLOADS["c2_dense_bf16_n4k"]
    inp = W.dense_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], "bf16")
    check_full(lib, inp, BF16_TOL, LSE_TOL, "c2")


def test_deterministic(lib):
    inp = W.dense_inputs(5, 1, 8, 1, 700, 128, "bf16")
    q, k, v = prefill_to_device(inp)
    o1, l1 = lib.prefill_dense(q, k, v)
    o2, l2 = lib.prefill_dense(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_row_zero_is_v0_and_uniform_v(lib):
    inp = W.dense_inputs(6, 1, 8, 2, 256, 128, "bf16")
    q, k, v = prefill_to_device(inp)
    o, _ = lib.prefill_dense(q, k, v)
    torch.cuda.synchronize()
    for h in range(8):
        assert torch.equal(o[0, h, 0], v[0, h // 4, 0])
    vu = v[:, :, :1].expand_as(v).contiguous()
    o2, _ = lib.prefill_dense(q, k, vu)
    torch.cuda.synchronize()
    ref = vu[:, :, :1].float().repeat_interleave(4, dim=1).expand(-1, -1, 256, -1)
    assert (o2.float() - ref).abs().max().item() <= 8e-3


@pytest.mark.parametrize("name,per_head", [("dense_bf16_n32k", 256), ("c3_sparse_bf16_n32k", 256),
                                           ("c4_sparse_bf16_n128k", 256)])
def test_dense_long_sampled(lib, name, per_head):
    """Dense prefill over the long-context workloads' Q/K/V, checked on 256 seeded rows per head, always holding
    rows 0 and N-1 and block-boundary rows: the plain N(0,1) 32K workload the throughput line times (same inputs,
    same launch), and the planted 32K/128K workloads, whose samples also hold every planted query row."""
    w = W.WORKLOADS[name]
    say(f"[dense] {name}: generating inputs")
    if w["kind"] == "dense":
        inp = W.make(name)
        rows = W.sample_rows(w["seed"], w["N"], w["Hq"], per_head)
    else:
        inp = W.planted_inputs(w["seed"], w["B"], w["Hq"], w["Hkv"], w["N"], w["D"], w["block"])
        rows = W.sample_rows(w["seed"], w["N"], w["Hq"], per_head, block=w["block"], planted=inp.planted)
    q, k, v = prefill_to_device(inp)
    say(f"[dense] {name}: launching")
    o, lse = lib.prefill_dense(q, k, v, scale=inp.scale)
    torch.cuda.synchronize()
    og, lg = take_rows(o, rows), take_rows(lse.unsqueeze(-1), rows)[..., 0]
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    say(f"[dense] {name}: oracle on {rows.size} rows")
    Oref, Lref = sampled_oracle(inp, rows)
    eo, el = max_err(og, Oref), max_err(lg, Lref)
    say(f"[dense] {name}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= BF16_TOL and el <= LSE_TOL


def test_binding_rejects_mismatched_buffers(lib):
    """The library gets plain pointers and trusts sizes: the binding refuses wrong-sized outputs and workspaces
    before anything is launched."""
    dev = torch.device("cuda", 0)
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device=dev)
    with pytest.raises(lib.LcattnError):
        lib.prefill_dense(q, k, k, out=torch.empty(1, 4, 63, 64, dtype=torch.bfloat16, device=dev))
    with pytest.raises(lib.LcattnError):
        lib.prefill_dense(q, k, k, out=torch.empty(1, 4, 64, 64, dtype=torch.float32, device=dev))
    cnt = torch.ones(1, 4, 1, dtype=torch.int32, device=dev)
    idx = torch.zeros(1, 4, 1, 1, dtype=torch.int32, device=dev)
    with pytest.raises(lib.LcattnError):
        lib.prefill_block_sparse(q, k, k, cnt, idx, 64, out=torch.empty(2, 4, 64, 64, dtype=torch.bfloat16,
                                                                          device=dev))
    m = lib.block_mask_build(q, k, 64, 100, 1.0)
    m.kv_index = torch.empty(1, 4, 1, 2, dtype=torch.int32, device=dev)
    with pytest.raises(lib.LcattnError):
        lib.block_mask_build(q, k, 64, 100, 1.0, outputs=m)
    q1 = torch.zeros(2, 4, 64, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(8, 2, 16, 64, dtype=torch.bfloat16, device=dev)
    bt = torch.zeros(2, 4, dtype=torch.int32, device=dev)
    with pytest.raises(lib.LcattnError):   # one sequence length for two sequences
        lib.decode_paged(q1, kc, kc, bt, torch.ones(1, dtype=torch.int32, device=dev), 64)
    with pytest.raises(lib.LcattnError):   # workspace of the wrong element type
        lib.decode_paged(q1, kc, kc, bt, torch.ones(2, dtype=torch.int32, device=dev), 64,
                         workspace=torch.empty(1 << 20, dtype=torch.float32, device=dev))
