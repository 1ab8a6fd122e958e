"""The hot path under HIP graph capture: every entry point launches only kernels (no allocation, no memset), so a
captured step replays. The replays run with eager work and synchronisations between them, and each must match the
eager results bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import dev_bf16, dev_i32, say

pytestmark = pytest.mark.gpu


def test_captured_step_replays_bitwise(lib):
    inp = W.planted_inputs(71, 1, 8, 2, 64 * 16, 128, 64)
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    d = W.decode_inputs(72, 4, 16, 2, 64, 16, 100, 2000)
    dq, dk, dv = dev_bf16(d.q), dev_bf16(d.k_cache), dev_bf16(d.v_cache)
    dbt, dsl = dev_i32(d.block_table), dev_i32(d.seq_lens)
    f8 = W.decode_inputs_fp8(73, 4, 16, 2, 64, 16, 100, 2000)
    fq = dev_bf16(f8.q)
    fk = torch.from_numpy(f8.k_cache).cuda()
    fv = torch.from_numpy(f8.v_cache_t).cuda()
    fbt, fsl = dev_i32(f8.block_table), dev_i32(f8.seq_lens)
    pp = W.paged_prefill_inputs(74, 1, 8, 2, 128, 256, 16, 4096, 4096)
    pq, pk, pv = dev_bf16(pp.q), dev_bf16(pp.cache.k_cache), dev_bf16(pp.cache.v_cache)
    pbt, psl = dev_i32(pp.cache.block_table), dev_i32(pp.cache.seq_lens)

    # outputs and workspaces allocated up front, as a captured region requires
    o_dense = torch.empty_like(q)
    mask = lib.block_mask_build(q, k, 64, 150, 1.0, scale=inp.scale, rescue_mode=1)
    o_sparse = torch.empty_like(q)
    o_dec = torch.empty_like(dq)
    ws_dec = torch.empty(lib.decode_workspace_bytes(dq, dk, dbt, 2000), dtype=torch.uint8, device="cuda")
    o_f8 = torch.empty_like(fq)
    o_pp = torch.empty_like(pq)
    ws_pp = torch.empty(max(lib.prefill_paged_workspace_bytes(pq, pk, pbt), 256), dtype=torch.uint8, device="cuda")
    assert lib.prefill_paged_workspace_bytes(pq, pk, pbt) > 0, "the chunk is meant to take the key-range split"

    def step():
        lib.prefill_dense(q, k, v, scale=inp.scale, out=o_dense, return_lse=False)
        lib.block_mask_build(q, k, 64, 150, 1.0, scale=inp.scale, outputs=mask, rescue_mode=1)
        lib.prefill_block_sparse(q, k, v, mask.kv_count, mask.kv_index, 64, scale=inp.scale, out=o_sparse,
                                 return_lse=False)
        lib.decode_paged(dq, dk, dv, dbt, dsl, 2000, scale=d.scale, out=o_dec, return_lse=False, workspace=ws_dec)
        lib.decode_paged_fp8(fq, fk, fv, f8.k_scale, f8.v_scale, fbt, fsl, 2000, scale=f8.scale, out=o_f8,
                             return_lse=False, workspace=ws_dec)
        lib.prefill_paged(pq, pk, pv, pbt, psl, scale=pp.scale, out=o_pp, return_lse=False, workspace=ws_pp)

    outs = (o_dense, mask.mask, mask.kv_count, o_sparse, o_dec, o_f8, o_pp)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dense", "mask", "kv_count", "sparse", "decode", "decode fp8", "paged prefill"),
                                   outs, eager):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from eager"
        # eager work between replays
        junk = torch.ones(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        say(f"[graph] replay {rep} matches eager ({float(junk):.0f})")
