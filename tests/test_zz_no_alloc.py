"""attn_decode_paged_noalloc (the decode entry point that allocates nothing, its chunk partials in the library's
own per-GPU scratch) against attn_decode_paged on the same inputs: two calls in a row, the second on a smaller
problem, each bit-identical to the workspace entry point (the same kernels) and within the bf16 bar of the oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_util import BF16_TOL, LSE_TOL, dev_bf16, dev_i32, host64, max_err, say

pytestmark = pytest.mark.gpu


def _inputs(d):
    return dev_bf16(d.q), dev_bf16(d.k_cache), dev_bf16(d.v_cache), dev_i32(d.block_table), dev_i32(d.seq_lens)


def test_noalloc_decode_matches_workspace_entry_point(lib):
    w = W.WORKLOADS["c5_decode_paged_bf16"]
    cases = [("c5 shape", W.make("c5_decode_paged_bf16"), w["len_hi"], w["chunk"]),
             ("smaller", W.decode_inputs(81, 5, 16, 2, 64, 16, 1, 3000, seq_lens=np.array([3000, 1, 0, 700, 2049])),
              3000, 512)]
    for label, d, maxlen, chunk in cases:
        say(f"[noalloc] {label}: B={d.q.shape[0]} Hq={d.q.shape[1]} max_len={maxlen} chunk={chunk}")
        q, kc, vc, bt, sl = _inputs(d)
        o_ref, l_ref = lib.decode_paged(q, kc, vc, bt, sl, maxlen, chunk_tokens=chunk, scale=d.scale)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        lib.decode_paged_noalloc(q, kc, vc, bt, sl, maxlen, chunk_tokens=chunk, scale=d.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"{label}: output differs from attn_decode_paged"
        assert torch.equal(lse, l_ref), f"{label}: lse differs from attn_decode_paged"
        Oref, Lref = A.paged_decode(W.f64_from_bf16_bits(d.q), W.f64_from_bf16_bits(d.k_cache),
                                    W.f64_from_bf16_bits(d.v_cache), d.block_table, d.seq_lens, d.scale)
        live = d.seq_lens > 0
        eo, el = max_err(host64(o), Oref), max_err(host64(lse)[live], Lref[live])
        say(f"[noalloc] {label}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= BF16_TOL and el <= LSE_TOL


def test_noalloc_refuses_oversized_shapes(lib):
    """A shape whose partials exceed the scratch is refused before anything is enqueued."""
    d = W.decode_inputs(82, 2, 16, 2, 64, 16, 1, 64)
    q, kc, vc, bt, _ = _inputs(d)
    big_bt = torch.zeros(1024, 8192, dtype=torch.int32, device=q.device)
    qb = torch.zeros(1024, 16, 64, dtype=torch.bfloat16, device=q.device)
    slb = torch.ones(1024, dtype=torch.int32, device=q.device)
    with pytest.raises(lib.LcattnError) as e:
        lib.decode_paged_noalloc(qb, kc, vc, big_bt, slb, 131072, chunk_tokens=64, out=torch.empty_like(qb))
    assert e.value.status == 5
