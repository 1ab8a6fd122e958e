"""GPU parity of attn_prefill_paged (chunked prefill over a paged cache, optional sliding window) against the fp64
oracle, and bit-equality with the dense kernel when the chunk is the whole sequence."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_util import BF16_TOL, LSE_TOL, dev_bf16, dev_i32, host64, max_err, say

pytestmark = pytest.mark.gpu


def run(lib, p: W.PagedPrefillInputs):
    c = p.cache
    o, lse = lib.prefill_paged(dev_bf16(p.q), dev_bf16(c.k_cache), dev_bf16(c.v_cache), dev_i32(c.block_table),
                               dev_i32(c.seq_lens), window=p.window, scale=p.scale)
    torch.cuda.synchronize()
    return o, lse


def compare(lib, p, label, rows=None):
    o, lse = run(lib, p)
    c = p.cache
    say(f"[paged prefill] {label}: oracle")
    Oref, Lref = A.paged_prefill(W.f64_from_bf16_bits(p.q), W.f64_from_bf16_bits(c.k_cache),
                                 W.f64_from_bf16_bits(c.v_cache), c.block_table, c.seq_lens,
                                 float(np.float32(p.scale)), window=p.window, rows=rows)
    og, lg = host64(o), host64(lse)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    eo, el = max_err(og, Oref), max_err(lg, Lref)
    say(f"[paged prefill] {label}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert np.isfinite(og).all()
    assert eo <= BF16_TOL and el <= LSE_TOL


@pytest.mark.parametrize("B,Hq,Hkv,D,Nq,lens,window", [
    (2, 8, 2, 128, 100, [100, 300], 0),
    (3, 16, 2, 64, 64, [64, 65, 1000], 0),
    (2, 8, 8, 128, 37, [37, 515], 0),
    (1, 16, 1, 64, 200, [900], 0),
    (2, 8, 2, 128, 150, [150, 700], 1),
    (2, 8, 2, 128, 150, [150, 700], 17),
    (2, 8, 2, 64, 150, [150, 700], 64),
    (2, 8, 2, 128, 150, [160, 701], 100),
    (2, 8, 2, 128, 150, [150, 700], 1000),
    (2, 64, 8, 64, 300, [2000, 3001], 128),
    (3, 8, 2, 64, 1, [1, 17, 999], 0),           # one-token chunks
    (2, 8, 2, 128, 64, [64, 1024], 1),           # window 1 at tile boundaries
    (1, 4, 1, 64, 40, [4096], 1),                # window 1, head_dim 64
    (2, 8, 2, 64, 70, [512, 70], 20),            # window narrower than a 32-row slice
])
def test_small(lib, B, Hq, Hkv, D, Nq, lens, window):
    p = W.paged_prefill_inputs(61, B, Hq, Hkv, D, Nq, 16, Nq, max(lens), window=window, seq_lens=np.array(lens))
    compare(lib, p, f"B{B} Hq{Hq} Hkv{Hkv} D{D} Nq{Nq} L{lens} W{window}")


def _rows(Nq, n, seed):
    rng = np.random.default_rng(seed)
    fixed = {0, 31, 32, 63, 64, Nq // 2, Nq - 1}
    extra = rng.choice(Nq, size=n, replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)))


@pytest.mark.parametrize("name", ["c6_paged_prefill_chunk", "c7_paged_prefill_window"])
def test_full_size_sampled(lib, name):
    w = W.WORKLOADS[name]
    say(f"[paged prefill] {name}: generating inputs")
    p = W.make(name)
    compare(lib, p, name, rows=_rows(w["Nq"], 64, w["seed"]))


@pytest.mark.parametrize("D,N", [(128, 1000), (64, 4096)])
def test_whole_sequence_equals_dense_kernel_bitwise(lib, D, N):
    """One chunk covering the whole sequence: the same work-groups, tiles and arithmetic as the dense kernel, only
    gathered through the block table, so the outputs must agree bit for bit."""
    Hq, Hkv, page = 8, 2, 16
    inp = W.dense_inputs(62, 1, Hq, Hkv, N, D, "bf16")
    npg = -(-N // page)
    perm = np.random.default_rng(63).permutation(npg + 5)[:npg].astype(np.int32)
    kc = np.full((npg + 5, Hkv, page, D), W.BF16_NAN_BITS, np.uint16)
    vc = kc.copy()
    for t in range(N):
        kc[perm[t // page], :, t % page] = inp.k[0, :, t]
        vc[perm[t // page], :, t % page] = inp.v[0, :, t]
    q = dev_bf16(inp.q)
    o1, l1 = lib.prefill_paged(q, dev_bf16(kc), dev_bf16(vc), dev_i32(perm[None, :]), dev_i32(np.array([N])),
                               scale=inp.scale)
    o2, l2 = lib.prefill_dense(q, dev_bf16(inp.k), dev_bf16(inp.v), scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("D,Nq,lens", [(128, 256, [4096]), (64, 200, [3000, 700]), (128, 96, [2500, 96, 1200])])
def test_key_range_split_matches_oracle_and_unsplit(lib, D, Nq, lens):
    """Chunks closing long sequences take the key-range split (a workspace is allocated); with a one-byte
    workspace the same call runs unsplit. Both match the oracle, and each other within rounding; a sequence whose
    chunk is all of it leaves later splits empty (their lse is -inf and they carry no weight)."""
    p = W.paged_prefill_inputs(64, len(lens), 8, 2, D, Nq, 16, Nq, max(lens), seq_lens=np.array(lens))
    c = p.cache
    args = (dev_bf16(p.q), dev_bf16(c.k_cache), dev_bf16(c.v_cache), dev_i32(c.block_table), dev_i32(c.seq_lens))
    q_dev = args[0]
    need = lib.prefill_paged_workspace_bytes(q_dev, args[1], args[3])
    assert need > 0, "this shape is meant to take the split"
    o_split, l_split = lib.prefill_paged(*args, scale=p.scale)
    tiny = torch.empty(1, dtype=torch.uint8, device=q_dev.device)
    o_one, l_one = lib.prefill_paged(*args, scale=p.scale, workspace=tiny)
    torch.cuda.synchronize()
    Oref, Lref = A.paged_prefill(W.f64_from_bf16_bits(p.q), W.f64_from_bf16_bits(c.k_cache),
                                 W.f64_from_bf16_bits(c.v_cache), c.block_table, c.seq_lens,
                                 float(np.float32(p.scale)))
    for o, l, tag in ((o_split, l_split, "split"), (o_one, l_one, "unsplit")):
        eo, el = max_err(host64(o), Oref), max_err(host64(l), Lref)
        say(f"[paged prefill] {tag} D{D} Nq{Nq} L{lens}: max|dO|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= BF16_TOL and el <= LSE_TOL
    assert (o_split.float() - o_one.float()).abs().max().item() <= BF16_TOL


def test_one_token_chunk_matches_decode_kernel(lib):
    """A one-token chunk is a decode step: the paged prefill and the split-KV decode kernel agree within rounding."""
    p = W.paged_prefill_inputs(65, 4, 16, 2, 64, 1, 16, 1, 3000, seq_lens=np.array([1, 16, 1500, 3000]))
    c = p.cache
    o, lse = run(lib, p)
    od, ld = lib.decode_paged(dev_bf16(p.q[:, :, 0]), dev_bf16(c.k_cache), dev_bf16(c.v_cache), dev_i32(c.block_table),
                              dev_i32(c.seq_lens), 3000, scale=p.scale)
    torch.cuda.synchronize()
    assert (o[:, :, 0].float() - od.float()).abs().max().item() <= BF16_TOL
    assert (lse[:, :, 0] - ld).abs().max().item() <= LSE_TOL


def test_sequence_filling_its_block_table(lib):
    """seq_len equal to max_pages_per_seq * page_size: the last page is full and the table has no spare entry."""
    p = W.paged_prefill_inputs(66, 1, 8, 2, 128, 96, 16, 1024, 1024)
    assert p.cache.block_table.shape[1] * 16 == 1024 and int(p.cache.seq_lens[0]) == 1024
    compare(lib, p, "full block table")
