"""GPU parity of attn_decode_paged against the fp64 oracle, plus element-exact gather probes."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_util import BF16_TOL, LSE_TOL, dev_bf16, dev_i32, host64, max_err, say

pytestmark = pytest.mark.gpu


def to_dev(d: W.DecodeInputs):
    return (dev_bf16(d.q), dev_bf16(d.k_cache), dev_bf16(d.v_cache), dev_i32(d.block_table), dev_i32(d.seq_lens))


def oracle(d: W.DecodeInputs):
    return A.paged_decode(W.f64_from_bf16_bits(d.q), W.f64_from_bf16_bits(d.k_cache),
                          W.f64_from_bf16_bits(d.v_cache), d.block_table, d.seq_lens, d.scale)


def run(lib, d, chunk=512, max_len=None):
    q, kc, vc, bt, sl = to_dev(d)
    ml = int(d.seq_lens.max()) if max_len is None else max_len
    o, lse = lib.decode_paged(q, kc, vc, bt, sl, ml, chunk_tokens=chunk, scale=d.scale)
    torch.cuda.synchronize()
    return o, lse


def compare(lib, d, label, chunk=512):
    o, lse = run(lib, d, chunk)
    Oref, Lref = oracle(d)
    og, lg = host64(o), host64(lse)
    live = d.seq_lens > 0
    eo = max_err(og, Oref)
    el = max_err(lg[live], Lref[live])
    say(f"[decode] {label} chunk={chunk} max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert np.isfinite(og).all()
    assert eo <= BF16_TOL and el <= LSE_TOL
    if (~live).any():
        assert (og[~live] == 0).all() and np.isneginf(lg[~live]).all()
    return o, lse


def test_c5_full(lib):
    w = W.WORKLOADS["c5_decode_paged_bf16"]
    say("[decode] c5: generating inputs")
    d = W.make("c5_decode_paged_bf16")
    compare(lib, d, "c5", chunk=w["chunk"])


@pytest.mark.parametrize("lens,D,G", [
    ([1, 15, 16, 17, 511, 512, 513, 1000, 0, 2049], 64, 8),
    ([3, 64, 700, 1, 0, 128], 128, 4),
    ([129, 1030, 20], 64, 16),
    ([5000, 77], 128, 1),
])
def test_edges(lib, lens, D, G):
    Hkv = 2
    d = W.decode_inputs(31, len(lens), Hkv * G, Hkv, D, 16, 1, max(lens), seq_lens=np.array(lens))
    compare(lib, d, f"edges D={D} G={G}")


# chunk sizes that select every launch shape: one, two and four waves per work-group, both head dims
@pytest.mark.parametrize("chunk,D", [(64, 64), (128, 64), (1024, 64), (4096, 64), (64, 128), (512, 128), (1024, 128),
                                     (4096, 128)])
def test_split_sizes_agree_with_oracle(lib, chunk, D):
    d = W.decode_inputs(33, 6, 16, 2, D, 16, 1, 5000)
    compare(lib, d, f"split D={D}", chunk=chunk)


def test_split_vs_unsplit_on_gpu(lib):
    d = W.decode_inputs(34, 8, 64, 8, 64, 16, 100, 4096)
    o1, l1 = run(lib, d, 512, max_len=4096)
    o2, l2 = run(lib, d, 4096, max_len=4096)
    # each split rounds its probabilities to bf16 against its own chunk max (round to nearest: at most 2^-8
    # relative, bf16 keeping 8 significant bits), so each sum of rounded weights is within 2^-8 relative of the
    # exact one and its natural log within 2^-8 absolute; the two lse differ by at most 2 * 2^-8 = 7.8e-3 plus
    # fp32 noise, inside LSE_TOL = 1e-2
    assert (o1.float() - o2.float()).abs().max().item() <= BF16_TOL
    assert (l1 - l2).abs().max().item() <= LSE_TOL


@pytest.mark.parametrize("tstar", [0, 15, 16, 511, 512, "last", "rand"])
def test_needle_is_element_exact(lib, tstar):
    """All keys zero except logical position t*, whose key makes its score 200 above every other: every other
    weight underflows to exactly 0 in fp32, so the output must be V[t*] bit for bit."""
    n = 1300
    d = W.decode_inputs(35, 2, 16, 2, 64, 16, n, n, seq_lens=np.array([n, 900]))
    t = {"last": n - 1, "rand": 777}.get(tstar, tstar)
    q = np.zeros_like(d.q)
    one = W.bf16_bits_from_f32(np.float32([1.0]))[0]
    q[0, :, 0] = one
    kc = np.zeros_like(d.k_cache)
    pid = d.block_table[0, t // 16]
    big = W.bf16_bits_from_f32(np.float32([200.0 / d.scale]))[0]
    kc[pid, :, t % 16, 0] = big
    d2 = W.DecodeInputs(q=q, k_cache=kc, v_cache=d.v_cache, block_table=d.block_table, seq_lens=d.seq_lens,
                        page=16, scale=d.scale)
    o, _ = run(lib, d2)
    want = torch.from_numpy(d.v_cache[pid, :, t % 16, :].view(np.int16)).view(torch.bfloat16)
    got = o[0].cpu()
    for h in range(16):
        assert torch.equal(got[h], want[h // 8]), (tstar, h)


def test_deterministic(lib):
    d = W.decode_inputs(36, 4, 64, 8, 64, 16, 1000, 9000)
    o1, l1 = run(lib, d)
    o2, l2 = run(lib, d)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("fp8", [False, True])
def test_workspace_reuse_across_lengths(lib, fp8):
    """One workspace reused across calls whose sequences change length (single-chunk, empty and many-chunk
    sequences): the partials a call leaves behind never leak into the next call's result."""
    B, Hq, Hkv, D, chunk, maxlen = 6, 16, 2, 64, 256, 3000
    dev = torch.device("cuda", 0)
    shape_q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    shape_k = torch.empty(1, Hkv, 16, D, dtype=torch.bfloat16, device=dev)
    bt0 = torch.empty(B, -(-maxlen // 16), dtype=torch.int32, device=dev)
    ws = torch.empty(lib.decode_workspace_bytes(shape_q, shape_k, bt0, maxlen, chunk), dtype=torch.uint8, device=dev)
    for trial, lens in enumerate([[3000, 1, 256, 0, 257, 2999], [100, 3000, 0, 0, 1500, 255],
                                  [0, 0, 0, 0, 0, 0], [2048, 2048, 2048, 2048, 2048, 2048]]):
        seed = 60 + trial
        if fp8:
            d = W.decode_inputs_fp8(seed, B, Hq, Hkv, D, 16, 1, maxlen, 2.0 ** -6, 2.0 ** -6, seq_lens=np.array(lens))
            q, kc, vc = dev_bf16(d.q), torch.from_numpy(d.k_cache).cuda(), torch.from_numpy(d.v_cache_t).cuda()
            bt, sl = dev_i32(d.block_table), dev_i32(d.seq_lens)
            o, lse = lib.decode_paged_fp8(q, kc, vc, d.k_scale, d.v_scale, bt, sl, maxlen, chunk_tokens=chunk,
                                          scale=d.scale, workspace=ws)
            Oref, Lref = A.paged_decode_fp8(W.f64_from_bf16_bits(d.q), d.k_cache, d.v_cache_t, d.k_scale, d.v_scale,
                                            d.block_table, d.seq_lens, d.scale)
        else:
            d = W.decode_inputs(seed, B, Hq, Hkv, D, 16, 1, maxlen, seq_lens=np.array(lens))
            q, kc, vc, bt, sl = to_dev(d)
            o, lse = lib.decode_paged(q, kc, vc, bt, sl, maxlen, chunk_tokens=chunk, scale=d.scale, workspace=ws)
            Oref, Lref = oracle(d)
        torch.cuda.synchronize()
        og, lg = host64(o), host64(lse)
        live = d.seq_lens > 0
        say(f"[decode reuse] fp8={fp8} lens={lens} max|dO|={max_err(og, Oref):.3e}")
        assert max_err(og, Oref) <= BF16_TOL
        assert max_err(lg[live], Lref[live]) <= LSE_TOL
        assert (og[~live] == 0).all() and np.isneginf(lg[~live]).all()
