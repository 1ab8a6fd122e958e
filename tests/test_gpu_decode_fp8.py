"""GPU parity of attn_decode_paged_fp8 (E4M3 paged KV cache, value pages transposed) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests.gpu_util import BF16_TOL, LSE_TOL, dev_bf16, dev_i32, host64, max_err, say

pytestmark = pytest.mark.gpu


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def run(lib, d, chunk=512, max_len=None):
    ml = int(d.seq_lens.max()) if max_len is None else max_len
    o, lse = lib.decode_paged_fp8(dev_bf16(d.q), dev_u8(d.k_cache), dev_u8(d.v_cache_t), d.k_scale, d.v_scale,
                                  dev_i32(d.block_table), dev_i32(d.seq_lens), ml, chunk_tokens=chunk, scale=d.scale)
    torch.cuda.synchronize()
    return o, lse


def compare(lib, d, label, chunk=512):
    o, lse = run(lib, d, chunk)
    # the library takes the scales as float32
    Oref, Lref = A.paged_decode_fp8(W.f64_from_bf16_bits(d.q), d.k_cache, d.v_cache_t, float(np.float32(d.k_scale)),
                                    float(np.float32(d.v_scale)), d.block_table, d.seq_lens,
                                    float(np.float32(d.scale)))
    og, lg = host64(o), host64(lse)
    live = d.seq_lens > 0
    eo = max_err(og, Oref)
    el = max_err(lg[live], Lref[live])
    say(f"[decode fp8] {label} chunk={chunk} max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert np.isfinite(og).all()
    assert eo <= BF16_TOL and el <= LSE_TOL
    if (~live).any():
        assert (og[~live] == 0).all() and np.isneginf(lg[~live]).all()
    return o, lse


def test_c5_fp8_full(lib):
    w = W.WORKLOADS["c5_decode_paged_fp8"]
    say("[decode fp8] c5: generating inputs")
    d = W.make("c5_decode_paged_fp8")
    compare(lib, d, "c5 fp8", chunk=w["chunk"])


@pytest.mark.parametrize("lens,D,G", [
    ([1, 15, 16, 17, 511, 512, 513, 1000, 0, 2049], 64, 8),
    ([3, 64, 700, 1, 0, 128], 128, 4),
    ([129, 1030, 20], 64, 16),
    ([5000, 77], 128, 1),
])
def test_edges(lib, lens, D, G):
    Hkv = 2
    d = W.decode_inputs_fp8(41, len(lens), Hkv * G, Hkv, D, 16, 1, max(lens), seq_lens=np.array(lens))
    compare(lib, d, f"edges D={D} G={G}")


# chunk sizes that select every launch shape: one, two and four waves per work-group, both head dims
@pytest.mark.parametrize("chunk,D", [(64, 64), (128, 64), (1024, 64), (4096, 64), (64, 128), (512, 128), (1024, 128),
                                     (4096, 128)])
def test_split_sizes_agree_with_oracle(lib, chunk, D):
    d = W.decode_inputs_fp8(43, 6, 16, 2, D, 16, 1, 5000)
    compare(lib, d, f"split D={D}", chunk=chunk)


@pytest.mark.parametrize("ks,vs", [(0.0137, 0.021), (2.0 ** -3, 3.0), (1.0, 2.0 ** -9)])
def test_scales(lib, ks, vs):
    """Scales that are not powers of two (folded into the exponent scale and the final normalisation in fp32)."""
    d = W.decode_inputs_fp8(44, 5, 32, 4, 64, 16, 1, 3000, k_scale=ks, v_scale=vs)
    compare(lib, d, f"scales k={ks} v={vs}")


@pytest.mark.parametrize("tstar", [0, 15, 16, 511, 512, "last", "rand"])
def test_needle_is_element_exact(lib, tstar):
    """All keys zero except logical position t*, whose key (code 192, k_scale 8, q = e0, scale 1/8) scores 192 above
    every other; every other weight underflows to exactly 0 in fp32, so the output is V[t*] * v_scale bit for bit
    (v_scale is a power of two and every E4M3 value is a bf16 number). V[t*] is read from the transposed page."""
    n = 1300
    d = W.decode_inputs_fp8(45, 2, 16, 2, 64, 16, n, n, k_scale=8.0, v_scale=2.0 ** -6, seq_lens=np.array([n, 900]))
    t = {"last": n - 1, "rand": 777}.get(tstar, tstar)
    q = np.zeros_like(d.q)
    q[0, :, 0] = W.bf16_bits_from_f32(np.float32([1.0]))[0]
    kc = np.zeros_like(d.k_cache)
    pid = d.block_table[0, t // 16]
    kc[pid, :, t % 16, 0] = W.e4m3_codes_from_f32(np.float32([192.0]))[0]
    d2 = W.DecodeInputsFP8(q=q, k_cache=kc, v_cache_t=d.v_cache_t, k_scale=8.0, v_scale=d.v_scale,
                           block_table=d.block_table, seq_lens=d.seq_lens, page=16, scale=0.125)
    o, _ = run(lib, d2)
    vrow = torch.from_numpy(d.v_cache_t[pid, :, :, t % 16].copy()).view(torch.float8_e4m3fn).float() * d.v_scale
    want = vrow.to(torch.bfloat16)
    got = o[0].cpu()
    for h in range(16):
        assert torch.equal(got[h], want[h // 8]), (tstar, h)


def test_deterministic(lib):
    d = W.decode_inputs_fp8(46, 4, 64, 8, 64, 16, 1000, 9000)
    o1, l1 = run(lib, d)
    o2, l2 = run(lib, d)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_binding_rejects_mismatched_value_layout(lib):
    d = W.decode_inputs_fp8(47, 2, 16, 2, 64, 16, 10, 40)
    with pytest.raises(Exception):
        lib.decode_paged_fp8(dev_bf16(d.q), dev_u8(d.k_cache), dev_u8(d.k_cache), 1.0, 1.0, dev_i32(d.block_table),
                             dev_i32(d.seq_lens), 40)
