"""The C ABI without a GPU: the library loads, exports what include/lcattn.h declares, sizes workspaces, and
rejects bad arguments on the host before enqueueing anything. No call here reaches a kernel launch: every
argument set is invalid, or the problem is empty."""
import ctypes
import math
import os
import re

import pytest

import long_context_attention_causal_amd as lca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcattn.h")
FAKE = 1 << 20          # aligned, non-null, never dereferenced: validation fails before any launch
MISALIGNED = FAKE + 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lca.LIB_PATH):
        from long_context_attention_causal_amd import build
        build.build(verbose=False)
    return lca.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:attn_status_t|size_t|const char\*|int32_t)\s+(attn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(L):
    decl = declared_functions()
    assert len(decl) == 14
    for name in decl:
        assert hasattr(L, name), name
    assert set(decl) == set(lca.EXPORTS)


def test_version_and_status_strings(L):
    assert lca.abi_version() == 7
    for st in range(7):
        assert L.attn_status_string(st)
    assert L.attn_status_string(99) == b"unknown status"


def shape(B=1, Hq=4, Hkv=2, N=128, D=128, scale=0.1, dtype=0):
    return lca.AttnShape(B, Hq, Hkv, N, D, scale, dtype)


def dense(L, s, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None):
    return L.attn_prefill_dense(ctypes.byref(s) if s is not None else None, q, k, v, o, lse, None)


@pytest.mark.parametrize("s,code", [
    (None, 1),
    (shape(Hq=3, Hkv=2), 2),
    (shape(D=96), 3),
    (shape(scale=0.0), 2),
    (shape(scale=math.inf), 2),
    (shape(dtype=7), 3),
    (shape(B=0), 2),
    (shape(N=-1), 2),
])
def test_prefill_dense_rejects(L, s, code):
    assert dense(L, s) == code
    assert L.attn_last_error()


@pytest.mark.parametrize("N,D,dtype,code", [
    (1 << 24, 128, 0, 3),          # 4 GiB per head: refused before any launch
    ((1 << 23), 128, 0, 3),        # exactly 2^31 bytes
    ((1 << 23) - 64, 128, 0, 1),   # accepted shape: the call then stops at the NULL q pointer
    ((1 << 24) - 64, 64, 0, 1),
    (1 << 24, 64, 0, 3),
    ((1 << 22), 128, 1, 3),        # fp32: 4 bytes per element
    ((1 << 22) - 64, 128, 1, 1),
])
def test_prefill_rejects_unaddressable_lengths(L, N, D, dtype, code):
    """A per-head K/V slab of 2^31 bytes or more cannot be addressed by the kernels' 32-bit buffer views; such a
    shape is refused with ATTN_ERR_UNSUPPORTED by every prefill-like entry point. An accepted shape is shown by the
    next check failing instead (q is NULL), so no kernel is launched."""
    s = shape(B=1, Hq=1, Hkv=1, N=N, D=D, dtype=dtype)
    assert dense(L, s, q=None) == code
    if code == 3:
        assert b"2^31" in L.attn_last_error()
    if dtype == 0 and code == 3:
        # the shape check comes before the sparse path's own block-count limit
        assert L.attn_prefill_block_sparse(ctypes.byref(s), 256, None, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                           None) == 3
        assert b"2^31" in L.attn_last_error()
    if dtype == 0:
        p = params(block=2048)
        ws = L.attn_block_mask_workspace_bytes(ctypes.byref(s), ctypes.byref(p))
        assert (ws == 0) if code == 3 else (ws > 0 or N % 2048)


def test_prefill_dense_pointer_checks(L):
    assert dense(L, shape(), q=None) == 1
    assert dense(L, shape(), v=MISALIGNED) == 4
    assert dense(L, shape(), lse=MISALIGNED) == 4
    assert dense(L, shape(N=0), q=None) == 0      # empty problem: nothing to do, nothing read


def params(block=64, keep=100, alpha=1.0, lo=50, hi=90, mode=0):
    return lca.AttnMaskParams(block, keep, alpha, lo, hi, mode)


@pytest.mark.parametrize("s,p,code", [
    (shape(dtype=1), params(), 3),
    (shape(N=100), params(), 2),
    (shape(), params(block=32), 3),
    (shape(), params(keep=1001), 2),
    (shape(), params(alpha=-1.0), 2),
    (shape(), params(alpha=math.nan), 2),
    (shape(), params(lo=90, hi=50), 2),
    (shape(N=64 * 5000), params(), 3),
    (shape(), params(mode=2), 2),
    (shape(), params(mode=-1), 2),
])
def test_mask_build_rejects(L, s, p, code):
    assert L.attn_block_mask_workspace_bytes(ctypes.byref(s), ctypes.byref(p)) == 0
    assert L.attn_block_mask_build(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   1 << 40, None) == code


def test_mask_workspace_size_and_check(L):
    B, Hq, Hkv, N, D, blk = 2, 8, 2, 512, 128, 64
    nb = N // blk
    s, p = shape(B, Hq, Hkv, N, D), params(blk)
    need = L.attn_block_mask_workspace_bytes(ctypes.byref(s), ctypes.byref(p))
    # the query-aware rescue reads only buffers the workspace already holds
    assert L.attn_block_mask_workspace_bytes(ctypes.byref(s), ctypes.byref(params(blk, mode=1))) == need
    assert ctypes.sizeof(lca.AttnMaskParams) == 32
    a = lambda x: (x + 255) // 256 * 256
    want = (a(B * Hq * nb * D * 8) + a(B * Hkv * nb * D * 8) + a(B * Hkv * nb * 8) + a(B * Hkv * 32)
            + a(B * Hkv * nb) + a(B * Hq * nb * nb * 8))
    assert need == want
    assert L.attn_block_mask_build(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   need - 1, None) == 5
    assert L.attn_block_mask_build(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                   need, None) == 5
    assert L.attn_block_mask_build(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   FAKE + 16, need, None) == 4
    assert L.attn_block_mask_build(ctypes.byref(s), ctypes.byref(p), FAKE, None, FAKE, FAKE, FAKE, None, FAKE,
                                   need, None) == 1


@pytest.mark.parametrize("blk,N,code", [(32, 128, 3), (64, 100, 2), (512, 1024, 3), (64, 64 * 4097, 3)])
def test_sparse_rejects(L, blk, N, code):
    s = shape(N=N)
    assert L.attn_prefill_block_sparse(ctypes.byref(s), blk, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == code


def test_sparse_pointer_checks(L):
    s = shape()
    assert L.attn_prefill_block_sparse(ctypes.byref(s), 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None) == 1
    assert L.attn_prefill_block_sparse(ctypes.byref(s), 64, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, None,
                                       None) == 4
    fp32 = shape(dtype=1)
    assert L.attn_prefill_block_sparse(ctypes.byref(fp32), 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 3


def dshape(B=4, Hq=16, Hkv=2, D=64, page=16, maxp=64, pages=100, chunk=512, scale=0.125):
    return lca.AttnDecodeShape(B, Hq, Hkv, D, page, maxp, pages, chunk, scale)


@pytest.mark.parametrize("s,maxlen,code", [
    (dshape(Hq=15), 100, 2),
    (dshape(Hq=64, Hkv=2), 100, 3),
    (dshape(D=80), 100, 3),
    (dshape(page=32), 100, 3),
    (dshape(chunk=500), 100, 3),
    (dshape(), 64 * 16 + 1, 2),
    (dshape(), -1, 2),
    (dshape(scale=-1.0), 100, 2),
    (dshape(pages=0), 100, 2),
    (dshape(B=65536), 100, 3),
    (dshape(Hq=4096, Hkv=4096, chunk=64, maxp=300000), 4097 * 64, 3),
    (dshape(Hq=16 * 4097, Hkv=4097), 100, 3),
])
def test_decode_rejects(L, s, maxlen, code):
    assert L.attn_decode_paged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, maxlen, FAKE, None, FAKE, 1 << 40,
                               None) == code


def decode8(L, s, maxlen, ks=1.0, vs=1.0, ws=1 << 40, k=FAKE, bt=FAKE, wsp=FAKE):
    return L.attn_decode_paged_fp8(ctypes.byref(s), FAKE, k, FAKE, ks, vs, bt, FAKE, maxlen, FAKE, None, wsp, ws, None)


@pytest.mark.parametrize("s,maxlen,ks,vs,code", [
    (dshape(), 100, 0.0, 1.0, 2),
    (dshape(), 100, 1.0, -1.0, 2),
    (dshape(), 100, math.nan, 1.0, 2),
    (dshape(), 100, 1.0, math.inf, 2),
    (dshape(Hq=15), 100, 1.0, 1.0, 2),
    (dshape(D=80), 100, 1.0, 1.0, 3),
    (dshape(page=32), 100, 1.0, 1.0, 3),
    (dshape(), 64 * 16 + 1, 1.0, 1.0, 2),
])
def test_decode_fp8_rejects(L, s, maxlen, ks, vs, code):
    assert decode8(L, s, maxlen, ks, vs) == code
    assert L.attn_last_error()


def test_decode_fp8_checks_like_bf16(L):
    s = dshape()
    need = L.attn_decode_workspace_bytes(ctypes.byref(s), 1000)
    assert decode8(L, s, 1000, ws=need - 1) == 5
    assert decode8(L, s, 1000, ws=need, wsp=FAKE + 64) == 4
    assert decode8(L, s, 1000, ws=need, bt=None) == 1
    assert decode8(L, s, 1000, ws=need, k=None) == 1


def test_decode_workspace(L):
    s = dshape()
    need = L.attn_decode_workspace_bytes(ctypes.byref(s), 1000)
    C = -(-1000 // 512)
    a = lambda x: (x + 255) // 256 * 256
    assert need == a(4 * 16 * C * 64 * 4) + a(4 * 16 * C * 4)
    assert L.attn_decode_paged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 1000, FAKE, None, FAKE, need - 1,
                               None) == 5
    assert L.attn_decode_paged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, 1000, FAKE, None, FAKE + 64, need,
                               None) == 4
    assert L.attn_decode_paged(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, 1000, FAKE, None, FAKE, need,
                               None) == 1
    assert L.attn_decode_workspace_bytes(ctypes.byref(dshape(page=8)), 1000) == 0


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(lca.LcattnError):
        lca.prefill_dense(q, q[:, :1].contiguous(), q[:, :1].contiguous())


def pshape(B=2, Hq=8, Hkv=2, D=128, Nq=100, page=16, maxp=64, pages=200, window=0, scale=0.1):
    return lca.AttnPagedPrefillShape(B, Hq, Hkv, D, Nq, page, maxp, pages, window, scale)


@pytest.mark.parametrize("s,code", [
    (pshape(Hq=7), 2),
    (pshape(D=96), 3),
    (pshape(page=32), 3),
    (pshape(window=-1), 2),
    (pshape(Nq=-1), 2),
    (pshape(scale=0.0), 2),
    (pshape(Nq=64 * 16 + 1), 2),
    (pshape(pages=0), 2),
])
def test_prefill_paged_rejects(L, s, code):
    assert L.attn_prefill_paged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == code
    assert L.attn_last_error()


def test_prefill_paged_pointer_checks(L):
    s = pshape()
    assert L.attn_prefill_paged(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == 1
    assert L.attn_prefill_paged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, None, 0, None) == 4
    assert L.attn_prefill_paged(ctypes.byref(pshape(Nq=0)), None, None, None, None, None, None, None, None, 0,
                                None) == 0


def test_prefill_paged_workspace_policy(L):
    """A chunk closing a long sequence is split (its work-groups are too few and too even); a whole short
    sequence or a windowed chunk is not; the workspace holds the fp32 partials and their lse."""
    long_chunk = pshape(B=1, Hq=32, Hkv=4, D=128, Nq=4096, maxp=2048, pages=2048)
    need = L.attn_prefill_paged_workspace_bytes(ctypes.byref(long_chunk))
    assert need > 0 and need % (1 * 32 * 4096 * 129 * 4) == 0
    assert L.attn_prefill_paged_workspace_bytes(ctypes.byref(pshape(Nq=4096, maxp=256, pages=256))) == 0
    windowed = pshape(B=8, Hq=64, Hkv=8, D=64, Nq=2048, maxp=1024, pages=8000, window=128)
    assert L.attn_prefill_paged_workspace_bytes(ctypes.byref(windowed)) == 0
    assert L.attn_prefill_paged_workspace_bytes(ctypes.byref(pshape(D=96))) == 0


def test_mask_build_fp8k_checks(L):
    s, p = shape(), params()
    need = L.attn_block_mask_workspace_bytes(ctypes.byref(s), ctypes.byref(p))
    call = lambda ks, k=FAKE, ws=need: L.attn_block_mask_build_fp8k(ctypes.byref(s), ctypes.byref(p), FAKE, k, ks,
                                                                    FAKE, FAKE, FAKE, None, FAKE, ws, None)
    assert call(0.0) == 2 and call(math.nan) == 2 and call(-1.0) == 2
    assert call(1.0, k=None) == 1
    assert call(1.0, k=MISALIGNED) == 4
    assert call(1.0, ws=need - 1) == 5


def test_decode_noalloc_rejects_before_touching_the_device(L):
    """The entry point without a workspace validates like attn_decode_paged, and refuses shapes whose partials
    exceed the library's fixed per-GPU scratch, all on the host (no GPU here, so any device call would fail)."""
    assert lca.DECODE_SCRATCH_BYTES == 64 << 20
    noalloc = lambda s, maxlen, q=FAKE, o=FAKE: L.attn_decode_paged_noalloc(
        ctypes.byref(s) if s is not None else None, q, FAKE, FAKE, FAKE, FAKE, maxlen, o, None, None)
    assert noalloc(None, 1000) == 1
    assert noalloc(dshape(page=8), 1000) == 3
    assert noalloc(dshape(), 1000, q=None) == 1
    assert noalloc(dshape(), 1000, o=MISALIGNED) == 4
    # B=32, Hq=64, D=64, 512-token chunks, lengths up to 32768: 32 * 64 * 64 chunks * 64 * 4 B = 32 MiB fits
    big = dshape(B=32, Hq=64, Hkv=8, D=64, maxp=2048, pages=100)
    need = L.attn_decode_workspace_bytes(ctypes.byref(big), 32768)
    assert 0 < need <= lca.DECODE_SCRATCH_BYTES
    assert noalloc(big, 32768, q=None) == 1      # the shape is accepted; the NULL q is what stops it
    # twice the length needs more than the scratch holds
    bigger = dshape(B=32, Hq=64, Hkv=8, D=64, maxp=8192, pages=100)
    assert L.attn_decode_workspace_bytes(ctypes.byref(bigger), 131072) > lca.DECODE_SCRATCH_BYTES
    assert noalloc(bigger, 131072) == 5
    assert b"scratch" in L.attn_last_error()
