"""MI355X-native long-context causal attention: Python binding of liblcattn.so (include/lcattn.h).

Argument marshalling only. Every step of the computation runs in the library's HIP kernels; PyTorch supplies
device memory and the current stream. There is no fallback: if the library is missing or cannot be loaded, every
call raises LcattnError.

    import long_context_attention_causal_amd as lca
    o, lse = lca.prefill_dense(q, k, v)                         # dense causal GQA prefill
    m = lca.block_mask_build(q, k, block_size=64, keep_permille=100, rescue_alpha=1.0)
    o, _ = lca.prefill_block_sparse(q, k, v, m.kv_count, m.kv_index, block_size=64)
    o, lse = lca.decode_paged(q1, k_cache, v_cache, block_table, seq_lens, max_seq_len)
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch  # imported before the library so both bind the same HIP runtime (shared SONAME)

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, unless LCATTN_LIB names another build of the same library (e.g. a sanitizer build)
LIB_PATH = os.environ.get("LCATTN_LIB") or os.path.join(_HERE, "liblcattn.so")

ATTN_BF16, ATTN_FP32 = 0, 1
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
                4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP"}


class LcattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class AttnMaskParams(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("keep_permille", ctypes.c_int32),
                ("rescue_alpha", ctypes.c_double), ("q_lo_pct", ctypes.c_int32), ("q_hi_pct", ctypes.c_int32),
                ("rescue_mode", ctypes.c_int32)]


class AttnPagedPrefillShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("q_len", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("window", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class AttnDecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("chunk_tokens", ctypes.c_int32), ("scale", ctypes.c_float)]


EXPORTS = ("attn_prefill_dense", "attn_block_mask_workspace_bytes", "attn_block_mask_build",
           "attn_block_mask_build_fp8k",
           "attn_prefill_block_sparse", "attn_prefill_paged", "attn_prefill_paged_workspace_bytes",
           "attn_decode_workspace_bytes", "attn_decode_paged",
           "attn_decode_paged_fp8", "attn_decode_paged_noalloc", "attn_status_string", "attn_last_error",
           "attn_abi_version")
DECODE_SCRATCH_BYTES = 64 << 20   # LCATTN_DECODE_SCRATCH_BYTES

_lib: Optional[ctypes.CDLL] = None


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    except OSError:
        return []


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load liblcattn.so (built in-tree by `python -m long_context_attention_causal_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise LcattnError(6, f"{p} is not built; run python -m long_context_attention_causal_amd.build")
    lib = ctypes.CDLL(p)
    vp, i32, f32p, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_size_t
    lib.attn_abi_version.restype = i32
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i32]
    lib.attn_prefill_dense.restype = i32
    lib.attn_prefill_dense.argtypes = [ctypes.POINTER(AttnShape), vp, vp, vp, vp, vp, vp]
    lib.attn_block_mask_workspace_bytes.restype = sz
    lib.attn_block_mask_workspace_bytes.argtypes = [ctypes.POINTER(AttnShape), ctypes.POINTER(AttnMaskParams)]
    lib.attn_block_mask_build.restype = i32
    lib.attn_block_mask_build.argtypes = [ctypes.POINTER(AttnShape), ctypes.POINTER(AttnMaskParams), vp, vp, vp, vp,
                                          vp, vp, vp, sz, vp]
    lib.attn_block_mask_build_fp8k.restype = i32
    lib.attn_block_mask_build_fp8k.argtypes = [ctypes.POINTER(AttnShape), ctypes.POINTER(AttnMaskParams), vp, vp,
                                               ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.attn_prefill_block_sparse.restype = i32
    lib.attn_prefill_block_sparse.argtypes = [ctypes.POINTER(AttnShape), i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.attn_prefill_paged.restype = i32
    lib.attn_prefill_paged.argtypes = [ctypes.POINTER(AttnPagedPrefillShape), vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                       vp]
    lib.attn_prefill_paged_workspace_bytes.restype = sz
    lib.attn_prefill_paged_workspace_bytes.argtypes = [ctypes.POINTER(AttnPagedPrefillShape)]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(AttnDecodeShape), i32]
    lib.attn_decode_paged.restype = i32
    lib.attn_decode_paged.argtypes = [ctypes.POINTER(AttnDecodeShape), vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.attn_decode_paged_noalloc.restype = i32
    lib.attn_decode_paged_noalloc.argtypes = [ctypes.POINTER(AttnDecodeShape), vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.attn_decode_paged_fp8.restype = i32
    lib.attn_decode_paged_fp8.argtypes = [ctypes.POINTER(AttnDecodeShape), vp, vp, vp, ctypes.c_float,
                                          ctypes.c_float, vp, vp, i32, vp, vp, vp, sz, vp]
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise LcattnError(6, f"two HIP runtimes mapped in this process: {runtimes}")
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load().attn_abi_version())


def _check(status: int) -> None:
    if status != 0:
        raise LcattnError(status, load().attn_last_error().decode(errors="replace"))


def _stream(stream, device: torch.device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else None)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise LcattnError(1, f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise LcattnError(2, f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise LcattnError(2, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise LcattnError(3, f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise LcattnError(2, f"{name} must have {ndim} dims")


def _like(t: torch.Tensor, name: str, shape, dtype, device: torch.device) -> None:
    """A caller-supplied output or workspace must match exactly: the library gets plain pointers and trusts sizes."""
    _need(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise LcattnError(2, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise LcattnError(2, f"{name} is on {t.device}, the inputs on {device}")


def _same_device(device: torch.device, *named) -> None:
    for t, n in named:
        if t.device != device:
            raise LcattnError(2, f"{n} is on {t.device}, q on {device}")


def _prefill_shape(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float]) -> AttnShape:
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise LcattnError(3, "q must be bf16 or fp32")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype, 4)
    B, Hq, N, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != D:
        raise LcattnError(2, f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    _same_device(q.device, (k, "k"), (v, "v"))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return AttnShape(B, Hq, k.shape[1], N, D, sc, ATTN_BF16 if q.dtype == torch.bfloat16 else ATTN_FP32)


def prefill_dense(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Causal GQA prefill. q [B,Hq,N,D], k/v [B,Hkv,N,D] (bf16 or fp32). Returns (o, lse or None)."""
    lib = load()
    shp = _prefill_shape(q, k, v, scale)
    o = torch.empty_like(q) if out is None else out
    _like(o, "out", q.shape, q.dtype, q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_prefill_dense(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _stream(stream, q.device)))
    return o, lse


@dataclass
class BlockMask:
    mask: torch.Tensor          # uint8 [B,Hq,nb,nb]
    kv_count: torch.Tensor      # int32 [B,Hq,nb]
    kv_index: torch.Tensor      # int32 [B,Hq,nb,nb]; entries past kv_count unspecified
    radius_stats: Optional[torch.Tensor]  # float64 [B,Hkv,nb+3]: radii, med, p_hi, tau
    workspace: torch.Tensor


def block_mask_workspace_bytes(q: torch.Tensor, k: torch.Tensor, block_size: int, keep_permille: int,
                               rescue_alpha: float, q_lo_pct: int = 50, q_hi_pct: int = 90,
                               scale: Optional[float] = None, rescue_mode: int = 0) -> int:
    shp = _prefill_shape(q, k, k, scale)
    prm = AttnMaskParams(block_size, keep_permille, float(rescue_alpha), q_lo_pct, q_hi_pct, rescue_mode)
    return int(load().attn_block_mask_workspace_bytes(ctypes.byref(shp), ctypes.byref(prm)))


def block_mask_build(q: torch.Tensor, k: torch.Tensor, block_size: int, keep_permille: int, rescue_alpha: float,
                     q_lo_pct: int = 50, q_hi_pct: int = 90, scale: Optional[float] = None,
                     want_radius_stats: bool = True, workspace: Optional[torch.Tensor] = None,
                     outputs: Optional[BlockMask] = None, stream=None, rescue_mode: int = 0,
                     k_scale: Optional[float] = None) -> BlockMask:
    """The centroid + radius-rescue block mask. Returns the mask, CSR lists and optional stats.
    rescue_mode 0 rescues a flagged block in every row; 1 keeps it only in rows whose centroid cutoff its
    score plus the radius allowance beats. q is bf16; k is bf16, or E4M3 codes (uint8) with k_scale."""
    lib = load()
    fp8k = k.dtype == torch.uint8
    if fp8k and k_scale is None:
        raise LcattnError(2, "fp8 key codes need k_scale")
    if fp8k:
        _need(q, "q", torch.bfloat16, 4)
        _need(k, "k", torch.uint8, 4)
        if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]:
            raise LcattnError(2, "k codes must be [B, Hkv, N, D] matching q")
        _same_device(q.device, (k, "k"))
        Dq = q.shape[3]
        shp = AttnShape(q.shape[0], q.shape[1], k.shape[1], q.shape[2], Dq,
                        1.0 / math.sqrt(Dq) if scale is None else float(scale), ATTN_BF16)
    else:
        shp = _prefill_shape(q, k, k, scale)
    prm = AttnMaskParams(block_size, keep_permille, float(rescue_alpha), q_lo_pct, q_hi_pct, rescue_mode)
    need = int(lib.attn_block_mask_workspace_bytes(ctypes.byref(shp), ctypes.byref(prm)))
    if need == 0:   # the library rejects these parameters; this call reports why
        _check(lib.attn_block_mask_build(ctypes.byref(shp), ctypes.byref(prm), _ptr(q), _ptr(k), None, None, None,
                                         None, None, 0, _stream(stream, q.device)))
    B, Hq, N, _ = q.shape
    Hkv = k.shape[1]
    nb = N // block_size
    dev = q.device
    if outputs is None:
        ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
        outputs = BlockMask(mask=torch.empty((B, Hq, nb, nb), dtype=torch.uint8, device=dev),
                            kv_count=torch.empty((B, Hq, nb), dtype=torch.int32, device=dev),
                            kv_index=torch.empty((B, Hq, nb, nb), dtype=torch.int32, device=dev),
                            radius_stats=(torch.empty((B, Hkv, nb + 3), dtype=torch.float64, device=dev)
                                          if want_radius_stats else None),
                            workspace=ws)
    _like(outputs.mask, "mask", (B, Hq, nb, nb), torch.uint8, dev)
    _like(outputs.kv_count, "kv_count", (B, Hq, nb), torch.int32, dev)
    _like(outputs.kv_index, "kv_index", (B, Hq, nb, nb), torch.int32, dev)
    if outputs.radius_stats is not None:
        _like(outputs.radius_stats, "radius_stats", (B, Hkv, nb + 3), torch.float64, dev)
    _need(outputs.workspace, "workspace", torch.uint8)
    _same_device(dev, (outputs.workspace, "workspace"))
    if fp8k:
        _check(lib.attn_block_mask_build_fp8k(ctypes.byref(shp), ctypes.byref(prm), _ptr(q), _ptr(k), float(k_scale),
                                              _ptr(outputs.mask), _ptr(outputs.kv_count), _ptr(outputs.kv_index),
                                              _ptr(outputs.radius_stats), _ptr(outputs.workspace),
                                              outputs.workspace.numel(), _stream(stream, dev)))
        return outputs
    _check(lib.attn_block_mask_build(ctypes.byref(shp), ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(outputs.mask),
                                     _ptr(outputs.kv_count), _ptr(outputs.kv_index), _ptr(outputs.radius_stats),
                                     _ptr(outputs.workspace), outputs.workspace.numel(), _stream(stream, dev)))
    return outputs


def prefill_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_count: torch.Tensor,
                         kv_index: torch.Tensor, block_size: int, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, return_lse: bool = True, stream=None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Causal prefill over the kept key blocks of each query block (bf16)."""
    lib = load()
    shp = _prefill_shape(q, k, v, scale)
    B, Hq, N, _ = q.shape
    nb = N // block_size if block_size > 0 else 0
    _need(kv_count, "kv_count", torch.int32)
    _need(kv_index, "kv_index", torch.int32)
    if tuple(kv_count.shape) != (B, Hq, nb) or tuple(kv_index.shape) != (B, Hq, nb, nb):
        raise LcattnError(2, "kv_count/kv_index shapes do not match q and block_size")
    _same_device(q.device, (kv_count, "kv_count"), (kv_index, "kv_index"))
    o = torch.empty_like(q) if out is None else out
    _like(o, "out", q.shape, q.dtype, q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_prefill_block_sparse(ctypes.byref(shp), int(block_size), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(kv_count), _ptr(kv_index), _ptr(o), _ptr(lse),
                                         _stream(stream, q.device)))
    return o, lse


def _decode_shape(q, k_cache, block_table, chunk_tokens, scale) -> AttnDecodeShape:
    B, Hq, D = q.shape
    P, Hkv, page, D2 = k_cache.shape
    if D2 != D:
        raise LcattnError(2, "head_dim of q and cache differ")
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return AttnDecodeShape(B, Hq, Hkv, D, page, block_table.shape[1], P, chunk_tokens, sc)


def decode_workspace_bytes(q, k_cache, block_table, max_seq_len: int, chunk_tokens: int = 512,
                           scale: Optional[float] = None) -> int:
    shp = _decode_shape(q, k_cache, block_table, chunk_tokens, scale)
    return int(load().attn_decode_workspace_bytes(ctypes.byref(shp), int(max_seq_len)))


def decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, max_seq_len: int, chunk_tokens: int = 512, scale: Optional[float] = None,
                 out: Optional[torch.Tensor] = None, return_lse: bool = True,
                 workspace: Optional[torch.Tensor] = None, stream=None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV decode over a paged bf16 KV cache. q [B,Hq,D]; caches [pages,Hkv,16,D]."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise LcattnError(2, "k_cache and v_cache shapes differ")
    if block_table.shape[0] != q.shape[0] or seq_lens.shape[0] != q.shape[0]:
        raise LcattnError(2, "block_table and seq_lens need one row per sequence of q")
    _same_device(q.device, (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"))
    shp = _decode_shape(q, k_cache, block_table, chunk_tokens, scale)
    need = int(lib.attn_decode_workspace_bytes(ctypes.byref(shp), int(max_seq_len)))
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(ws, "workspace", torch.uint8)
    _same_device(q.device, (ws, "workspace"))
    o = torch.empty_like(q) if out is None else out
    _like(o, "out", q.shape, torch.bfloat16, q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_decode_paged(ctypes.byref(shp), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                 _ptr(seq_lens), int(max_seq_len), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                 _stream(stream, q.device)))
    return o, lse


def decode_paged_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, chunk_tokens: int = 512,
                         scale: Optional[float] = None, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         stream=None) -> None:
    """decode_paged through the entry point that allocates nothing: the chunk partials live in the library's own
    per-GPU scratch. `out` (and `lse`, when wanted) must be given; nothing is allocated here either."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise LcattnError(2, "k_cache and v_cache shapes differ")
    if block_table.shape[0] != q.shape[0] or seq_lens.shape[0] != q.shape[0]:
        raise LcattnError(2, "block_table and seq_lens need one row per sequence of q")
    if out is None:
        raise LcattnError(1, "out must be given (this entry point allocates nothing)")
    _like(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is not None:
        _like(lse, "lse", q.shape[:2], torch.float32, q.device)
    _same_device(q.device, (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"))
    shp = _decode_shape(q, k_cache, block_table, chunk_tokens, scale)
    _check(lib.attn_decode_paged_noalloc(ctypes.byref(shp), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                         _ptr(seq_lens), int(max_seq_len), _ptr(out), _ptr(lse),
                                         _stream(stream, q.device)))


def decode_paged_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache_t: torch.Tensor, k_scale: float,
                     v_scale: float, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                     chunk_tokens: int = 512, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     return_lse: bool = True, workspace: Optional[torch.Tensor] = None, stream=None
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV decode over a paged E4M3 KV cache (uint8 codes). q [B,Hq,D] bf16; k_cache [pages,Hkv,16,D];
    v_cache_t [pages,Hkv,D,16] (each page transposed); cached values are code value * scale."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.uint8, 4)
    _need(v_cache_t, "v_cache_t", torch.uint8, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    P, Hkv, page, D = k_cache.shape
    if tuple(v_cache_t.shape) != (P, Hkv, D, page):
        raise LcattnError(2, "v_cache_t must be [pages, Hkv, head_dim, page_size] for k_cache [pages, Hkv, page_size, "
                             "head_dim]")
    if block_table.shape[0] != q.shape[0] or seq_lens.shape[0] != q.shape[0]:
        raise LcattnError(2, "block_table and seq_lens need one row per sequence of q")
    _same_device(q.device, (k_cache, "k_cache"), (v_cache_t, "v_cache_t"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"))
    shp = _decode_shape(q, k_cache, block_table, chunk_tokens, scale)
    need = int(lib.attn_decode_workspace_bytes(ctypes.byref(shp), int(max_seq_len)))
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _need(ws, "workspace", torch.uint8)
    _same_device(q.device, (ws, "workspace"))
    o = torch.empty_like(q) if out is None else out
    _like(o, "out", q.shape, torch.bfloat16, q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if return_lse else None
    _check(lib.attn_decode_paged_fp8(ctypes.byref(shp), _ptr(q), _ptr(k_cache), _ptr(v_cache_t), float(k_scale),
                                     float(v_scale), _ptr(block_table), _ptr(seq_lens), int(max_seq_len), _ptr(o),
                                     _ptr(lse), _ptr(ws), ws.numel(), _stream(stream, q.device)))
    return o, lse


def prefill_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                  seq_lens: torch.Tensor, window: int = 0, scale: Optional[float] = None,
                  out: Optional[torch.Tensor] = None, return_lse: bool = True,
                  workspace: Optional[torch.Tensor] = None, stream=None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill over a paged bf16 cache. q [B,Hq,Nq,D]: the last Nq of each sequence's seq_lens[b] tokens
    (already in the cache [pages,Hkv,16,D]); window 0 = causal over the whole sequence, W > 0 = the W latest keys."""
    lib = load()
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if k_cache.shape != v_cache.shape:
        raise LcattnError(2, "k_cache and v_cache shapes differ")
    B, Hq, Nq, D = q.shape
    P, Hkv, page, D2 = k_cache.shape
    if D2 != D:
        raise LcattnError(2, "head_dim of q and cache differ")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise LcattnError(2, "block_table and seq_lens need one row per sequence of q")
    _same_device(q.device, (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"))
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    shp = AttnPagedPrefillShape(B, Hq, Hkv, D, Nq, page, block_table.shape[1], P, int(window), sc)
    o = torch.empty_like(q) if out is None else out
    _like(o, "out", q.shape, torch.bfloat16, q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if return_lse else None
    need = int(lib.attn_prefill_paged_workspace_bytes(ctypes.byref(shp)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
        _same_device(q.device, (workspace, "workspace"))
    _check(lib.attn_prefill_paged(ctypes.byref(shp), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                  _ptr(seq_lens), _ptr(o), _ptr(lse), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream(stream, q.device)))
    return o, lse


def prefill_paged_workspace_bytes(q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor,
                                  window: int = 0) -> int:
    B, Hq, Nq, D = q.shape
    P, Hkv, page, _ = k_cache.shape
    shp = AttnPagedPrefillShape(B, Hq, Hkv, D, Nq, page, block_table.shape[1], P, int(window), 1.0)
    return int(load().attn_prefill_paged_workspace_bytes(ctypes.byref(shp)))
