// The C ABI declared in include/lcattn.h: argument validation on the host, workspace sizing, and the kernel
// launches on the caller's stream. No allocation, no host<->device copies, no synchronisation.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/lcattn.h"
#include "internal.hpp"

static_assert(LCATTN_DECODE_SCRATCH_BYTES == lcattn::kDecodeScratchBytes, "header and library scratch sizes differ");

namespace {

thread_local std::string g_last_error;

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

attn_status_t ok() {
    g_last_error.clear();
    return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Checks common to every prefill-like call. `need_bf16` restricts the dtype.
attn_status_t check_prefill_shape(const attn_shape_t* s, bool need_bf16) {
    if (!s) return fail(ATTN_ERR_NULL, "shape is NULL");
    if (s->batch < 1 || s->heads_q < 1 || s->heads_kv < 1 || s->seq_len < 0)
        return fail(ATTN_ERR_SHAPE, "batch, heads_q, heads_kv must be >= 1 and seq_len >= 0");
    if (s->heads_q % s->heads_kv)
        return fail(ATTN_ERR_SHAPE, "heads_q (%d) must be a multiple of heads_kv (%d)", s->heads_q, s->heads_kv);
    if (s->head_dim != 64 && s->head_dim != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", s->head_dim);
    if (!(std::isfinite(s->scale) && s->scale > 0.0f)) return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
    if (s->dtype != ATTN_BF16 && s->dtype != ATTN_FP32) return fail(ATTN_ERR_UNSUPPORTED, "unknown dtype %d", s->dtype);
    if (need_bf16 && s->dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "this operation supports bf16 only");
    const double elems = (double)s->batch * s->heads_q * s->seq_len * s->head_dim;
    if (elems > 9.0e15) return fail(ATTN_ERR_SHAPE, "tensor too large");
    // the kernels address one head's K or V slab through a buffer view with a 32-bit signed byte extent
    const long long slab = (long long)s->seq_len * s->head_dim * (s->dtype == ATTN_FP32 ? 4 : 2);
    if (slab >= (1LL << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "seq_len %d x head_dim %d: a per-head K/V slab of %lld bytes exceeds 2^31 - 1",
                    s->seq_len, s->head_dim, slab);
    if ((double)s->batch * s->heads_q * ((s->seq_len + 31) / 32) >= 4294967295.0)
        return fail(ATTN_ERR_SHAPE, "grid too large");
    return ATTN_OK;
}

attn_status_t check_ptrs(std::initializer_list<const void*> req) {
    for (const void* p : req)
        if (!p) return fail(ATTN_ERR_NULL, "a required tensor pointer is NULL");
    for (const void* p : req)
        if (!aligned16(p)) return fail(ATTN_ERR_ALIGN, "tensor base pointers must be 16-byte aligned");
    return ATTN_OK;
}

lcattn::PrefillProblem to_problem(const attn_shape_t* s, const void* q, const void* k, const void* v, void* o,
                                  float* lse) {
    lcattn::PrefillProblem p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.B = s->batch;
    p.Hq = s->heads_q;
    p.Hkv = s->heads_kv;
    p.N = s->seq_len;
    p.D = s->head_dim;
    p.scale = s->scale;
    return p;
}

attn_status_t check_mask_params(const attn_shape_t* s, const attn_mask_params_t* m) {
    if (!m) return fail(ATTN_ERR_NULL, "mask params are NULL");
    if (m->block_size < 64 || m->block_size % 64)
        return fail(ATTN_ERR_UNSUPPORTED, "block_size %d must be a positive multiple of 64", m->block_size);
    if (s->seq_len % m->block_size) return fail(ATTN_ERR_SHAPE, "seq_len must be a multiple of block_size");
    const int nb = s->seq_len / m->block_size;
    if (nb < 1 || nb > 4096) return fail(ATTN_ERR_UNSUPPORTED, "block count %d outside 1..4096", nb);
    if (m->keep_permille < 0 || m->keep_permille > 1000) return fail(ATTN_ERR_SHAPE, "keep_permille outside 0..1000");
    if (std::isnan(m->rescue_alpha) || m->rescue_alpha < 0.0) return fail(ATTN_ERR_SHAPE, "rescue_alpha must be >= 0");
    if (m->q_lo_pct < 0 || m->q_hi_pct > 100 || m->q_lo_pct > m->q_hi_pct)
        return fail(ATTN_ERR_SHAPE, "need 0 <= q_lo_pct <= q_hi_pct <= 100");
    if (m->rescue_mode != 0 && m->rescue_mode != 1) return fail(ATTN_ERR_SHAPE, "rescue_mode must be 0 or 1");
    return ATTN_OK;
}

attn_status_t check_decode_shape(const attn_decode_shape_t* s, int32_t max_seq_len) {
    if (!s) return fail(ATTN_ERR_NULL, "shape is NULL");
    if (s->batch < 1 || s->heads_q < 1 || s->heads_kv < 1 || s->num_pages < 0 || s->max_pages_per_seq < 1)
        return fail(ATTN_ERR_SHAPE, "batch, heads, max_pages_per_seq must be >= 1 and num_pages >= 0");
    if (s->heads_q % s->heads_kv) return fail(ATTN_ERR_SHAPE, "heads_q must be a multiple of heads_kv");
    if (s->heads_q / s->heads_kv > 16) return fail(ATTN_ERR_UNSUPPORTED, "more than 16 query heads per kv head");
    if (s->heads_q > 65536) return fail(ATTN_ERR_UNSUPPORTED, "heads_q above 65536");
    if (s->batch > 65535) return fail(ATTN_ERR_UNSUPPORTED, "batch above 65535");
    if (s->head_dim != 64 && s->head_dim != 128) return fail(ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (s->page_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "page_size must be 16");
    if (s->chunk_tokens < 64 || s->chunk_tokens % 64 || s->chunk_tokens > 4096)
        return fail(ATTN_ERR_UNSUPPORTED, "chunk_tokens must be a multiple of 64 in [64, 4096]");
    if (!(std::isfinite(s->scale) && s->scale > 0.0f)) return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
    if (max_seq_len < 0) return fail(ATTN_ERR_SHAPE, "max_seq_len must be >= 0");
    if ((long long)max_seq_len > (long long)s->max_pages_per_seq * s->page_size)
        return fail(ATTN_ERR_SHAPE, "max_seq_len exceeds max_pages_per_seq * page_size");
    const long long chunks = ((long long)max_seq_len + s->chunk_tokens - 1) / s->chunk_tokens;
    if (chunks * s->heads_kv > 16777215LL) return fail(ATTN_ERR_UNSUPPORTED, "chunks * heads_kv above 16777215");
    return ATTN_OK;
}

}  // namespace

extern "C" {

int32_t attn_abi_version(void) { return LCATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_last_error.c_str(); }

const char* attn_status_string(attn_status_t st) {
    switch (st) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "null pointer";
        case ATTN_ERR_SHAPE: return "bad shape";
        case ATTN_ERR_UNSUPPORTED: return "unsupported";
        case ATTN_ERR_ALIGN: return "misaligned pointer";
        case ATTN_ERR_WORKSPACE: return "workspace too small";
        case ATTN_ERR_HIP: return "HIP runtime error";
        default: break;
    }
    return "unknown status";
}

attn_status_t attn_prefill_dense(const attn_shape_t* shape, const void* q, const void* k, const void* v, void* o,
                                 float* lse, void* stream) {
    attn_status_t st = check_prefill_shape(shape, false);
    if (st != ATTN_OK) return st;
    if (shape->seq_len == 0) return ok();
    if ((st = check_ptrs({q, k, v, o})) != ATTN_OK) return st;
    if (lse && !aligned16(lse)) return fail(ATTN_ERR_ALIGN, "lse must be 16-byte aligned");
    const lcattn::PrefillProblem p = to_problem(shape, q, k, v, o, lse);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (shape->dtype == ATTN_FP32) return hip_status(lcattn::launch_prefill_dense_f32(p, s), "attn_prefill_dense");
    return hip_status(lcattn::launch_prefill_dense_bf16(p, s), "attn_prefill_dense");
}

size_t attn_block_mask_workspace_bytes(const attn_shape_t* shape, const attn_mask_params_t* params) {
    if (check_prefill_shape(shape, true) != ATTN_OK || check_mask_params(shape, params) != ATTN_OK) return 0;
    const int nb = shape->seq_len / params->block_size;
    return lcattn::mask_workspace_layout(shape->batch, shape->heads_q, shape->heads_kv, nb, shape->head_dim, nullptr)
        .total;
}

namespace {

attn_status_t mask_build(const attn_shape_t* shape, const attn_mask_params_t* params, const void* q, const void* k,
                         const uint8_t* k8, double k_scale, uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                         double* radius_stats, void* workspace, size_t workspace_bytes, void* stream,
                         const char* what) {
    attn_status_t st = check_prefill_shape(shape, true);
    if (st != ATTN_OK) return st;
    if ((st = check_mask_params(shape, params)) != ATTN_OK) return st;
    if ((st = check_ptrs({q, k8 ? static_cast<const void*>(k8) : k, mask, kv_count, kv_index})) != ATTN_OK) return st;
    if (radius_stats && !aligned16(radius_stats)) return fail(ATTN_ERR_ALIGN, "radius_stats must be 16-byte aligned");
    const int nb = shape->seq_len / params->block_size;
    const lcattn::MaskWorkspace need = lcattn::mask_workspace_layout(shape->batch, shape->heads_q, shape->heads_kv,
                                                                     nb, shape->head_dim, nullptr);
    if (!workspace || workspace_bytes < need.total)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
    const lcattn::MaskWorkspace ws = lcattn::mask_workspace_layout(shape->batch, shape->heads_q, shape->heads_kv, nb,
                                                                   shape->head_dim, static_cast<char*>(workspace));
    lcattn::MaskProblem p;
    p.q = q;
    p.k = k;
    p.k8 = k8;
    p.k_scale = k_scale;
    p.B = shape->batch;
    p.Hq = shape->heads_q;
    p.Hkv = shape->heads_kv;
    p.N = shape->seq_len;
    p.D = shape->head_dim;
    p.block = params->block_size;
    p.nb = nb;
    p.scale = (double)shape->scale;
    p.keep_permille = params->keep_permille;
    p.alpha = params->rescue_alpha;
    p.lo_pct = params->q_lo_pct;
    p.hi_pct = params->q_hi_pct;
    p.rescue_mode = params->rescue_mode;
    p.mask = mask;
    p.kv_count = kv_count;
    p.kv_index = kv_index;
    p.radius_stats = radius_stats;
    return hip_status(lcattn::launch_block_mask(p, ws, static_cast<hipStream_t>(stream)), what);
}

}  // namespace

attn_status_t attn_block_mask_build(const attn_shape_t* shape, const attn_mask_params_t* params, const void* q,
                                    const void* k, uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                                    double* radius_stats, void* workspace, size_t workspace_bytes, void* stream) {
    return mask_build(shape, params, q, k, nullptr, 1.0, mask, kv_count, kv_index, radius_stats, workspace,
                      workspace_bytes, stream, "attn_block_mask_build");
}

attn_status_t attn_block_mask_build_fp8k(const attn_shape_t* shape, const attn_mask_params_t* params, const void* q,
                                         const uint8_t* k_codes, float k_scale, uint8_t* mask, int32_t* kv_count,
                                         int32_t* kv_index, double* radius_stats, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    if (!(std::isfinite(k_scale) && k_scale > 0.0f)) return fail(ATTN_ERR_SHAPE, "k_scale must be finite and > 0");
    if (!k_codes) return fail(ATTN_ERR_NULL, "k_codes is NULL");
    return mask_build(shape, params, q, nullptr, k_codes, (double)k_scale, mask, kv_count, kv_index, radius_stats,
                      workspace, workspace_bytes, stream, "attn_block_mask_build_fp8k");
}

attn_status_t attn_prefill_block_sparse(const attn_shape_t* shape, int32_t block_size, const void* q,
                                        const void* k, const void* v, const int32_t* kv_count,
                                        const int32_t* kv_index, void* o, float* lse, void* stream) {
    attn_status_t st = check_prefill_shape(shape, true);
    if (st != ATTN_OK) return st;
    if (block_size != 64 && block_size != 128 && block_size != 256)
        return fail(ATTN_ERR_UNSUPPORTED, "block_size %d is not supported (64, 128 or 256)", block_size);
    if (shape->seq_len % block_size) return fail(ATTN_ERR_SHAPE, "seq_len must be a multiple of block_size");
    if (shape->seq_len / block_size > 4096) return fail(ATTN_ERR_UNSUPPORTED, "more than 4096 blocks per row");
    if (shape->seq_len == 0) return ok();
    if ((st = check_ptrs({q, k, v, o, kv_count, kv_index})) != ATTN_OK) return st;
    if (lse && !aligned16(lse)) return fail(ATTN_ERR_ALIGN, "lse must be 16-byte aligned");
    const lcattn::PrefillProblem p = to_problem(shape, q, k, v, o, lse);
    return hip_status(
        lcattn::launch_prefill_sparse_bf16(p, block_size, kv_count, kv_index, static_cast<hipStream_t>(stream)),
        "attn_prefill_block_sparse");
}

size_t attn_decode_workspace_bytes(const attn_decode_shape_t* shape, int32_t max_seq_len) {
    if (check_decode_shape(shape, max_seq_len) != ATTN_OK) return 0;
    return lcattn::decode_workspace_bytes(shape->batch, shape->heads_q, shape->head_dim, shape->chunk_tokens,
                                          max_seq_len);
}

namespace {

// Checks and problem set-up shared by the bf16 and fp8 decode entry points.
attn_status_t decode_problem(const attn_decode_shape_t* shape, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                             int32_t max_seq_len, void* o, float* lse, void* workspace, size_t workspace_bytes,
                             lcattn::DecodeProblem& p) {
    attn_status_t st = check_decode_shape(shape, max_seq_len);
    if (st != ATTN_OK) return st;
    if ((st = check_ptrs({q, block_table, seq_lens, o})) != ATTN_OK) return st;
    if (max_seq_len > 0 && shape->num_pages > 0 && (st = check_ptrs({k_cache, v_cache})) != ATTN_OK) return st;
    if (max_seq_len > 0 && shape->num_pages == 0)
        return fail(ATTN_ERR_SHAPE, "max_seq_len > 0 needs at least one cache page");
    if (lse && !aligned16(lse)) return fail(ATTN_ERR_ALIGN, "lse must be 16-byte aligned");
    const size_t need = lcattn::decode_workspace_bytes(shape->batch, shape->heads_q, shape->head_dim,
                                                       shape->chunk_tokens, max_seq_len);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.o = o;
    p.lse = lse;
    p.B = shape->batch;
    p.Hq = shape->heads_q;
    p.Hkv = shape->heads_kv;
    p.D = shape->head_dim;
    p.page = shape->page_size;
    p.max_pages = shape->max_pages_per_seq;
    p.num_pages = shape->num_pages;
    p.chunk = shape->chunk_tokens;
    p.max_seq_len = max_seq_len;
    p.scale = shape->scale;
    return ATTN_OK;
}

}  // namespace

attn_status_t attn_decode_paged(const attn_decode_shape_t* shape, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                int32_t max_seq_len, void* o, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
    lcattn::DecodeProblem p;
    const attn_status_t st = decode_problem(shape, q, k_cache, v_cache, block_table, seq_lens, max_seq_len, o, lse,
                                            workspace, workspace_bytes, p);
    if (st != ATTN_OK) return st;
    return hip_status(lcattn::launch_decode_paged(p, workspace, static_cast<hipStream_t>(stream)), "attn_decode_paged");
}

namespace {

int paged_splits(const attn_paged_prefill_shape_t& s) {
    return lcattn::paged_prefill_splits(s.batch, s.heads_q, s.heads_kv, s.head_dim, s.q_len,
                                        s.max_pages_per_seq * s.page_size, s.window);
}

}  // namespace

size_t attn_prefill_paged_workspace_bytes(const attn_paged_prefill_shape_t* shape) {
    if (!shape || shape->batch < 1 || shape->heads_q < 1 || shape->heads_kv < 1 || shape->q_len < 0 ||
        shape->max_pages_per_seq < 1 || shape->window < 0 || shape->heads_q % shape->heads_kv ||
        (shape->head_dim != 64 && shape->head_dim != 128) || shape->page_size != 16)
        return 0;
    return lcattn::paged_prefill_workspace_bytes(shape->batch, shape->heads_q, shape->head_dim, shape->q_len,
                                                 paged_splits(*shape));
}

attn_status_t attn_prefill_paged(const attn_paged_prefill_shape_t* shape, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table, const int32_t* seq_lens, void* o,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (!shape) return fail(ATTN_ERR_NULL, "shape is NULL");
    const attn_paged_prefill_shape_t& s = *shape;
    if (s.batch < 1 || s.heads_q < 1 || s.heads_kv < 1 || s.q_len < 0 || s.num_pages < 0 || s.max_pages_per_seq < 1 ||
        s.window < 0)
        return fail(ATTN_ERR_SHAPE, "batch, heads, max_pages_per_seq must be >= 1; q_len, num_pages, window >= 0");
    if (s.heads_q % s.heads_kv) return fail(ATTN_ERR_SHAPE, "heads_q must be a multiple of heads_kv");
    if (s.head_dim != 64 && s.head_dim != 128) return fail(ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (s.page_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "page_size must be 16");
    if (!(std::isfinite(s.scale) && s.scale > 0.0f)) return fail(ATTN_ERR_SHAPE, "scale must be finite and > 0");
    if ((long long)s.q_len > (long long)s.max_pages_per_seq * s.page_size)
        return fail(ATTN_ERR_SHAPE, "q_len exceeds max_pages_per_seq * page_size");
    // work-groups: ceil(q_len / positions per group) x batch x kv heads x head groups <= (q_len / 32 + 1) x batch x heads_q
    if (((long long)s.q_len / 32 + 1) * s.batch * s.heads_q > 0x7FFFFFFFLL)
        return fail(ATTN_ERR_UNSUPPORTED, "grid too large");
    if (s.q_len == 0) return ok();
    if (s.num_pages == 0) return fail(ATTN_ERR_SHAPE, "q_len > 0 needs at least one cache page");
    attn_status_t st = check_ptrs({q, k_cache, v_cache, block_table, seq_lens, o});
    if (st != ATTN_OK) return st;
    if (lse && !aligned16(lse)) return fail(ATTN_ERR_ALIGN, "lse must be 16-byte aligned");
    lcattn::PagedPrefillProblem p;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.o = o;
    p.lse = lse;
    p.B = s.batch;
    p.Hq = s.heads_q;
    p.Hkv = s.heads_kv;
    p.D = s.head_dim;
    p.Nq = s.q_len;
    p.max_pages = s.max_pages_per_seq;
    p.num_pages = s.num_pages;
    p.window = s.window;
    p.scale = s.scale;
    // key-range splits need their workspace; without it (NULL or too small) the chunk runs unsplit
    p.splits = paged_splits(s);
    const size_t need = lcattn::paged_prefill_workspace_bytes(s.batch, s.heads_q, s.head_dim, s.q_len, p.splits);
    if (p.splits > 1 && (!workspace || workspace_bytes < need)) p.splits = 1;
    if (p.splits > 1 && (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return fail(ATTN_ERR_ALIGN, "workspace must be 256-byte aligned");
    p.workspace = workspace;
    return hip_status(lcattn::launch_prefill_paged(p, static_cast<hipStream_t>(stream)), "attn_prefill_paged");
}

attn_status_t attn_decode_paged_fp8(const attn_decode_shape_t* shape, const void* q, const uint8_t* k_cache,
                                    const uint8_t* v_cache_t, float k_scale, float v_scale,
                                    const int32_t* block_table, const int32_t* seq_lens, int32_t max_seq_len,
                                    void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return fail(ATTN_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
    lcattn::DecodeProblem p;
    const attn_status_t st = decode_problem(shape, q, k_cache, v_cache_t, block_table, seq_lens, max_seq_len, o, lse,
                                            workspace, workspace_bytes, p);
    if (st != ATTN_OK) return st;
    return hip_status(lcattn::launch_decode_paged_fp8(p, k_scale, v_scale, workspace, static_cast<hipStream_t>(stream)),
                      "attn_decode_paged_fp8");
}

attn_status_t attn_decode_paged_noalloc(const attn_decode_shape_t* shape, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                        int32_t max_seq_len, void* o, float* lse, void* stream) {
    attn_status_t st = check_decode_shape(shape, max_seq_len);
    if (st != ATTN_OK) return st;
    const size_t need = lcattn::decode_workspace_bytes(shape->batch, shape->heads_q, shape->head_dim,
                                                       shape->chunk_tokens, max_seq_len);
    if (need > lcattn::kDecodeScratchBytes)
        return fail(ATTN_ERR_WORKSPACE, "this shape needs %zu bytes of decode scratch; the library holds %zu per GPU",
                    need, lcattn::kDecodeScratchBytes);
    // validate everything else against a stand-in workspace before touching the device
    lcattn::DecodeProblem p;
    if ((st = decode_problem(shape, q, k_cache, v_cache, block_table, seq_lens, max_seq_len, o, lse,
                             reinterpret_cast<void*>(uintptr_t(256)), lcattn::kDecodeScratchBytes, p)) != ATTN_OK)
        return st;
    void* scratch = nullptr;
    if ((st = hip_status(lcattn::decode_scratch(&scratch), "attn_decode_paged_noalloc: scratch lookup")) != ATTN_OK)
        return st;
    return hip_status(lcattn::launch_decode_paged(p, scratch, static_cast<hipStream_t>(stream)),
                      "attn_decode_paged_noalloc");
}

}  // extern "C"
