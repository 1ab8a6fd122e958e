/*
 * lcattn.h -- C ABI of the long-context causal attention library for AMD Instinct MI355X (gfx950).
 *
 * Four operations, all exact causal scaled-dot-product attention in the IO-aware tiled form with an online
 * softmax, so the N x N score matrix never reaches device memory:
 *
 *   attn_prefill_dense         causal grouped-query prefill
 *   attn_block_mask_build      the linear pre-pass that picks key blocks (centroid branch OR radius rescue)
 *   attn_prefill_block_sparse  prefill restricted to the picked key blocks
 *   attn_decode_paged          q_len = 1 decode over a paged KV cache, split over KV chunks and reduced by
 *                              log-sum-exp
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors are dense, row-major in the layouts
 *     stated per function (last dimension contiguous), and each base pointer is 16-byte aligned.
 *   - The library never allocates, frees, copies to or from the host, or synchronises. All work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL is the default stream) and runs asynchronously.
 *   - Arguments are validated on the host before anything is enqueued; a bad argument returns a status and
 *     enqueues nothing. After enqueueing, a launch failure reported by the HIP runtime returns ATTN_ERR_HIP.
 *     Faults while a kernel runs surface at the caller's next synchronisation, as with any HIP kernel.
 *   - attn_last_error() gives a thread-local text for the last non-OK status of the calling thread.
 *   - Queries are square and top-left aligned: query i attends keys 0..i. Query head h reads key/value head
 *     h / (heads_q / heads_kv) (contiguous groups).
 *   - The softmax uses exp(scale * q.k); lse outputs are natural-log log-sum-exps, fp32.
 */
#ifndef LCATTN_H
#define LCATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCATTN_ABI_VERSION 7

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,         /* a required pointer is NULL                                        */
    ATTN_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes                                */
    ATTN_ERR_UNSUPPORTED = 3,  /* valid request the library does not implement (dtype, head_dim ...) */
    ATTN_ERR_ALIGN = 4,        /* a base pointer is not 16-byte aligned                             */
    ATTN_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the *_workspace_bytes query        */
    ATTN_ERR_HIP = 6,          /* the HIP runtime reported an error while enqueueing                */
    /* Not statuses: these pin the enumeration's range to that of a 32-bit int, so any int32 value a caller
     * passes (e.g. to attn_status_string) is a value of the type on the C++ side of the ABI. */
    ATTN_STATUS_RANGE_MIN_ = -2147483647 - 1,
    ATTN_STATUS_RANGE_MAX_ = 2147483647
} attn_status_t;

typedef enum { ATTN_BF16 = 0, ATTN_FP32 = 1 } attn_dtype_t;

/* Prefill problem: Q [batch, heads_q, seq_len, head_dim]; K and V [batch, heads_kv, seq_len, head_dim];
 * O like Q in the same dtype. heads_q must be a multiple of heads_kv; scale must be finite and > 0. */
typedef struct {
    int32_t batch, heads_q, heads_kv, seq_len, head_dim;
    float scale;
    int32_t dtype; /* attn_dtype_t */
} attn_shape_t;

/* Block-mask rule parameters ("Your 128K Context Is 6x Slower Than It Needs to Be", section "The rescue
 * branch: two selection paths, one mask"). */
typedef struct {
    int32_t block_size;    /* rows per query block == keys per key block; a multiple of 64                 */
    int32_t keep_permille; /* centroid budget: row i keeps ceil((i+1) * keep_permille / 1000) blocks, 0..1000 */
    double rescue_alpha;   /* tau = med + alpha * (p_hi - med); +INF disables the rescue branch, >= 0       */
    int32_t q_lo_pct;      /* lower reference percentile of the radii (50 = median), 0..100                */
    int32_t q_hi_pct;      /* upper reference percentile (90), q_lo_pct <= q_hi_pct <= 100                 */
    int32_t rescue_mode;   /* 0: a flagged block is rescued for every row; 1: query-aware (step 4b), 0 or 1 */
} attn_mask_params_t;

/* Decode problem: q [batch, heads_q, head_dim]; caches [num_pages, heads_kv, page_size, head_dim];
 * block_table [batch, max_pages_per_seq] int32; seq_lens [batch] int32; O [batch, heads_q, head_dim]. */
typedef struct {
    int32_t batch, heads_q, heads_kv, head_dim, page_size, max_pages_per_seq, num_pages, chunk_tokens;
    float scale;
} attn_decode_shape_t;

/*
 * Dense causal GQA prefill ("attention-kernel-optimization", section "FlashAttention (1 -> 2 -> 3)": tiles of
 * Q, K, V on chip, online-normalised softmax, O(N d) memory).
 *   q, k, v  inputs in shape->dtype (bf16 or fp32), layouts as attn_shape_t.
 *   o        output, same dtype and layout as q.
 *   lse      optional fp32 [batch, heads_q, seq_len] (NULL to skip).
 * Supported: head_dim 64 or 128; bf16 (MFMA, fp32 accumulation) or fp32 (fp32 arithmetic throughout);
 * seq_len * head_dim * element size below 2^31 bytes (one head's K or V slab; 8,388,607 tokens at head_dim 128
 * in bf16), else ATTN_ERR_UNSUPPORTED. The same bound holds for attn_block_mask_build(_fp8k) and
 * attn_prefill_block_sparse. seq_len 0 is a no-op.
 */
attn_status_t attn_prefill_dense(const attn_shape_t* shape, const void* q, const void* k, const void* v, void* o,
                                 float* lse, void* stream);

/* Bytes of device workspace attn_block_mask_build needs for this shape and block size (0 on bad input). */
size_t attn_block_mask_workspace_bytes(const attn_shape_t* shape, const attn_mask_params_t* params);

/*
 * The block-selection pre-pass ("Your 128K Context Is 6x Slower Than It Needs to Be", sections "Why
 * block-sparse attention underperforms: the mean-dilution trap" and "The rescue branch"), with nb =
 * seq_len / block_size query blocks and as many key blocks:
 *   1. per query head and query block, the mean of the block's query rows; per kv head and key block, the key
 *      centroid and the radius (largest Euclidean key-to-centroid distance); float64, one pass over Q and K;
 *   2. per (batch, kv head): type-7 (linear) quantiles of the radii at q_lo_pct and q_hi_pct, and
 *      tau = med + alpha * (p_hi - med);
 *   3. rescue flag of key block j: radius_j > tau (strict), shared by the kv head's query heads;
 *   4. centroid branch of row (h, i): among key blocks j <= i, the ceil((i+1) * keep_permille / 1000) largest
 *      S_ij = scale * <query-block mean, key centroid> (float64), ties to the smaller j;
 *   4b. rescue_mode 0: every flagged j <= i is rescued in row (h, i). rescue_mode 1 (query-aware; the section's
 *      coefficient from the median and the upper percentile, candidates scored against the base path): with
 *      lambda = (p_hi - med) / p_hi (0 if p_hi == 0) and cut_i the smallest score the centroid branch kept in the
 *      row, a flagged j is rescued in row (h, i) only if S_ij + lambda * scale * |query-block mean| * (radius_j -
 *      med) > cut_i (no rescue when the row keeps no centroid pick);
 *   5. mask[h,i,j] = 1 iff j <= i and (centroid pick or rescued or j == i).
 * Inputs: q, k bf16 in the prefill layouts. Outputs:
 *   mask      uint8 [batch, heads_q, nb, nb], 0/1, written in full.
 *   kv_count  int32 [batch, heads_q, nb], number of kept blocks per row.
 *   kv_index  int32 [batch, heads_q, nb, nb], kept key blocks of each row in ascending order in the first
 *             kv_count entries; later entries are not written.
 *   radius_stats  optional float64 [batch, heads_kv, nb + 3]: the nb radii, then med, p_hi, tau (NULL to skip).
 * Workspace (>= attn_block_mask_workspace_bytes, 256-byte aligned) holds, in order and each 256-byte aligned:
 * query-block means f64 [batch, heads_q, nb, head_dim], key centroids f64 [batch, heads_kv, nb, head_dim],
 * radii f64 [batch, heads_kv, nb], (med, p_hi, tau, lambda) f64 [batch, heads_kv, 4], rescue flags u8
 * [batch, heads_kv, nb], centroid scores f64 [batch, heads_q, nb, nb] (lower triangle only).
 * Supported: bf16, head_dim 64 or 128, block_size a multiple of 64 dividing seq_len, 1 <= nb <= 4096.
 */
attn_status_t attn_block_mask_build(const attn_shape_t* shape, const attn_mask_params_t* params, const void* q,
                                    const void* k, uint8_t* mask, int32_t* kv_count, int32_t* kv_index,
                                    double* radius_stats, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_block_mask_build with the keys given as 8-bit E4M3 codes, one scale per tensor (key = code value * k_scale;
 * OCP E4M3 as for attn_decode_paged_fp8). The centroids and radii are computed from those key values, which asks
 * whether the rescue signal survives eight-bit keys ("Your 128K Context Is 6x Slower Than It Needs to Be", section
 * "The numbers, stated honestly": the benchmark model's FP8 keys kept accuracy). Each code is widened exactly and
 * scaled once in float64; every later step, output and the workspace are attn_block_mask_build's.
 *   k_codes  E4M3 [batch, heads_kv, seq_len, head_dim] (16-byte aligned); q bf16 as before; k_scale finite > 0.
 */
attn_status_t attn_block_mask_build_fp8k(const attn_shape_t* shape, const attn_mask_params_t* params, const void* q,
                                         const uint8_t* k_codes, float k_scale, uint8_t* mask, int32_t* kv_count,
                                         int32_t* kv_index, double* radius_stats, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * Block-sparse causal prefill: dense prefill restricted, for query row t of query block i = t / block_size, to
 * the keys u <= t whose key block u / block_size is listed in kv_index[b, h, i, 0 .. kv_count[b,h,i]) ("Your
 * 128K Context Is 6x Slower Than It Needs to Be", sections "Why block-sparse attention underperforms" and "The
 * rescue branch": the combined mask runs as ordinary block-sparse tiled attention and skipped blocks cost
 * nothing). Lists must be ascending, within [0, i], and hold i itself (every row then sees at least its own
 * key); the kernel trusts them, so the caller validates untrusted lists. kv_count/kv_index as produced by
 * attn_block_mask_build. Supported: bf16, head_dim 64 or 128, block_size 64, 128 or 256 dividing seq_len, at
 * most 4096 blocks.
 */
attn_status_t attn_prefill_block_sparse(const attn_shape_t* shape, int32_t block_size, const void* q,
                                        const void* k, const void* v, const int32_t* kv_count,
                                        const int32_t* kv_index, void* o, float* lse, void* stream);

/* Chunked prefill over a paged cache: q [batch, heads_q, q_len, head_dim]; caches as for decode. */
typedef struct {
    int32_t batch, heads_q, heads_kv, head_dim, q_len, page_size, max_pages_per_seq, num_pages;
    int32_t window;  /* 0: causal over the whole sequence; > 0: each query sees its `window` latest keys */
    float scale;
} attn_paged_prefill_shape_t;

/*
 * Chunked prefill over a paged KV cache, optionally with a sliding window ("attention-kernel-optimization",
 * section "PagedAttention": fixed-size pages found through a block table; "Your Context Length Decides What a
 * Kernel Is Worth": sliding-window attention on some layers). Sequence b holds seq_lens[b] = L_b tokens in its
 * pages, the last q_len of which are the new chunk (their K/V already written); chunk row r sits at position
 * p = L_b - q_len + r and sees the keys t <= p, and with window > 0 only those with t > p - window. Each row is
 * exact attention over those keys with the dense prefill's arithmetic.
 *   q            bf16 [batch, heads_q, q_len, head_dim]
 *   k_cache, v_cache  bf16 [num_pages, heads_kv, page_size, head_dim]
 *   block_table  int32 [batch, max_pages_per_seq]; entries below ceil(L_b / page_size) are read (trusted, in
 *                [0, num_pages); an entry outside reads as zeros)
 *   seq_lens     int32 [batch], each in [q_len, max_pages_per_seq * page_size] (trusted)
 *   o            bf16 like q; lse optional fp32 [batch, heads_q, q_len] (NULL to skip).
 *   workspace    device scratch of attn_prefill_paged_workspace_bytes(shape) bytes, or NULL (see there).
 * Cache slots at or past a sequence's end may hold any bits; they never reach the output. q_len 0 is a no-op.
 * Supported: head_dim 64 or 128, page_size 16.
 */
attn_status_t attn_prefill_paged(const attn_paged_prefill_shape_t* shape, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table, const int32_t* seq_lens, void* o,
                                 float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace (256-byte aligned) with which attn_prefill_paged splits each row set's keys across
 * several work-groups and merges them by log-sum-exp: chosen from the shape when the chunk alone has too few, or
 * too evenly loaded, work-groups to fill the GPU (a chunk closing a long sequence). 0 when no split is taken.
 * attn_prefill_paged given less (or NULL) runs unsplit, with the same result up to rounding. */
size_t attn_prefill_paged_workspace_bytes(const attn_paged_prefill_shape_t* shape);

/* Bytes of device workspace attn_decode_paged needs when no sequence is longer than max_seq_len. */
size_t attn_decode_workspace_bytes(const attn_decode_shape_t* shape, int32_t max_seq_len);

/*
 * Split-KV decode over a paged KV cache ("attention-kernel-optimization", sections "Inference-specific:
 * Flash-Decoding and FlashInfer" -- split the keys, attend the pieces in parallel, reduce -- and
 * "PagedAttention" -- fixed-size pages placed anywhere, found through a block table).
 * The query of sequence b is the token at position seq_lens[b] - 1; it attends all seq_lens[b] cached tokens
 * (the caller has already written its own K/V). Token t of sequence b sits in slot t % page_size of page
 * block_table[b, t / page_size]. Each work-group takes chunk_tokens tokens of one (sequence, kv head) for all
 * heads_q / heads_kv query heads; a second kernel merges the chunks by log-sum-exp.
 *   q         bf16 [batch, heads_q, head_dim]
 *   k_cache, v_cache  bf16 [num_pages, heads_kv, page_size, head_dim]
 *   block_table  int32 [batch, max_pages_per_seq]; only entries < ceil(seq_lens[b] / page_size) are read and
 *             each must lie in [0, num_pages) (trusted, not checked on the device).
 *   seq_lens  int32 [batch], each in [0, max_seq_len] (trusted, not checked on the device).
 *   max_seq_len  host-side upper bound of seq_lens, sizes the grid and the workspace.
 *   o         bf16 [batch, heads_q, head_dim]; lse optional fp32 [batch, heads_q] (NULL to skip).
 * Cache slots at or past seq_lens[b] and pages the table does not reference may hold any bits, NaN included;
 * they never reach the output. seq_lens[b] == 0 gives o = 0 and lse = -inf.
 * Supported: head_dim 64 or 128, page_size 16, chunk_tokens a multiple of 64 up to 4096, heads_q / heads_kv <= 16.
 */
attn_status_t attn_decode_paged(const attn_decode_shape_t* shape, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                int32_t max_seq_len, void* o, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * attn_decode_paged over an fp8 KV cache, which halves the bytes a decode step moves ("Your Context Length
 * Decides What a Kernel Is Worth": decode is bandwidth-bound and an fp8 KV cache is one of the two things that
 * help). Codes are OCP E4M3 (bias 7, 3 mantissa bits, subnormals, NaN at S.1111.111); a cached key is
 * code value * k_scale and a cached value code value * v_scale.
 *   k_cache    E4M3 [num_pages, heads_kv, page_size, head_dim] (token-major, like the bf16 cache)
 *   v_cache_t  E4M3 [num_pages, heads_kv, head_dim, page_size]: each page transposed, its tokens contiguous
 *   k_scale, v_scale  finite and > 0.
 * Everything else -- q, block table, lengths, output, lse, workspace (attn_decode_workspace_bytes), the trusted
 * inputs, the handling of slots past a sequence's end (any byte, the NaN code included) -- is as in
 * attn_decode_paged. The codes are widened to bf16 exactly and the arithmetic is the bf16 path's.
 */
attn_status_t attn_decode_paged_fp8(const attn_decode_shape_t* shape, const void* q, const uint8_t* k_cache,
                                    const uint8_t* v_cache_t, float k_scale, float v_scale,
                                    const int32_t* block_table, const int32_t* seq_lens, int32_t max_seq_len,
                                    void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged without a workspace argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that must not call hipMalloc, harnesses that forbid allocation. The chunk partials go
 * to a scratch array the library holds in each GPU's memory (LCATTN_DECODE_SCRATCH_BYTES per GPU, reserved when
 * the library's device code is loaded on that GPU and held until the process ends); the call itself allocates
 * nothing. Arguments, layouts, trusted inputs, outputs and results are attn_decode_paged's (the same kernels).
 * A shape whose attn_decode_workspace_bytes(shape, max_seq_len) exceeds LCATTN_DECODE_SCRATCH_BYTES returns
 * ATTN_ERR_WORKSPACE before anything is enqueued. Every call on one GPU uses that GPU's one scratch array: calls
 * that overlap in time on the same GPU (different streams, or host threads, without ordering) race and may return
 * wrong results; calls ordered on one stream are safe. Nothing in the scratch needs to start at zero: each call
 * writes every partial it reads.
 */
#define LCATTN_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
attn_status_t attn_decode_paged_noalloc(const attn_decode_shape_t* shape, const void* q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_table, const int32_t* seq_lens,
                                        int32_t max_seq_len, void* o, float* lse, void* stream);

const char* attn_status_string(attn_status_t status);
const char* attn_last_error(void);
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LCATTN_H */
