// Host-side interface between the C ABI layer (abi.hip) and the kernel translation units. Arguments reaching
// these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcattn {

struct PrefillProblem {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;  // may be null
    int B, Hq, Hkv, N, D;
    float scale;
};

hipError_t launch_prefill_dense_bf16(const PrefillProblem& p, hipStream_t s);
hipError_t launch_prefill_dense_f32(const PrefillProblem& p, hipStream_t s);
hipError_t launch_prefill_sparse_bf16(const PrefillProblem& p, int block, const int32_t* kv_count,
                                      const int32_t* kv_index, hipStream_t s);

struct MaskProblem {
    const void* q;
    const void* k;         // bf16 keys, unless k8 is set
    const uint8_t* k8 = nullptr;   // E4M3 key codes, value = code value * k_scale
    double k_scale = 1.0;
    int B, Hq, Hkv, N, D, block, nb;
    double scale;
    int keep_permille;
    double alpha;
    int lo_pct, hi_pct;
    int rescue_mode;       // 0 query-blind, 1 query-aware
    uint8_t* mask;
    int32_t* kv_count;
    int32_t* kv_index;
    double* radius_stats;  // may be null
};

struct MaskWorkspace {
    double* qbar;
    double* kbar;
    double* radius;
    double* thresh;
    uint8_t* flags;
    double* scores;
    size_t total;
};

MaskWorkspace mask_workspace_layout(int B, int Hq, int Hkv, int nb, int D, char* base);
hipError_t launch_block_mask(const MaskProblem& p, const MaskWorkspace& ws, hipStream_t s);

struct DecodeProblem {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* o;
    float* lse;  // may be null
    int B, Hq, Hkv, D, page, max_pages, num_pages, chunk, max_seq_len;
    float scale;
};

// Chunked prefill over a paged bf16 cache ([num_pages, Hkv, 16, D]); q/o [B, Hq, Nq, D].
struct PagedPrefillProblem {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* seq_lens;
    void* o;
    float* lse;  // may be null
    int B, Hq, Hkv, D, Nq, max_pages, num_pages, window;
    float scale;
    int splits;           // key-range splits (1: no workspace)
    void* workspace;      // splits > 1: paged_prefill_workspace_bytes
};
hipError_t launch_prefill_paged(const PagedPrefillProblem& p, hipStream_t s);
int paged_prefill_splits(int B, int Hq, int Hkv, int D, int Nq, int max_seq_len, int window);
size_t paged_prefill_workspace_bytes(int B, int Hq, int D, int Nq, int splits);

size_t decode_workspace_bytes(int B, int Hq, int D, int chunk, int max_seq_len);
// The library's own decode scratch (attn_decode_paged_noalloc): kDecodeScratchBytes per GPU, device address of the
// current device's copy.
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode_paged(const DecodeProblem& p, void* workspace, hipStream_t s);
// k_cache holds E4M3 codes [pages, Hkv, 16, D], v_cache E4M3 codes transposed per page [pages, Hkv, D, 16]
hipError_t launch_decode_paged_fp8(const DecodeProblem& p, float k_scale, float v_scale, void* workspace,
                                   hipStream_t s);

}  // namespace lcattn
