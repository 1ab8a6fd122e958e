// Split-KV decode over a paged KV cache for gfx950, then a log-sum-exp combine.
//
// Method: with one query token there is no query-length parallelism, so the keys of each sequence are cut into
// chunks that are attended in parallel and merged afterwards ("attention-kernel-optimization", section
// "Inference-specific: Flash-Decoding and FlashInfer"); the KV cache is a pool of fixed-size pages placed
// anywhere and found through a per-sequence block table (same page, section "PagedAttention").
//
// Split kernel: work-group = (chunk of chunk_tokens tokens, kv head, sequence), 4 waves, each wave a quarter of
// the chunk's pages. Every (page, kv head) is one contiguous slab of 16 x head_dim bf16, so the K slab is read
// straight into the A operand of v_mfma_f32_16x16x32_bf16 (lane = token row, 16-byte pieces of the head dim)
// and S^T = K Q^T comes out with the group's query heads as columns. All page loads of a wave are issued
// before any is used, to keep many bytes in flight. V is written transposed into LDS (zero for slots past the
// sequence end, so NaN padding cannot leak) and read back as the A operand of v_mfma_f32_16x16x16_bf16 with the
// bf16 probabilities as B, which are already in B-operand order in the lane that computed them.
// The four wave partials are merged in LDS; the chunk's normalised output and natural-log lse go to the
// workspace. Combine kernel: one wave per (sequence, query head) merges the chunks by log-sum-exp.
#include "device_common.hpp"
#include "internal.hpp"

namespace lcattn {
namespace {

constexpr int kPage = 16;
constexpr int kVtPitch = kPage * 2 + 8;   // bytes per V^T row inside one page's slab in LDS

struct SplitArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* bt;
    const int32_t* lens;
    float* opart;   // [B, Hq, C, D]
    float* lpart;   // [B, Hq, C]
    int B, Hq, Hkv, G, max_pages, num_pages, C, chunk, ppw;  // ppw = pages per wave
    float c2;
};

// PB pages per batch and wave; the wave walks its ppw pages in batches.
template <int D, int PB>
__global__ __launch_bounds__(256) void decode_split_kernel(const SplitArgs a) {
    constexpr int KS = D / 32;                  // K operand pieces per page (16x16x32 MFMAs per page)
    constexpr int VL = (kPage * D) / (64 * 8);  // 16-byte V loads per lane per page
    constexpr int DT = D / 16;                  // 16-row tiles of the head dim
    __shared__ __attribute__((aligned(16))) char vt_all[4 * PB * D * kVtPitch];
    __shared__ float red_m[4][16];
    __shared__ float red_l[4][16];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = a.lens[b];
    if (c * a.chunk >= L) return;  // uniform over the work-group
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int n = lane & 15, grp = lane >> 4;
    char* vt = vt_all + w * PB * D * kVtPitch;

    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = n < a.G ? __builtin_bit_cast(bf16x8, load16(a.q + ((size_t)b * a.Hq + g * a.G + n) * D + 32 * ks +
                                                                 8 * grp))
                         : bf16x8{};

    const int npages_seq = (L + kPage - 1) / kPage;
    const int wpage0 = c * (a.chunk / kPage) + w * a.ppw;
    const int32_t* btrow = a.bt + (size_t)b * a.max_pages;
    const size_t slab = (size_t)kPage * D;

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
    float m = -INFINITY, l = 0.0f;

    for (int pb0 = 0; pb0 < a.ppw; pb0 += PB) {
        u32x4 kr[PB][KS], vr[PB][VL];
        bool pv[PB];
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const int lp = wpage0 + pb0 + p;
            pv[p] = (pb0 + p < a.ppw) && lp < npages_seq && lp < a.max_pages;
            const uint16_t* ks_ = nullptr;
            const uint16_t* vs_ = nullptr;
            if (pv[p]) {
                const int pid = btrow[lp];
                pv[p] = (unsigned)pid < (unsigned)a.num_pages;   // out-of-pool entries read as masked slots
                ks_ = a.kc + ((size_t)pid * a.Hkv + g) * slab;
                vs_ = a.vc + ((size_t)pid * a.Hkv + g) * slab;
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kr[p][ks] = pv[p] ? load16(ks_ + n * D + 32 * ks + 8 * grp) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < VL; ++i) vr[p][i] = pv[p] ? load16(vs_ + (i * 64 + lane) * 8) : u32x4{0u, 0u, 0u, 0u};
        }
        // scores: S^T[token = 4*grp + r][head n] per page
        f32x4 s[PB];
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            s[p] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[p][ks]), qf[ks], s[p], 0,
                                                               0, 0);
            const int tok0 = (wpage0 + pb0 + p) * kPage + 4 * grp;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (!pv[p] || tok0 + r >= L) s[p][r] = -INFINITY;
                mx = fmaxf(mx, s[p][r]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxs = mx * a.c2;
        if (mxs > m) {
            const float alpha = exp2f(m - mxs);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            m = mxs;
        }
        const float bias = (m == -INFINITY) ? 0.0f : -m;
        // V^T into LDS: slab row t, 8 head-dim values per 16-byte load
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            char* vp = vt + p * D * kVtPitch;
#pragma unroll
            for (int i = 0; i < VL; ++i) {
                const int e0 = (i * 64 + lane) * 8;
                const int t = e0 / D, d0 = e0 % D;
                const bool ok = pv[p] && (wpage0 + pb0 + p) * kPage + t < L;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t word = vr[p][i][e >> 1];
                    const uint16_t hv = ok ? (uint16_t)((e & 1) ? (word >> 16) : (word & 0xFFFFu)) : (uint16_t)0;
                    *reinterpret_cast<uint16_t*>(vp + (d0 + e) * kVtPitch + t * 2) = hv;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            float p4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p4[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][r], a.c2, bias));
            }
            const uint32_t w0 = pack_bf16x2(p4[0], p4[1]), w1 = pack_bf16x2(p4[2], p4[3]);
            const bf16x4 pb = __builtin_bit_cast(bf16x4, (u32x2{w0, w1}));
            bf16x2 ones;
            ones[0] = (__bf16)1.0f;
            ones[1] = (__bf16)1.0f;
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, l, false);
            const char* vp = vt + p * D * kVtPitch;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16x4 av =
                    __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2*>(vp + (16 * dt + n) * kVtPitch + 8 * grp));
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pb, o[dt], 0, 0, 0);
            }
        }
    }
    // wave partial -> LDS: this lane holds O^T[d = 16*dt + 4*grp + r][head n], sum share l, max m (same over a
    // head's lanes)
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();  // all waves are done with their V^T slabs; reuse the space for the merge
    float* red_o = reinterpret_cast<float*>(vt_all);  // [4 waves][16 heads][D]
    if (grp == 0) {
        red_m[w][n] = m;
        red_l[w][n] = l;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_o[(w * 16 + n) * D + 16 * dt + 4 * grp + r] = o[dt][r];
    __syncthreads();
    // merge: thread -> (head, d) pairs
    for (int e = tid; e < a.G * D; e += 256) {
        const int hn = e / D, d = e % D;
        float M = red_m[0][hn];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, red_m[ww][hn]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float mw = red_m[ww][hn];
            const float sc = mw == -INFINITY ? 0.0f : exp2f(mw - M);
            acc += sc * red_o[(ww * 16 + hn) * D + d];
            lsum += sc * red_l[ww][hn];
        }
        const size_t row = ((size_t)b * a.Hq + g * a.G + hn) * a.C + c;
        a.opart[row * D + d] = acc / lsum;
        if (d == 0) a.lpart[row] = (M + log2f(lsum)) * kLn2;
    }
}

struct CombineArgs {
    const float* opart;
    const float* lpart;
    const int32_t* lens;
    uint16_t* o;
    float* lse;
    int B, Hq, C, chunk;
};

template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const CombineArgs a) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + w;
    if (bh >= a.B * a.Hq) return;
    const int b = bh / a.Hq;
    const int L = a.lens[b];
    const int nc = min(a.C, (L + a.chunk - 1) / a.chunk);
    const float* lp = a.lpart + (size_t)bh * a.C;
    const float* op = a.opart + (size_t)bh * a.C * D;
    uint16_t* orow = a.o + (size_t)bh * D;
    if (nc == 0) {
        for (int d = lane; d < D; d += 64) orow[d] = 0;
        if (a.lse && lane == 0) a.lse[bh] = -INFINITY;
        return;
    }
    float M = -INFINITY;
    for (int c = lane; c < nc; c += 64) M = fmaxf(M, lp[c]);
    M = wave_max(M);
    float acc[D / 64];
#pragma unroll
    for (int k = 0; k < D / 64; ++k) acc[k] = 0.0f;
    float sw = 0.0f;
    for (int c = 0; c < nc; ++c) {
        const float wc = expf(lp[c] - M);
        sw += wc;
#pragma unroll
        for (int k = 0; k < D / 64; ++k) acc[k] = __builtin_fmaf(wc, op[(size_t)c * D + lane + 64 * k], acc[k]);
    }
    const float inv = 1.0f / sw;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) orow[lane + 64 * k] = __builtin_bit_cast(uint16_t, (__bf16)(acc[k] * inv));
    if (a.lse && lane == 0) a.lse[bh] = M + logf(sw);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int D, int chunk, int max_seq_len) {
    const size_t C = (size_t)((max_seq_len + chunk - 1) / chunk);
    const size_t o_bytes = (size_t)B * Hq * (C ? C : 1) * D * sizeof(float);
    const size_t l_bytes = (size_t)B * Hq * (C ? C : 1) * sizeof(float);
    return ((o_bytes + 255) / 256) * 256 + ((l_bytes + 255) / 256) * 256;
}

hipError_t launch_decode_paged(const DecodeProblem& p, void* workspace, hipStream_t s) {
    const int C = (p.max_seq_len + p.chunk - 1) / p.chunk;
    const size_t o_bytes = (size_t)p.B * p.Hq * (C ? C : 1) * p.D * sizeof(float);
    SplitArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.kc = static_cast<const uint16_t*>(p.k_cache);
    a.vc = static_cast<const uint16_t*>(p.v_cache);
    a.bt = p.block_table;
    a.lens = p.seq_lens;
    a.opart = static_cast<float*>(workspace);
    a.lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((o_bytes + 255) / 256) * 256);
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.G = p.Hq / p.Hkv;
    a.max_pages = p.max_pages;
    a.num_pages = p.num_pages;
    a.C = C ? C : 1;
    a.chunk = p.chunk;
    a.ppw = p.chunk / kPage / 4;
    a.c2 = p.scale * kLog2e;
    if (C > 0) {
        const dim3 grid((unsigned)C, (unsigned)p.Hkv, (unsigned)p.B);
        if (p.D == 64) hipLaunchKernelGGL((decode_split_kernel<64, 8>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((decode_split_kernel<128, 4>), grid, dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    CombineArgs cb;
    cb.opart = a.opart;
    cb.lpart = a.lpart;
    cb.lens = p.seq_lens;
    cb.o = static_cast<uint16_t*>(p.o);
    cb.lse = p.lse;
    cb.B = p.B;
    cb.Hq = p.Hq;
    cb.C = a.C;
    cb.chunk = p.chunk;
    const dim3 grid2((unsigned)((p.B * p.Hq + 3) / 4));
    if (p.D == 64) hipLaunchKernelGGL((decode_combine_kernel<64>), grid2, dim3(256), 0, s, cb);
    else hipLaunchKernelGGL((decode_combine_kernel<128>), grid2, dim3(256), 0, s, cb);
    return hipGetLastError();
}

}  // namespace lcattn
