// Split-KV decode over a paged KV cache for gfx950, then a log-sum-exp combine.
//
// Method: with one query token there is no query-length parallelism, so the keys of each sequence are cut into
// chunks that are attended in parallel and merged afterwards ("attention-kernel-optimization", section
// "Inference-specific: Flash-Decoding and FlashInfer"); the KV cache is a pool of fixed-size pages placed
// anywhere and found through a per-sequence block table (same page, section "PagedAttention").
//
// Split kernel: work-group = (chunk of chunk_tokens tokens, kv head, sequence), 1, 2 or 4 waves, each streaming its
// share of the chunk's pages in batches of 2 or 4 pages with the next batch in flight. Every (page, kv head) is
// one contiguous slab of 16 x head_dim bf16, so the K slab is read straight into the A operand of
// v_mfma_f32_16x16x32_bf16 (lane = token row, 16-byte pieces of the head dim) and S^T = K Q^T comes out with the
// group's query heads as columns. V goes from HBM straight into LDS in its natural layout and comes back as the A
// operand of v_mfma_f32_16x16x16_bf16 through ds_read_b64_tr_b16, with the bf16 probabilities as B, which are
// already in B-operand order in the lane that computed them. Each page's buffer view ends at the sequence end,
// so slots past it read as zeros and NaN padding cannot leak.
// The wave partials are merged in LDS; the chunk's normalised output and natural-log lse go to the workspace.
// Combine kernel: one wave per (sequence, query head) merges the chunks by log-sum-exp.
#include <mutex>
#include <vector>

#include "device_common.hpp"
#include "internal.hpp"

namespace lcattn {
namespace {

constexpr int kPage = 16;
typedef short v4i16 __attribute__((ext_vector_type(4)));
struct SplitArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int32_t* bt;
    const int32_t* lens;
    float* opart;   // [B, C, Hq, D]: a work-group's rows (its kv group's query heads) are one contiguous run
    float* lpart;   // [B, C, Hq]
    int B, Hq, Hkv, G, max_pages, num_pages, C, chunk, ppw;  // ppw = pages per wave
    float c2;
};

// A buffer view of one (page, kv head) slab of 16 x D bf16 whose size stops at the sequence end: slots past it, and
// whole pages past it or outside the pool, read as zeros, so cache padding (NaN included) never reaches the maths.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const uint16_t* cache, int pid, int hkv, int g, int valid,
                                                            int D) {
    const uint16_t* base = cache + ((size_t)pid * hkv + g) * (size_t)kPage * D;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, valid * D * 2, 0x00020000);
}

// One page's transposed V reads (head-dim tiles 32 bytes apart from one lane address), complete on return. They are
// written as one asm block ending in its own LDS wait because the compiler, when it cannot tell them apart from the
// direct-to-LDS loads still in flight into the other buffer, would otherwise wait for all of those first.
typedef __attribute__((address_space(3))) char lds_char;
template <int DT>
__device__ __forceinline__ void tr_read_page(v4i16 (&av)[DT], const lds_char* addr);
template <>
__device__ __forceinline__ void tr_read_page<4>(v4i16 (&av)[4], const lds_char* addr) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %4 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %4 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(av[0]), "=&v"(av[1]), "=&v"(av[2]), "=&v"(av[3])
        : "v"(addr)
        : "memory");
}
template <>
__device__ __forceinline__ void tr_read_page<8>(v4i16 (&av)[8], const lds_char* addr) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:160\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:224\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(av[0]), "=&v"(av[1]), "=&v"(av[2]), "=&v"(av[3]), "=&v"(av[4]), "=&v"(av[5]), "=&v"(av[6]),
          "=&v"(av[7])
        : "v"(addr)
        : "memory");
}

template <int D, int PB>
struct Batch {
    u32x4 k[PB][D / 32];   // K slabs straight into the MFMA A-operand layout
    int tok0;               // first logical token of the batch
};

// Work-group = (chunk of chunk_tokens tokens, kv head, sequence); NW waves, each streaming its ppw pages in
// batches of PB pages with the next batch in flight while the current one is used. K goes to VGPRs in the A
// layout of v_mfma_f32_16x16x32_bf16 (lane = token row, 16-byte pieces of the head dim) and S^T = K Q^T has the
// kv group's query heads as columns. V goes straight to LDS in its natural layout and comes back as the A
// operand of v_mfma_f32_16x16x16_bf16 through ds_read_b64_tr_b16 (a 16-lane group receives 16 head-dim rows x 4
// tokens); the bf16 probabilities are the B operand in the lane that computed them.
template <int D, int NW, int PB>
__global__ __launch_bounds__(NW * 64) void decode_split_kernel(const SplitArgs a) {
    constexpr int KS = D / 32;                    // 16x16x32 MFMAs per page for S^T
    constexpr int DT = D / 16;                    // 16-row tiles of the head dim for O^T
    constexpr int SLAB = kPage * D * 2;           // bytes per page slab
    constexpr int VLOADS = SLAB / 1024;           // 1 KiB direct loads per slab
    constexpr int kPB = PB;
    // the two V buffers are distinct arrays: reads of one are then known not to alias direct-to-LDS loads still in
    // flight into the other, so the compiler does not wait for those loads before reading
    __shared__ __attribute__((aligned(1024))) char vbuf0[NW][kPB * SLAB];   // [wave]
    __shared__ __attribute__((aligned(1024))) char vbuf1[NW][kPB * SLAB];
    static_assert(NW * 16 * D * sizeof(float) <= sizeof(vbuf0), "merge partials must fit the first V buffer");
    static_assert(2 * NW * 16 * sizeof(float) <= sizeof(vbuf1), "merge maxima and sums must fit the second");

    const int g = (int)(blockIdx.x % a.Hkv), c = (int)(blockIdx.x / a.Hkv), b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so page lookups stay scalar
    const int n = lane & 15, grp = lane >> 4;
    // the sequence length, the query rows and the wave's block-table entries (lane i <-> page wpage0 + i, ppw <= 64;
    // read out later with readlane) are all requested before any of them is waited for; entries past the
    // sequence end are read but never used
    const int L = a.lens[b];
    const int wpage0 = c * (a.chunk / kPage) + w * a.ppw;
    const int32_t* btrow = a.bt + (size_t)b * a.max_pages;
    const int my_page = wpage0 + lane;
    const int my_pid = (lane < a.ppw && my_page < a.max_pages) ? btrow[my_page] : 0;
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = n < a.G ? __builtin_bit_cast(bf16x8, load16(a.q + ((size_t)b * a.Hq + g * a.G + n) * D + 32 * ks +
                                                                 8 * grp))
                         : bf16x8{};
    if (c * a.chunk >= L) return;  // uniform over the work-group

    const int npages_seq = (L + kPage - 1) / kPage;
    // an even batch count, so the loop below runs both buffers every trip; batches past the wave's pages read
    // zeros through empty buffer views and are masked
    const int nbatch = ((a.ppw + 2 * kPB - 1) / (2 * kPB)) * 2;

    // issue batch `bi` into buffer `buf`
    auto issue = [&](int bi, int buf, Batch<D, PB>& bt) {
        bt.tok0 = (wpage0 + bi * kPB) * kPage;
#pragma unroll
        for (int p = 0; p < kPB; ++p) {
            const int lp = wpage0 + bi * kPB + p;
            const bool inrange = bi * kPB + p < a.ppw && lp < npages_seq && lp < a.max_pages;
            int pid = inrange ? __builtin_amdgcn_readlane(my_pid, min(bi * kPB + p, 63)) : 0;
            int valid = inrange ? min(kPage, L - lp * kPage) : 0;
            if ((unsigned)pid >= (unsigned)a.num_pages) {
                pid = 0;
                valid = 0;
            }
            const __amdgpu_buffer_rsrc_t kr = slab_rsrc(a.kc, pid, a.Hkv, g, valid, D);
            const __amdgpu_buffer_rsrc_t vr = slab_rsrc(a.vc, pid, a.Hkv, g, valid, D);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                bt.k[p][ks] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, (n * D + 32 * ks + 8 * grp) * 2, 0, 0));
            lds_char* dst = (buf ? (lds_char*)&vbuf1[w][0] : (lds_char*)&vbuf0[w][0]) + p * SLAB;
#pragma unroll
            for (int i = 0; i < VLOADS; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(dst + i * 1024),
                                                         16, (i * 64 + lane) * 16, 0, 0, 0);
        }
    };

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
    float m = -INFINITY, l = 0.0f;
    bf16x2 ones;
    ones[0] = (__bf16)1.0f;
    ones[1] = (__bf16)1.0f;

    // one batch: issue the next batch into the other register set and LDS buffer (an empty one past the last), wait
    // for this one, use it. The issue and the wait are unconditional so that the only loads still outstanding
    // during the maths are the next batch's, whatever the path.
    auto run = [&](int bi, int buf, Batch<D, PB>& cur, Batch<D, PB>& nxt) {
        issue(bi + 1, buf ^ 1, nxt);
        __builtin_amdgcn_s_waitcnt(0x0F70 | ((KS + VLOADS) * kPB & 15) | ((((KS + VLOADS) * kPB) >> 4) << 14));
        // scores S^T[token = 4*grp + r][head n] per page
        f32x4 s[kPB];
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < kPB; ++p) {
            s[p] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                s[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[p][ks]), qf[ks], s[p],
                                                               0, 0, 0);
            const int tok = cur.tok0 + p * kPage + 4 * grp;
            const bool page_in_wave = bi * kPB + p < a.ppw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (tok + r >= L || !page_in_wave) s[p][r] = -INFINITY;
                mx = fmaxf(mx, s[p][r]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxs = mx * a.c2;
        if (mxs > m) {
            const float alpha = __builtin_amdgcn_exp2f(m - mxs);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            m = mxs;
        }
        const float bias = (m == -INFINITY) ? 0.0f : -m;
        // the V slabs of this batch must be visible to every lane of the wave before the transposed reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int p = 0; p < kPB; ++p) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][0], a.c2, bias));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][1], a.c2, bias));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][2], a.c2, bias));
            const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][3], a.c2, bias));
            const uint32_t w0 = pack_bf16x2(p0, p1), w1 = pack_bf16x2(p2, p3);
            const bf16x4 pb = __builtin_bit_cast(bf16x4, (u32x2{w0, w1}));
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, l, false);
            // source lane 4*jj + aa of 16-lane group grp points at V[token 4*grp + jj][16*dt + 4*aa]
            const lds_char* slab = (buf ? (const lds_char*)&vbuf1[w][0] : (const lds_char*)&vbuf0[w][0]) + p * SLAB;
            const int src = (4 * grp + ((lane & 15) >> 2)) * D * 2 + 8 * (lane & 3);
            v4i16 av[DT];
            tr_read_page<DT>(av, slab + src);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, av[dt]), pb, o[dt], 0, 0,
                                                                   0);
        }
        // all lanes are done reading this buffer before the next batch's loads may target it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    Batch<D, PB> ba, bb;
    issue(0, 0, ba);
    for (int bi = 0; bi < nbatch; bi += 2) {
        run(bi, 0, ba, bb);
        run(bi + 1, 1, bb, ba);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // the empty batch issued last targets the first V buffer, reused below
    // wave partial -> LDS: this lane holds O^T[d = 16*dt + 4*grp + r][head n], sum share l, max m (same over a
    // head's lanes)
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();  // every wave is done with its V buffers; reuse the space for the merge
    // the merge reuses the V buffers: partial outputs [NW waves][16 heads][D] in the first, maxima and sums in the
    // second
    float* red_o = reinterpret_cast<float*>(&vbuf0[0][0]);
    float (*red_m)[16] = reinterpret_cast<float (*)[16]>(&vbuf1[0][0]);
    float (*red_l)[16] = red_m + NW;
    if (grp == 0) {
        red_m[w][n] = m;
        red_l[w][n] = l;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_o[(w * 16 + n) * D + 16 * dt + 4 * grp + r] = o[dt][r];
    __syncthreads();
    // each thread finishes four consecutive head dims of one head and stores them as one 16-byte write
    for (int e = tid; e < a.G * (D / 4); e += NW * 64) {
        const int hn = e / (D / 4), d = 4 * (e % (D / 4));
        float M = red_m[0][hn];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, red_m[ww][hn]);
        f32x4 acc = f32x4{};
        float lsum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = red_m[ww][hn];
            const float sc = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            acc += sc * *reinterpret_cast<const f32x4*>(&red_o[(ww * 16 + hn) * D + d]);
            lsum += sc * red_l[ww][hn];
        }
        const size_t row = ((size_t)b * a.C + c) * a.Hq + g * a.G + hn;
        *reinterpret_cast<f32x4*>(&a.opart[row * D + d]) = acc * (1.0f / lsum);
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

// One wave per (sequence, query head). The chunk rows are fetched with 16-byte loads that each cover 64 / (D / 4)
// rows, all rows of a group of 64 chunks in flight at once (a buffer view clipped at the last chunk reads zeros
// past it); lane c holds chunk c's log-sum-exp, and each row's weight reaches the lanes that loaded it by shuffle.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const CombineArgs a) {
    constexpr int LPR = D / 4;      // lanes per partial row
    constexpr int RPL = 64 / LPR;   // partial rows per wave load
    constexpr int NL = 64 / RPL;    // loads per group of 64 chunks
    // wave-uniform (sequence, head): its length is a scalar load and the partial rows' buffer views stay scalar
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int bh = blockIdx.x * 4 + w;
    if (bh >= a.B * a.Hq) return;
    const int b = bh / a.Hq, h = bh % a.Hq;
    const int L = a.lens[b];
    const int nc = min(a.C, (L + a.chunk - 1) / a.chunk);
    // chunk c of this (sequence, head) sits at row (b * C + c) * Hq + h
    const float* lp = a.lpart + (size_t)b * a.C * a.Hq + h;
    const float* op = a.opart + ((size_t)b * a.C * a.Hq + h) * D;
    const int hs = a.Hq;
    uint16_t* orow = a.o + (size_t)bh * D;
    if (nc == 0) {
        for (int d = lane; d < D; d += 64) orow[d] = 0;
        if (a.lse && lane == 0) a.lse[bh] = -INFINITY;
        return;
    }
    const int rr = lane / LPR, dq = 4 * (lane % LPR);
    // the rows of a group of 64 chunks, requested at once (those of the first group before the maximum is known)
    auto load_rows = [&](int c0, f32x4 (&v)[NL]) {
        const int rows = min(64, nc - c0);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(op + (size_t)c0 * hs * D), (short)0, ((rows - 1) * hs * D + D) * 4, 0x00020000);
#pragma unroll
        for (int i = 0; i < NL; ++i)
            v[i] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, ((RPL * i + rr) * hs * D + dq) * 4, 0, 0));
    };
    f32x4 v[NL];
    load_rows(0, v);
    const float lp0 = lane < nc ? lp[(size_t)lane * hs] : -INFINITY;
    float M = lp0;
    for (int c0 = 64; c0 < nc; c0 += 64) M = fmaxf(M, c0 + lane < nc ? lp[(size_t)(c0 + lane) * hs] : -INFINITY);
    M = wave_max(M);
    f32x4 acc = f32x4{};
    float sw = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += 64) {
        if (c0 > 0) load_rows(c0, v);
        const float lv = c0 == 0 ? lp0 : (c0 + lane < nc ? lp[(size_t)(c0 + lane) * hs] : -INFINITY);
        const float wl = lv == -INFINITY ? 0.0f : expf(lv - M);
        sw += wl;
#pragma unroll
        for (int i = 0; i < NL; ++i) acc += __shfl(wl, RPL * i + rr) * v[i];
    }
#pragma unroll
    for (int sh = LPR; sh < 64; sh <<= 1)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] += __shfl_xor(acc[k], sh);
    sw = wave_sum(sw);
    const float inv = 1.0f / sw;
    if (rr == 0) {
        const uint32_t w0 = pack_bf16x2(acc[0] * inv, acc[1] * inv), w1 = pack_bf16x2(acc[2] * inv, acc[3] * inv);
        *reinterpret_cast<u32x2*>(orow + dq) = u32x2{w0, w1};
    }
    if (a.lse && lane == 0) a.lse[bh] = M + logf(sw);
}

// ------------------------------------------------------------------------------------------------- fp8 cache
// The same split over an E4M3 cache: K pages token-major [16 x D] bytes, V pages transposed [D x 16] bytes, one
// scale per cache. Every load moves 16 bytes per lane. A lane reads 16 consecutive bytes of its token's key row per
// 64 head dims; the head dims of the S^T product's contraction are taken in that order (the query operand uses the
// same order, so the sum is unchanged). The transposed value pages go to LDS whole (one 1 KiB direct load per 64
// head dims) and come back as the 4 consecutive tokens of one head-dim row that the A operand of the O^T product
// holds per lane. Codes are widened to bf16 by the hardware conversion (exact: every E4M3 value is a bf16 number).
// k_scale is folded into the exponent scale and v_scale into the final normalisation.
struct SplitArgs8 {
    const uint16_t* q;
    const uint8_t* kc;
    const uint8_t* vc;
    const int32_t* bt;
    const int32_t* lens;
    float* opart;
    float* lpart;
    int B, Hq, Hkv, G, max_pages, num_pages, C, chunk, ppw;
    float c2;       // softmax scale * log2(e) * k_scale
    float vscale;
};

// bytes 0-1 (HI false) or 2-3 (HI true) of w as two bf16
template <bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <int D, int PB>
struct Batch8 {
    u32x4 k[PB][D / 64];     // 16 key bytes per 64 head dims
    int tok0;
};

template <int D, int NW, int PB>
__global__ __launch_bounds__(NW * 64) void decode_split_fp8_kernel(const SplitArgs8 a) {
    constexpr int KS = D / 32, DT = D / 16;
    constexpr int KL = D / 64;                    // 16-byte key loads per lane and page
    constexpr int VPAGE = kPage * D;              // bytes of one transposed value page
    constexpr int VL = VPAGE / 1024;              // 1 KiB direct loads per value page
    // the two V buffers are distinct arrays, so reads of one are known not to alias loads into the other
    __shared__ __attribute__((aligned(1024))) char vbuf0[NW][PB * VPAGE];
    __shared__ __attribute__((aligned(1024))) char vbuf1[NW][PB * VPAGE];
    __shared__ float red_o[NW * 16 * D];
    __shared__ float red_m[NW][16], red_l[NW][16];
    const int g = (int)(blockIdx.x % a.Hkv), c = (int)(blockIdx.x / a.Hkv), b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, grp = lane >> 4;
    const int L = a.lens[b];
    const int wpage0 = c * (a.chunk / kPage) + w * a.ppw;
    const int32_t* btrow = a.bt + (size_t)b * a.max_pages;
    const int my_page = wpage0 + lane;
    const int my_pid = (lane < a.ppw && my_page < a.max_pages) ? btrow[my_page] : 0;
    // query operand in the key loads' head-dim order: k-slot i of lane group grp in step ks is head dim
    // 64 * (ks / 2) + 16 * grp + 8 * (ks % 2) + i
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = n < a.G ? __builtin_bit_cast(bf16x8, load16(a.q + ((size_t)b * a.Hq + g * a.G + n) * D +
                                                                 64 * (ks >> 1) + 16 * grp + 8 * (ks & 1)))
                         : bf16x8{};
    if (c * a.chunk >= L) return;  // uniform over the work-group

    const int npages_seq = (L + kPage - 1) / kPage;
    const int nbatch = ((a.ppw + 2 * PB - 1) / (2 * PB)) * 2;
    constexpr int kLoads = (KL + VL) * PB;   // vector loads per batch
    static_assert(kLoads < 64, "vmcnt holds at most 63");

    auto issue = [&](int bi, int buf, Batch8<D, PB>& bt) {
        bt.tok0 = (wpage0 + bi * PB) * kPage;
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const int lp = wpage0 + bi * PB + p;
            const bool inrange = bi * PB + p < a.ppw && lp < npages_seq && lp < a.max_pages;
            int pid = inrange ? __builtin_amdgcn_readlane(my_pid, min(bi * PB + p, 63)) : 0;
            int valid = inrange ? min(kPage, L - lp * kPage) : 0;
            if ((unsigned)pid >= (unsigned)a.num_pages) {
                pid = 0;
                valid = 0;
            }
            const uint8_t* kbase = a.kc + ((size_t)pid * a.Hkv + g) * (size_t)(kPage * D);
            const uint8_t* vbase = a.vc + ((size_t)pid * a.Hkv + g) * (size_t)(kPage * D);
            // key rows past the sequence end read as zeros; the value page is read whole (its tokens are the
            // inner dimension) and its bytes past the end are cleared after the LDS read
            const __amdgpu_buffer_rsrc_t kr =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kbase), (short)0, valid * D, 0x00020000);
            const __amdgpu_buffer_rsrc_t vr =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vbase), (short)0, valid ? VPAGE : 0,
                                                  0x00020000);
#pragma unroll
            for (int h = 0; h < KL; ++h)
                bt.k[p][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                           kr, n * D + 64 * h + 16 * grp, 0, 0));
            lds_char* dst = (buf ? (lds_char*)&vbuf1[w][0] : (lds_char*)&vbuf0[w][0]) + p * VPAGE;
#pragma unroll
            for (int i = 0; i < VL; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(dst + i * 1024),
                                                         16, (i * 64 + lane) * 16, 0, 0, 0);
        }
    };

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{};
    float m = -INFINITY, l = 0.0f;
    bf16x2 ones;
    ones[0] = (__bf16)1.0f;
    ones[1] = (__bf16)1.0f;

    auto run = [&](int bi, int buf, Batch8<D, PB>& cur, Batch8<D, PB>& nxt) {
        issue(bi + 1, buf ^ 1, nxt);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (kLoads & 15) | ((kLoads >> 4) << 14));
        f32x4 s[PB];
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            s[p] = f32x4{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint32_t w0 = cur.k[p][ks >> 1][2 * (ks & 1)], w1 = cur.k[p][ks >> 1][2 * (ks & 1) + 1];
                const u32x4 kw = {widen2<false>(w0), widen2<true>(w0), widen2<false>(w1), widen2<true>(w1)};
                s[p] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qf[ks], s[p], 0, 0, 0);
            }
            const int tok = cur.tok0 + p * kPage + 4 * grp;
            const bool page_in_wave = bi * PB + p < a.ppw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (tok + r >= L || !page_in_wave) s[p][r] = -INFINITY;
                mx = fmaxf(mx, s[p][r]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxs = mx * a.c2;
        if (mxs > m) {
            const float alpha = __builtin_amdgcn_exp2f(m - mxs);
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            m = mxs;
        }
        const float bias = (m == -INFINITY) ? 0.0f : -m;
        // the value pages of this batch must be visible to every lane of the wave before the LDS reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][0], a.c2, bias));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][1], a.c2, bias));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][2], a.c2, bias));
            const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[p][3], a.c2, bias));
            const uint32_t w0 = pack_bf16x2(p0, p1), w1 = pack_bf16x2(p2, p3);
            const bf16x4 pb = __builtin_bit_cast(bf16x4, (u32x2{w0, w1}));
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, l, false);
            l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, l, false);
            // this lane's tokens 4*grp .. 4*grp+3 that exist; bytes past the sequence end are cleared
            const int valid = min(kPage, L - (cur.tok0 + p * kPage));
            const int nv = min(max(valid - 4 * grp, 0), 4);
            const uint32_t keep = nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);
            const lds_char* vp = (buf ? (const lds_char*)&vbuf1[w][0] : (const lds_char*)&vbuf0[w][0]) + p * VPAGE;
            // V^T[d = 16*dt + n][tokens 4*grp .. 4*grp+3] is the A operand of the 16x16x16 product as read
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint32_t vw4 =
                    *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(vp + (16 * dt + n) * kPage +
                                                                                         4 * grp) & keep;
                const u32x2 vw = {widen2<false>(vw4), widen2<true>(vw4)};
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vw), pb, o[dt], 0, 0, 0);
            }
        }
        // all lanes are done reading this buffer before the next batch's loads may target it
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    Batch8<D, PB> ba, bb;
    issue(0, 0, ba);
    for (int bi = 0; bi < nbatch; bi += 2) {
        run(bi, 0, ba, bb);
        run(bi + 1, 1, bb, ba);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // the empty batch issued last
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (grp == 0) {
        red_m[w][n] = m;
        red_l[w][n] = l;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_o[(w * 16 + n) * D + 16 * dt + 4 * grp + r] = o[dt][r];
    __syncthreads();
    for (int e = tid; e < a.G * (D / 4); e += NW * 64) {
        const int hn = e / (D / 4), d = 4 * (e % (D / 4));
        float M = red_m[0][hn];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, red_m[ww][hn]);
        f32x4 acc = f32x4{};
        float lsum = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = red_m[ww][hn];
            const float sc = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            acc += sc * *reinterpret_cast<const f32x4*>(&red_o[(ww * 16 + hn) * D + d]);
            lsum += sc * red_l[ww][hn];
        }
        const size_t row = ((size_t)b * a.C + c) * a.Hq + g * a.G + hn;
        *reinterpret_cast<f32x4*>(&a.opart[row * D + d]) = acc * (a.vscale / lsum);
        if (d == 0) a.lpart[row] = (M + log2f(lsum)) * kLn2;
    }
}

template <int D, int NW>
void launch_split8(int pb, dim3 grid, const SplitArgs8& a, hipStream_t s) {
    const dim3 block(NW * 64);
    if (pb == 2) hipLaunchKernelGGL((decode_split_fp8_kernel<D, NW, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_split_fp8_kernel<D, NW, 4>), grid, block, 0, s, a);
}

template <int D>
void launch_split8(int nw, int pb, dim3 grid, const SplitArgs8& a, hipStream_t s) {
    if (nw == 1) launch_split8<D, 1>(pb, grid, a, s);
    else if (nw == 2) launch_split8<D, 2>(pb, grid, a, s);
    else launch_split8<D, 4>(pb, grid, a, s);
}

template <int D, int NW>
void launch_split(int pb, dim3 grid, const SplitArgs& a, hipStream_t s) {
    const dim3 block(NW * 64);
    if (pb == 2) hipLaunchKernelGGL((decode_split_kernel<D, NW, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_split_kernel<D, NW, 4>), grid, block, 0, s, a);
}

template <int D>
void launch_split(int nw, int pb, dim3 grid, const SplitArgs& a, hipStream_t s) {
    if (nw == 1) launch_split<D, 1>(pb, grid, a, s);
    else if (nw == 2) launch_split<D, 2>(pb, grid, a, s);
    else launch_split<D, 4>(pb, grid, a, s);
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int D, int chunk, int max_seq_len) {
    const size_t C = (size_t)((max_seq_len + chunk - 1) / chunk);
    const size_t o_bytes = (size_t)B * Hq * (C ? C : 1) * D * sizeof(float);
    const size_t l_bytes = (size_t)B * Hq * (C ? C : 1) * sizeof(float);
    return ((o_bytes + 255) / 256) * 256 + ((l_bytes + 255) / 256) * 256;
}

// The chunk merge both caches share.
hipError_t launch_combine(const DecodeProblem& p, const float* opart, const float* lpart, int C, hipStream_t s) {
    CombineArgs cb;
    cb.opart = opart;
    cb.lpart = lpart;
    cb.lens = p.seq_lens;
    cb.o = static_cast<uint16_t*>(p.o);
    cb.lse = p.lse;
    cb.B = p.B;
    cb.Hq = p.Hq;
    cb.C = C;
    cb.chunk = p.chunk;
    const dim3 grid2((unsigned)((p.B * p.Hq + 3) / 4));
    if (p.D == 64) hipLaunchKernelGGL((decode_combine_kernel<64>), grid2, dim3(256), 0, s, cb);
    else hipLaunchKernelGGL((decode_combine_kernel<128>), grid2, dim3(256), 0, s, cb);
    return hipGetLastError();
}

hipError_t launch_decode_paged_fp8(const DecodeProblem& p, float k_scale, float v_scale, void* workspace,
                                   hipStream_t s) {
    const int C = (p.max_seq_len + p.chunk - 1) / p.chunk;
    const size_t o_bytes = (size_t)p.B * p.Hq * (C ? C : 1) * p.D * sizeof(float);
    SplitArgs8 a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.kc = static_cast<const uint8_t*>(p.k_cache);
    a.vc = static_cast<const uint8_t*>(p.v_cache);
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
    // two waves per work-group up to 128 pages per chunk, four beyond (a wave holds at most 64 pages' block-table
    // entries); on the paged workload (512-token chunks) two waves of 16 pages measured 4.6% faster than one of 32
    // and 2.7% faster than four of 8, and 4 pages per batch beat 8
    const int pages = p.chunk / kPage;
    const int nw = pages <= 128 ? 2 : 4;
    const int pb = p.D == 64 ? 4 : 2;
    a.ppw = p.chunk / kPage / nw;
    a.c2 = p.scale * kLog2e * k_scale;
    a.vscale = v_scale;
    if (C > 0) {
        const dim3 grid((unsigned)(C * p.Hkv), (unsigned)p.B);
        if (p.D == 64) launch_split8<64>(nw, pb, grid, a, s);
        else launch_split8<128>(nw, pb, grid, a, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_combine(p, a.opart, a.lpart, a.C, s);
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
    // waves per work-group and pages per batch: about 16 pages per wave (all shapes from 8 to 32 pages per wave and
    // 2 or 4 pages per batch measured within 3% of each other on the paged workload, this one at the front); a wave
    // holds at most 64 pages' block-table entries, one per lane, which 4 waves reach at the largest chunk
    const int pages = p.chunk / kPage;
    const int nw = pages <= 16 ? 1 : pages <= 32 ? 2 : 4;
    const int pb = p.D == 64 ? 4 : 2;
    a.ppw = p.chunk / kPage / nw;
    a.c2 = p.scale * kLog2e;
    if (C > 0) {
        const dim3 grid((unsigned)(C * p.Hkv), (unsigned)p.B);   // kv head fastest: neighbours share pages
        if (p.D == 64) launch_split<64>(nw, pb, grid, a, s);
        else launch_split<128>(nw, pb, grid, a, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_combine(p, a.opart, a.lpart, a.C, s);
}

// Chunk partials of attn_decode_paged_noalloc: a file-scope device array, one copy per GPU, held until the process
// ends. Host code never uses the array's name as an address (on the host it is only a stand-in for the symbol): the
// device address is looked up once per device with hipGetSymbolAddress and cached.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
    static std::mutex mu;
    static std::vector<void*> per_device;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)per_device.size() <= dev) per_device.resize(dev + 1, nullptr);
    if (!per_device[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

}  // namespace lcattn
