// Causal prefill kernels for gfx950: dense GQA (bf16 MFMA), block-sparse (same tile body walking a kept-block
// list) and a plain fp32 path.
//
// Method ("attention-kernel-optimization", section "FlashAttention (1 -> 2 -> 3)"): K/V are streamed through
// on-chip memory in tiles, each query row keeps a running max and sum, and earlier partial results are
// rescaled whenever the max moves, so the score matrix never leaves the chip and the result equals plain
// softmax attention up to rounding.
//
// bf16 tile body (one wave = 32 query rows of one head, one KV tile = 64 keys, or 32 for 64-row sparse blocks):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the wave's Q rows held in VGPRs for
//   the whole work-group. In the 32x32 accumulator layout lane l owns query column l%32 and 16 keys, so a row
//   max is an in-lane chain of three-input maxima plus one exchange with lane l^32.
//   O^T += V^T P^T with the same MFMA: the bf16-rounded probabilities are already in B-operand order in the
//   lane that computed them (no LDS round trip); V stays in its natural row-major layout in LDS and each A
//   operand is two ds_read_b64_tr_b16 reads, which transpose 4 keys x 16 head dims per 16-lane group.
//   The running max is refreshed lazily: only when a tile's max exceeds it by more than 2^8, which keeps
//   every exp2 argument <= 8 and skips the O rescale on almost every tile. The final normalisation uses the
//   same max, so the result is unchanged up to rounding.
//   The row sum adds the bf16-rounded probabilities (v_dot2_f32_bf16), i.e. exactly the weights the PV
//   product uses.
// Staging: K and V tiles go from HBM straight into LDS (buffer_load ... lds, 16 bytes per lane, no staging
// registers).
// Schedule: every work-group walks its tiles single-buffered (QK, softmax, PV per tile; the next K tile requested
// once every wave is done with the current one, the next V tile once PV is done), small enough in LDS and registers
// that several work-groups share each CU and overlap each other's loads, softmax and MFMA streams.
// The file is compiled without NaN semantics (see the build script): a max then needs no quieting of its inputs.
#include "device_common.hpp"
#include "internal.hpp"

namespace lcattn {
namespace {

constexpr int kBN = 64;        // keys per KV tile
constexpr int kPageTokens = 16; // tokens per page of a paged cache
constexpr int kDenseWaves = 4; // waves per dense work-group
constexpr float kSlack = 8.0f; // lazy-rescale threshold, log2 units

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// K and V tiles (64 keys x D, bf16) live in LDS row-major with padded row strides chosen for gfx950's LDS, whose 64
// four-byte banks span 256 bytes, i.e. 16 slots of 16 bytes:
//   - a 16-byte K read serves 16 lanes at a time: 16 consecutive rows at one chunk. A K row stride of an odd number
//     of 16-byte chunks (D/8 + 1) puts them on 16 distinct slots.
//   - a transposed V read serves 32 lanes at a time: 4 consecutive keys (the first a multiple of 4) x 4 consecutive
//     chunks (likewise). A V row stride of D/8 + 4 chunks, i.e. 4 (D = 128) or 12 (D = 64) modulo 16, moves the
//     four keys' chunk groups onto four disjoint groups of slots.
// Both reads are then a per-lane base plus a compile-time offset, with no address arithmetic per read. (An XOR
// swizzle of the unpadded rows can avoid the conflicts too, but costs address work per read and registers.)
template <int D>
struct Lds {
    static constexpr int ROWB = D * 2;              // bytes per key row in HBM
    static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
    static constexpr int KSTR = ROWB + 16;          // LDS row stride of a K tile
    static constexpr int VSTR = ROWB + 64;          // LDS row stride of a V tile
    static constexpr int KTILE = kBN * KSTR;        // bytes of one K tile (a multiple of 1 KiB)
    static constexpr int VTILE = kBN * VSTR;
    static_assert(KTILE % 1024 == 0 && VTILE % 1024 == 0, "tiles are filled by whole 1 KiB direct loads");
};

// One head's K or V slab. The host rejects shapes whose slab reaches 2^31 bytes, so `bytes` and every tile offset
// kv0 * ROWB below stay within a signed 32-bit int.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes, 0x00020000);
}

// Direct global->LDS staging of one tile (row stride STR in LDS) by the work-group's NW waves: each 64-lane load
// moves 1 KiB into consecutive LDS bytes, lane l's 16 bytes to position l; the lane fetches the global chunk that
// lands there (a padding slot re-reads a chunk of the same row, so it costs no extra memory traffic). Buffer range
// checking returns zeros for keys outside [0, N) (including negative tile starts).
// A tile of BN rows whose bytes are not a whole number of loads gets one more load; its lanes past the last row
// carry an offset beyond any buffer (no fetch; the LDS bytes they fill lie in the tile's rounded-up allocation).
template <int D, int NW, int STR, int BN = kBN>
struct TileLoader {
    static constexpr int LOADS = (BN * STR + 1023) / 1024;
    static constexpr int PER = (LOADS + NW - 1) / NW;
    static constexpr int SPR = STR / 16;   // 16-byte slots per LDS row
    int voff[PER];
    int first;   // this wave's first load slot
    __device__ __forceinline__ void init(int w, int lane) {
        first = w * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int z = (first + i) * 64 + lane;   // 16-byte slot inside the tile
            const int r = z / SPR, c = z % SPR;
            voff[i] = r * Lds<D>::ROWB + min(c, Lds<D>::CPR - 1) * 16;
            if constexpr (BN * STR % 1024 != 0)
                if (r >= BN) voff[i] = (int)0x80000000u;   // with soff < 2^31 the sum stays past the buffer end
        }
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, lds_char* tile, int kv0) const {
        const int soff = kv0 * Lds<D>::ROWB;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (LOADS % NW == 0 || first + i < LOADS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (first + i) * 1024),
                                                         16, voff[i], soff, 0, 0);
    }
};

template <int D, int NW, int BN = kBN>
struct Loaders {
    TileLoader<D, NW, Lds<D>::KSTR, BN> k;
    TileLoader<D, NW, Lds<D>::VSTR, BN> v;
    __device__ __forceinline__ void init(int w, int lane) {
        k.init(w, lane);
        v.init(w, lane);
    }
};

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

template <int D>
struct RowState {
    f32x16 o[D / 32];
    float m;  // running max of scale*log2(e)*score (log2 units), -inf before the first key
    float l;  // this lane's share of the row sum
};

// S^T for one tile: T2 32x32 blocks (keys x this wave's 32 query rows; T2 = 2 for 64-key tiles, 1 for 32-key
// tiles), accumulated alternately. Fixed schedule: each K read is issued two MFMAs ahead of its use, and hard
// scheduling barriers keep that order; this measured 2-4% faster than the compiler's own order, bit for bit the
// same result. K rows sit KSTR bytes apart, or, for a tile gathered from 16-row pages (PSLOT > 0), in page slots
// PSLOT bytes apart: row r at (r / 16) * PSLOT + (r % 16) * KSTR. Either way every read is one per-lane base plus a
// compile-time offset. (The paged kernel's swizzled variant below keeps the compiler's order: with this schedule
// its D = 128 kernel spills registers.)
template <int D, int T2 = 2, int PSLOT = 0>
__device__ __forceinline__ void qk_tile_sched(const lds_char* kl, const bf16x8 (&qf)[D / 16], f32x16 (&s)[T2],
                                              int lane) {
    constexpr int NQK = (D / 16) * T2;   // (D / 16) k-steps x T2 key halves
    constexpr int AH = 2;
    const int hi = lane >> 5, ln = lane & 31;
    const lds_char* kp = kl + (ln / 16) * PSLOT + (ln % 16) * Lds<D>::KSTR;   // paged: this lane's row in page 0
    auto kread = [&](int i) {
        const int ks = i / T2, t = i % T2;
        const lds_char* at = PSLOT ? kp + 2 * t * PSLOT : kl + (32 * t + ln) * Lds<D>::KSTR;   // key half t: row 32t
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(at + (2 * ks + hi) * 16);
    };
    bf16x8 kf[NQK];
#pragma unroll
    for (int t = 0; t < T2; ++t) s[t] = f32x16{};
#pragma unroll
    for (int i = 0; i < AH; ++i) kf[i] = kread(i);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
        if (i + AH < NQK) kf[i + AH] = kread(i + AH);
        s[i % T2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i / T2], s[i % T2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ float pair_max(float x) {
    // lanes l and l^32 hold the two halves of one query row's keys
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Online-softmax update for one tile, first half: element mask on a diagonal tile, row max, lazy refresh of the
// running max (rescaling O and the sum when it moves by more than kSlack). Returns the exp2 bias.
template <int D, int T2 = 2>
__device__ __forceinline__ float softmax_max(f32x16 (&s)[T2], RowState<D>& st, float c2, bool diag, int kv0, int qrow,
                                             int lane) {
    const int hi = lane >> 5;
    if (diag) {
#pragma unroll
        for (int t = 0; t < T2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
                s[t][r] = key > qrow ? -INFINITY : s[t][r];
            }
    }
    // one chain of three-input maxima per key half (v_max3_f32: two values per instruction)
    float c[T2];
#pragma unroll
    for (int t = 0; t < T2; ++t) {
        c[t] = fmaxf(fmaxf(s[t][0], s[t][1]), s[t][2]);
#pragma unroll
        for (int r = 3; r + 1 < 16; r += 2) c[t] = fmaxf(fmaxf(c[t], s[t][r]), s[t][r + 1]);
        c[t] = fmaxf(c[t], s[t][15]);
    }
    float cm = c[0];
#pragma unroll
    for (int t = 1; t < T2; ++t) cm = fmaxf(cm, c[t]);
    const float mx = pair_max(cm);
    const float mxs = mx * c2;
    if (mxs > st.m + kSlack) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - mxs);
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) st.o[dt] *= alpha;
        st.m = mxs;
    }
    return (st.m == -INFINITY) ? 0.0f : -st.m;
}

// Second half, one slice: the two probabilities of accumulator slots 2w and 2w+1 of key half t, rounded to bf16 and
// packed in the B-operand order of the PV product; their sum (of the rounded values) goes into l.
template <int T2 = 2>
__device__ __forceinline__ void softmax_slice(const f32x16 (&s)[T2], uint32_t (&pw)[T2][8], int t, int w, float c2,
                                              float bias, float& l) {
    bf16x2 ones;
    ones[0] = (__bf16)1.0f;
    ones[1] = (__bf16)1.0f;
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * w], c2, bias));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * w + 1], c2, bias));
    pw[t][w] = pack_bf16x2(p0, p1);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[t][w]), ones, l, false);
}

// Whole online-softmax update for one tile.
template <int D, int T2 = 2>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[T2], uint32_t (&pw)[T2][8], RowState<D>& st, float c2,
                                             bool diag, int kv0, int qrow, int lane) {
    const float bias = softmax_max<D, T2>(s, st, c2, diag, kv0, qrow, lane);
    float l0 = st.l, l1 = 0.0f;
#pragma unroll
    for (int t = 0; t < T2; ++t)
#pragma unroll
        for (int w = 0; w < 8; ++w) softmax_slice<T2>(s, pw, t, w, c2, bias, (w & 1) ? l1 : l0);
    st.l = l0 + l1;
}

// Per-lane byte offsets of the transposed V reads. The A operand of a PV MFMA holds, in lane (ln, hi), the head
// dim d = 32*dt + ln for the eight keys of slots 8*hi .. 8*hi+7; two ds_read_b64_tr_b16 produce them, each
// giving a 16-lane group 16 consecutive d for 4 consecutive keys: source lane 4*jj + a of the group points at
// V[key_jj][d0 + 4a], and output lane i receives V[key_0..3][d0 + i].
template <int D>
struct VtAddr {
    int key_lo;  // this lane's source key inside a 16-key slice: 4*hi + jj (the second read adds 8)
    int dq;      // this lane's source head-dim offset inside a 32-wide tile: 16*half + 4*a
    __device__ __forceinline__ void init(int lane) {
        key_lo = 4 * (lane >> 5) + ((lane & 15) >> 2);
        dq = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    }
    __device__ __forceinline__ int at(int key, int d) const {
        return key * Lds<D>::VSTR + d * 2;
    }
};

// O^T += V^T P^T over a 64-key tile in the compiler's order (the paged walk).
template <int D>
__device__ __forceinline__ void pv_tile(const lds_char* vl, const VtAddr<D>& va, const uint32_t (&pw)[2][8],
                                        RowState<D>& st) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 b = __builtin_bit_cast(
                bf16x8, (u32x4{pw[t][4 * u], pw[t][4 * u + 1], pw[t][4 * u + 2], pw[t][4 * u + 3]}));
            const int key = 32 * t + 16 * u + va.key_lo;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int d = 32 * dt + va.dq;
                typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + va.at(key, d)));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + va.at(key + 8, d)));
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, (u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                   __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]}));
                st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, st.o[dt], 0, 0, 0);
            }
        }
}

// O^T += V^T P^T with the fixed schedule of qk_tile_sched: the two transposed reads of each MFMA's A operand are
// issued two MFMAs ahead.
template <int D, int T2 = 2>
__device__ __forceinline__ void pv_tile_sched(const lds_char* vl, const VtAddr<D>& va, const uint32_t (&pw)[T2][8],
                                              RowState<D>& st) {
    constexpr int NPV = T2 * (D / 16);   // T2 key halves x 2 16-key slices x (D / 32) head-dim tiles
    constexpr int AH = 2;
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    auto vread = [&](int j, v4i16& lo, v4i16& hi4) {
        const int t = j / (2 * (D / 32)), u = (j / (D / 32)) & 1, dt = j % (D / 32);
        const int key = 32 * t + 16 * u + va.key_lo, d = 32 * dt + va.dq;
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + va.at(key, d)));
        hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vl + va.at(key + 8, d)));
    };
    v4i16 vlo[NPV], vhi[NPV];
#pragma unroll
    for (int j = 0; j < AH; ++j) vread(j, vlo[j], vhi[j]);
#pragma unroll
    for (int j = 0; j < NPV; ++j) {
        if (j + AH < NPV) vread(j + AH, vlo[j + AH], vhi[j + AH]);
        const int t = j / (2 * (D / 32)), u = (j / (D / 32)) & 1, dt = j % (D / 32);
        const bf16x8 b = __builtin_bit_cast(
            bf16x8, (u32x4{pw[t][4 * u], pw[t][4 * u + 1], pw[t][4 * u + 2], pw[t][4 * u + 3]}));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, (u32x4{__builtin_bit_cast(u32x2, vlo[j])[0], __builtin_bit_cast(u32x2, vlo[j])[1],
                           __builtin_bit_cast(u32x2, vhi[j])[0], __builtin_bit_cast(u32x2, vhi[j])[1]}));
        st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, st.o[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qf)[D / 16], const uint16_t* qh, int qrow, int N, int lane) {
    const int hi = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        qf[ks] = qrow < N ? __builtin_bit_cast(bf16x8, load16(qh + (size_t)qrow * D + 16 * ks + 8 * hi))
                          : bf16x8{};
}

template <int D>
__device__ __forceinline__ void finish_rows(const RowState<D>& st, uint16_t* oh, float* lse_row, int qrow, int N,
                                            int lane) {
    const int hi = lane >> 5;
    const float lt = pair_sum(st.l);
    if (qrow >= N) return;
    const float inv = 1.0f / lt;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d0 = 32 * dt + 8 * a + 4 * hi;
            u32x2 w;
            w[0] = pack_bf16x2(st.o[dt][4 * a] * inv, st.o[dt][4 * a + 1] * inv);
            w[1] = pack_bf16x2(st.o[dt][4 * a + 2] * inv, st.o[dt][4 * a + 3] * inv);
            *reinterpret_cast<u32x2*>(oh + (size_t)qrow * D + d0) = w;
        }
    if (lse_row && hi == 0) lse_row[qrow] = (st.m + log2f(lt)) * kLn2;
}

template <int D>
__device__ __forceinline__ void init_state(RowState<D>& st) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) st.o[dt] = f32x16{};
    st.m = -INFINITY;
    st.l = 0.0f;
}

struct DenseArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, Hq, Hkv, N, G;
    int HPW;       // query heads of one kv group handled by a work-group
    int NHG;       // G / HPW
    int PPW;       // query positions per work-group
    int n_ptiles;  // ceil(N / PPW)
    float c2;      // scale * log2(e)
};


// Single-buffered tile walk: one K and one V tile in LDS. The next K tile is requested as soon as every wave has
// finished this tile's QK product (it lands during the softmax and PV), the next V tile once PV is done. With half
// the LDS of a double-buffered walk, twice as many work-groups share a CU and cover each other's load latency.
template <int D, int NW, typename KvOf, int T2 = 2>
__device__ __forceinline__ void attend_sb(const lds_char* kl, const lds_char* vl, __amdgpu_buffer_rsrc_t krs,
                                          __amdgpu_buffer_rsrc_t vrs, int ntiles, KvOf kv_of,
                                          const bf16x8 (&qf)[D / 16], RowState<D>& st, float c2, int q0, int w,
                                          int lane) {
    constexpr int BN = 32 * T2;   // keys per tile
    Loaders<D, NW, BN> ld;
    ld.init(w, lane);
    VtAddr<D> va;
    va.init(lane);
    const int qrow = q0 + (lane & 31);
    int kv = kv_of(0);
    ld.k.load(krs, (lds_char*)kl, kv);
    ld.v.load(vrs, (lds_char*)vl, kv);
    for (int j = 0; j < ntiles; ++j) {
        const int kv_n = j + 1 < ntiles ? kv_of(j + 1) : 0;
        wait_vmem();
        __syncthreads();
        f32x16 s[T2];
        uint32_t pw[T2][8];
        qk_tile_sched<D, T2>(kl, qf, s, lane);
        __syncthreads();   // every wave is done with K(j)
        if (j + 1 < ntiles) ld.k.load(krs, (lds_char*)kl, kv_n);
        softmax_tile<D, T2>(s, pw, st, c2, kv + BN - 1 > q0, kv, qrow, lane);
        pv_tile_sched<D, T2>(vl, va, pw, st);
        __syncthreads();   // and with V(j)
        if (j + 1 < ntiles) ld.v.load(vrs, (lds_char*)vl, kv_n);
        kv = kv_n;
    }
}

// Dense kernel. Work-group = HPW query heads of one kv group x PPW consecutive positions, one wave per head and
// 32-row slice (4 waves), all sharing each staged K/V tile; the single-buffered walk keeps a work-group at 38 KB of
// LDS and the register budget is held to three waves per SIMD, so three work-groups share a CU and overlap each
// other's loads, softmax and MFMA streams. Work-groups are issued heaviest (latest positions) first, and the kv head
// cycles fastest so that, with 8 XCDs dispatched round-robin, an XCD keeps seeing the same kv heads.
template <int D>
__global__ __launch_bounds__(kDenseWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_dense_kernel(const DenseArgs a) {
    __shared__ __attribute__((aligned(1024))) char k0[Lds<D>::KTILE];
    __shared__ __attribute__((aligned(1024))) char v0[Lds<D>::VTILE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per_tile = a.B * a.Hkv * a.NHG;
    const int pt = a.n_ptiles - 1 - (int)(blockIdx.x / per_tile);
    int rest = (int)(blockIdx.x % per_tile);
    const int g = rest % a.Hkv;
    rest /= a.Hkv;
    const int hg = rest % a.NHG;
    const int b = rest / a.NHG;
    const int h = g * a.G + hg * a.HPW + (w % a.HPW);
    const int p0 = pt * a.PPW;
    const int q0 = p0 + 32 * (w / a.HPW);
    const int wg_end = min(a.N, p0 + a.PPW);
    const int ntiles = (wg_end + kBN - 1) / kBN;
    const int qrow = q0 + (lane & 31);

    const size_t qoff = ((size_t)b * a.Hq + h) * (size_t)a.N * D;
    const size_t kvoff = ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + kvoff, a.N * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + kvoff, a.N * D * 2);

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + qoff, qrow, a.N, lane);
    RowState<D> st;
    init_state<D>(st);
    // every wave walks the work-group's tiles; a tile wholly past a wave's rows (possible when one work-group spans
    // several 32-row slices) is fully masked for it and adds nothing
    attend_sb<D, kDenseWaves>((lds_char*)k0, (lds_char*)v0, krs, vrs, ntiles, [](int t) { return t * kBN; }, qf, st,
                              a.c2, q0, w, lane);
    finish_rows<D>(st, a.o + qoff, a.lse ? a.lse + ((size_t)b * a.Hq + h) * a.N : nullptr, qrow, a.N, lane);
}

// ---------------------------------------------------------------------------------------- paged prefill
// Chunked prefill over a paged cache ("attention-kernel-optimization", section "PagedAttention"; sliding windows as
// in "Your Context Length Decides What a Kernel Is Worth"): the dense kernel's work-groups, tile body and
// single-buffered walk, with K/V tiles gathered from pages and an optional lower (window) bound on the keys.
struct PagedArgs {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    uint16_t* o;
    float* lse;
    const int32_t* bt;
    const int32_t* lens;
    int B, Hq, Hkv, Nq, G, max_pages, num_pages, window;
    int HPW, NHG, PPW, n_ptiles;
    float c2;
    int splits;             // work-groups sharing one row set's key tiles (gridDim.y); 1 writes O directly
    float* opart;           // splits > 1: [splits, B, Hq, Nq, D] normalised partial outputs
    float* lpart;           // splits > 1: [splits, B, Hq, Nq] their natural-log lse
};

// A split's rows: the output normalised by the split's own sum, and the split's lse (-inf with no key).
template <int D>
__device__ __forceinline__ void finish_partial(const RowState<D>& st, float* orow_base, float* lrow, int qrow, int N,
                                               int lane) {
    const int hi = lane >> 5;
    const float lt = pair_sum(st.l);
    if (qrow >= N) return;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    float* orow = orow_base + (size_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d0 = 32 * dt + 8 * a + 4 * hi;
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = st.o[dt][4 * a + j] * inv;
            *reinterpret_cast<f32x4*>(orow + d0) = v;
        }
    if (hi == 0) lrow[qrow] = lt > 0.0f ? (st.m + log2f(lt)) * kLn2 : -INFINITY;
}

// Page loads: with four waves and 64-key tiles each wave stages exactly one 16-token page of K and one of V. The
// wave builds one buffer view per page (64-bit base at the page's slab, size clipped at the sequence end, so rows
// past it and pages the table does not give read zeros) and issues whole 1 KiB direct-to-LDS loads whose per-lane
// source offsets inside the slab never change. V keeps the dense kernel's padded layout, whose pages are whole
// loads already. K takes one of two layouts:
//   - padded like the dense kernel's (row stride D*2 + 16), each page in a slot rounded up to whole loads (5 KiB at
//     D = 128: the last load's lanes past row 15 fall outside the page's view and fetch nothing), so the scheduled
//     QK product reads it at compile-time offsets;
//   - unpadded and XOR-swizzled (a page is then exactly its loads): 16-byte chunk c of row r sits at chunk
//     c ^ swz(r), which spreads any 16 consecutive rows' reads of one chunk over all banks, at the cost of address
//     arithmetic per read. It needs a fifth less load work and LDS per page, which pays on sliding-window chunks,
//     whose short walks are bound by their loads.
template <int D>
struct SwzK {
    static constexpr int ROWB = D * 2;
    static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
    static constexpr int RPL = 256 / ROWB;         // rows per 256-byte bank line
    static constexpr int TILE = kBN * ROWB;
    __device__ __forceinline__ static int swz(int r) { return (r / RPL) & (CPR - 1); }
};

template <int D, int ROWSTR, bool SWZ>
struct PageLoader {
    static constexpr int ROWB = D * 2;
    static constexpr int CPR = ROWB / 16;
    static constexpr int LPP = (kPageTokens * ROWSTR + 1023) / 1024;   // 1 KiB loads per page
    static constexpr int PAGEB = LPP * 1024;   // LDS slot of one page; slots past row 15 lie outside the page's view
    int voff[LPP];
    __device__ __forceinline__ void init(int lane) {
#pragma unroll
        for (int j = 0; j < LPP; ++j) {
            const int z = j * 64 + lane;   // 16-byte slot inside the page's LDS image
            if constexpr (SWZ) {
                const int r = z / CPR, cl = z % CPR;
                voff[j] = r * ROWB + (cl ^ SwzK<D>::swz(r)) * 16;
            } else {
                constexpr int SPR = ROWSTR / 16;
                const int r = z / SPR, c = z % SPR;
                voff[j] = r * ROWB + min(c, CPR - 1) * 16;   // a padding slot re-reads a chunk of its row
            }
        }
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t page, lds_char* tile, int w) const {
#pragma unroll
        for (int j = 0; j < LPP; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                page, (__attribute__((address_space(3))) void*)(tile + w * PAGEB + j * 1024), 16, voff[j], 0, 0, 0);
    }
};

// S^T of a 64-key tile from the swizzled K layout (the same result as qk_tile).
template <int D>
__device__ __forceinline__ void qk_tile_swz(const lds_char* kl, const bf16x8 (&qf)[D / 16], f32x16 (&s)[2], int lane) {
    const int hi = lane >> 5, ln = lane & 31;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = 32 * t + ln;
            const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                kl + r * SwzK<D>::ROWB + (((2 * ks + hi) ^ SwzK<D>::swz(r)) * 16));
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[t], 0, 0, 0);
        }
}

// Keys at or below qabs - window leave the row.
__device__ __forceinline__ void window_mask(f32x16 (&s)[2], int kv0, int qabs, int window, int lane) {
    const int hi = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key <= qabs - window) s[t][r] = -INFINITY;
        }
}

// PADK selects the K layout (padded with the scheduled tile products, or swizzled with the compiler's order). The
// body is a device function template: with it written in the kernel template itself, the host pass of the compiler
// left the launch stub of one instantiation undefined.
template <int D, bool PADK>
__device__ __forceinline__ void paged_body(const PagedArgs& a) {
    constexpr int NW = kDenseWaves;
    static_assert(NW * kPageTokens == kBN, "one page per wave");
    using KLoader = PageLoader<D, PADK ? Lds<D>::KSTR : SwzK<D>::ROWB, !PADK>;
    static_assert(PADK || KLoader::PAGEB == kPageTokens * SwzK<D>::ROWB, "swizzled K pages are whole loads");
    __shared__ __attribute__((aligned(1024))) char k0[NW * KLoader::PAGEB];
    __shared__ __attribute__((aligned(1024))) char v0[Lds<D>::VTILE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int per_tile = a.B * a.Hkv * a.NHG;
    const int pt = a.n_ptiles - 1 - (int)(blockIdx.x / per_tile);
    int rest = (int)(blockIdx.x % per_tile);
    const int g = rest % a.Hkv;
    rest /= a.Hkv;
    const int hg = rest % a.NHG;
    const int b = rest / a.NHG;
    const int h = g * a.G + hg * a.HPW + (w % a.HPW);
    const int p0 = pt * a.PPW;                    // first chunk row of the work-group
    const int r0 = p0 + 32 * (w / a.HPW);         // first chunk row of this wave
    const int qrow = r0 + (lane & 31);
    const int L = a.lens[b];
    const int base = L - a.Nq;                    // position of chunk row 0
    const int q0abs = base + r0;
    const int qabs = q0abs + (lane & 31);
    const int hi_key = base + min(a.Nq, p0 + a.PPW) - 1;   // latest key any row of the work-group sees
    const int lo_key = a.window > 0 ? max(0, base + p0 - a.window + 1) : 0;
    // tiles start at the page holding the earliest key, so a window's span needs no tile more than it covers
    const int k_first = lo_key / kPageTokens * kPageTokens;
    const int ntiles_all = hi_key >= 0 ? (hi_key - k_first) / kBN + 1 : 0;
    // this work-group's share of the tiles: split blockIdx.y of gridDim.y
    const int per_split = (ntiles_all + a.splits - 1) / a.splits;
    const int ntiles = max(0, min(per_split, ntiles_all - (int)blockIdx.y * per_split));

    const size_t qoff = ((size_t)b * a.Hq + h) * (size_t)a.Nq * D;

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + qoff, qrow, a.Nq, lane);
    RowState<D> st;
    init_state<D>(st);

    KLoader lk;
    PageLoader<D, Lds<D>::VSTR, false> lv;
    static_assert(NW * decltype(lv)::PAGEB == Lds<D>::VTILE, "V pages fill the dense tile layout");
    lk.init(lane);
    lv.init(lane);
    VtAddr<D> va;
    va.init(lane);
    const int32_t* btrow = a.bt + (size_t)b * a.max_pages;
    const int npages = min((L + kPageTokens - 1) / kPageTokens, a.max_pages);
    // this wave's page of the tile starting at key kv0: K and V views clipped at the sequence end
    auto views = [&](int kv0, __amdgpu_buffer_rsrc_t& kr, __amdgpu_buffer_rsrc_t& vr) {
        const int ix = kv0 / kPageTokens + w;
        int pid = ix < npages ? btrow[ix] : -1;
        int valid = min(kPageTokens, L - ix * kPageTokens);
        if ((unsigned)pid >= (unsigned)a.num_pages || valid <= 0) {
            pid = 0;
            valid = 0;
        }
        const size_t slab = ((size_t)pid * a.Hkv + g) * (size_t)(kPageTokens * D);
        kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.kc + slab), (short)0, valid * D * 2, 0x00020000);
        vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.vc + slab), (short)0, valid * D * 2, 0x00020000);
    };
    int kv = k_first + (int)blockIdx.y * per_split * kBN;
    if (ntiles > 0) {
        __amdgpu_buffer_rsrc_t kr, vr;
        views(kv, kr, vr);
        lk.load(kr, (lds_char*)k0, w);
        lv.load(vr, (lds_char*)v0, w);
    }
    for (int j = 0; j < ntiles; ++j) {
        const int kv_n = kv + kBN;
        __amdgpu_buffer_rsrc_t kn, vn;
        views(kv_n, kn, vn);   // past the last tile this is an empty view and is not used
        wait_vmem();
        __syncthreads();
        f32x16 sc[2];
        uint32_t pw[2][8];
        if constexpr (PADK) qk_tile_sched<D, 2, KLoader::PAGEB>((lds_char*)k0, qf, sc, lane);
        else qk_tile_swz<D>((lds_char*)k0, qf, sc, lane);
        __syncthreads();   // every wave is done with K(j)
        if (j + 1 < ntiles) lk.load(kn, (lds_char*)k0, w);
        if (a.window > 0 && kv <= q0abs + 31 - a.window) window_mask(sc, kv, qabs, a.window, lane);
        softmax_tile<D>(sc, pw, st, a.c2, kv + kBN - 1 > q0abs, kv, qabs, lane);
        if constexpr (PADK) pv_tile_sched<D, 2>((lds_char*)v0, va, pw, st);
        else pv_tile<D>((lds_char*)v0, va, pw, st);
        __syncthreads();   // and with V(j)
        if (j + 1 < ntiles) lv.load(vn, (lds_char*)v0, w);
        kv = kv_n;
    }
    if (a.splits == 1) {
        finish_rows<D>(st, a.o + qoff, a.lse ? a.lse + ((size_t)b * a.Hq + h) * a.Nq : nullptr, qrow, a.Nq, lane);
    } else {
        const size_t prow = ((size_t)blockIdx.y * a.B + b) * a.Hq + h;   // (split, b, h)
        finish_partial<D>(st, a.opart + prow * a.Nq * D, a.lpart + prow * a.Nq, qrow, a.Nq, lane);
    }
}

template <int D, bool PADK>
__global__ __launch_bounds__(kDenseWaves * 64) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_paged_kernel(const PagedArgs a) {
    paged_body<D, PADK>(a);
}

// Merge of the key-range splits: each lane merges four head dims of one (b, h, row) with 16-byte loads of the
// fp32 partials, so a wave covers 256 / D rows.
struct PagedCombineArgs {
    const float* opart;
    const float* lpart;
    uint16_t* o;
    float* lse;
    long rows;    // B * Hq * Nq
    int splits;
};

template <int D>
__global__ __launch_bounds__(256) void prefill_paged_combine_kernel(const PagedCombineArgs a) {
    constexpr int LPR = D / 4;      // lanes per row, four head dims (16 bytes of a partial row) each
    constexpr int RPW = 64 / LPR;   // rows per wave
    const int lane = threadIdx.x & 63;
    const long row = ((long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * RPW + lane / LPR;
    if (row >= a.rows) return;   // no barriers in this kernel
    const int d = 4 * (lane % LPR);
    float M = -INFINITY;
    for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, a.lpart[sp * a.rows + row]);
    f32x4 acc = f32x4{};
    float wsum = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp) {
        const float ls = a.lpart[sp * a.rows + row];
        const float w = ls == -INFINITY ? 0.0f : __expf(ls - M);
        wsum += w;
        const f32x4 v = *reinterpret_cast<const f32x4*>(a.opart + ((size_t)sp * a.rows + row) * D + d);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += w * v[j];
    }
    const float inv = 1.0f / wsum;
    u32x2 out;
    out[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    out[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2*>(a.o + (size_t)row * D + d) = out;
    if (a.lse && lane % LPR == 0) a.lse[row] = M + __logf(wsum);
}

struct SparseArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    const int32_t* kv_count;
    const int32_t* kv_index;
    int B, Hq, Hkv, N, G, block, nb;
    float c2;
};

// Work-group = one (batch, head, query block); NW = block / 32 waves. The tile loop walks the row's kept-block
// list (ascending, so the diagonal block, the only one needing an element mask, comes last); skipped blocks
// are never read. Rows are issued latest block first, as they tend to hold the longest lists. Work-groups of two
// waves (64-row blocks, over 32-key tiles) and four waves (128-row blocks, and each half of a 256-row block, over
// 64-key tiles) share a CU six and three at a time (three waves per SIMD, the register budget both are held to).
// A half of a 256-row block walks its diagonal block only as far as its own last row.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_sparse_bf16_kernel(const SparseArgs a) {
    // 64-row blocks walk 32-key tiles: 21 KB of LDS per work-group, so six of them (three waves per SIMD) share a CU
    constexpr int T2 = NW == 2 ? 1 : 2;   // 32-key halves per tile
    constexpr int BN = 32 * T2;
    constexpr int KT = (BN * Lds<D>::KSTR + 1023) / 1024 * 1024, VT = (BN * Lds<D>::VSTR + 1023) / 1024 * 1024;
    __shared__ __attribute__((aligned(1024))) char k0[KT];
    __shared__ __attribute__((aligned(1024))) char v0[VT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile offsets stay in scalar registers
    const int per = a.B * a.Hq;
    // a query block of more than 32 * NW rows (256-row blocks) is split over `parts` work-groups of 32 * NW rows
    const int parts = a.block / (32 * NW);
    const int ib = (int)(blockIdx.x / per);
    const int i = a.nb - 1 - ib / parts;
    const int part = parts - 1 - ib % parts;
    int rest = (int)(blockIdx.x % per);
    // work-groups go to the 8 XCDs round-robin; when the heads split evenly, XCD x takes the x-th run of per / 8
    // heads in kv-group order, so its L2 serves as few kv heads as possible
    if (per % 8 == 0) rest = (rest % 8) * (per / 8) + rest / 8;
    const int h = rest % a.Hq;
    const int b = rest / a.Hq;
    const int g = h / a.G;
    const int q0 = i * a.block + part * 32 * NW + 32 * w;
    const int qrow = q0 + (lane & 31);
    const size_t row = ((size_t)b * a.Hq + h) * a.nb + i;
    const int cnt = a.kv_count[row];
    const int32_t* list = a.kv_index + row * a.nb;
    const int sub = a.block / BN;   // tiles per key block

    const size_t qoff = ((size_t)b * a.Hq + h) * (size_t)a.N * D;
    const size_t kvoff = ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + kvoff, a.N * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + kvoff, a.N * D * 2);

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + qoff, qrow, a.N, lane);
    RowState<D> st;
    init_state<D>(st);
    if (cnt == 0) return;  // every valid list holds the diagonal; an empty one leaves the rows unwritten
    // the row's block list goes to LDS once, as each kept block's first key, so the tile loop finds the next tile's
    // first key with an LDS read and an add instead of a global round trip per tile
    extern __shared__ int lst[];   // nb entries, sized at launch
    const int blk = a.block;
    for (int e = tid; e < cnt; e += NW * 64) lst[e] = list[e] * blk;
    __syncthreads();
    // the diagonal block (the list's last) is walked only up to this work-group's last row
    const int diag_tiles = ((part + 1) * 32 * NW + BN - 1) / BN;
    const int ntiles = (cnt - 1) * sub + (lst[cnt - 1] == i * blk ? diag_tiles : sub);
    // sub is a power of two (block / tile: 2 or 4)
    const int lsub = __builtin_ctz(sub);
    // a tile's first key comes from LDS, which the compiler takes as per-lane; read out once as wave-uniform, so the
    // direct loads get it as their scalar offset instead of looping over lanes for it
    auto kv_of = [&](int t) { return __builtin_amdgcn_readfirstlane(lst[t >> lsub] + (t & (sub - 1)) * BN); };
    attend_sb<D, NW, decltype(kv_of), T2>((lds_char*)k0, (lds_char*)v0, krs, vrs, ntiles, kv_of, qf, st, a.c2, q0,
                                          w, lane);
    finish_rows<D>(st, a.o + qoff, a.lse ? a.lse + ((size_t)b * a.Hq + h) * a.N : nullptr, qrow, a.N, lane);
}

// ---------------------------------------------------------------------------------------------------- fp32
// fp32 end to end (no fp32-input MFMA shortcut with reduced precision exists on gfx950): one query row per
// D/64 lanes, each lane owning 64 of the head dimensions; K/V tiles of 32 keys staged in LDS and read as
// broadcasts; per-key online softmax with expf.
struct F32Args {
    const float* q;
    const float* k;
    const float* v;
    float* o;
    float* lse;
    int B, Hq, Hkv, N, G, n_qt;
    float scale;
};

template <int D>
__global__ __launch_bounds__(64) void prefill_dense_f32_kernel(const F32Args a) {
    constexpr int TPQ = D / 64, QPB = 64 / TPQ, KT = 32;
    __shared__ float ks[KT][D];
    __shared__ float vs[KT][D];
    const int lane = threadIdx.x;
    const int per = a.B * a.Hq;
    const int qt = a.n_qt - 1 - (int)(blockIdx.x / per);
    const int rest = (int)(blockIdx.x % per);
    const int h = rest % a.Hq, b = rest / a.Hq, g = h / a.G;
    const int qi = qt * QPB + lane / TPQ;
    const int dp = (lane % TPQ) * 64;
    const float* qh = a.q + ((size_t)b * a.Hq + h) * (size_t)a.N * D;
    const float* kh = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    const float* vh = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    float qv[64], ov[64];
#pragma unroll
    for (int d = 0; d < 64; ++d) {
        qv[d] = qi < a.N ? qh[(size_t)qi * D + dp + d] : 0.0f;
        ov[d] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const int kv_end = min(a.N, (qt + 1) * QPB);
    for (int kv0 = 0; kv0 < kv_end; kv0 += KT) {
        __syncthreads();
        for (int e = lane; e < KT * D; e += 64) {
            const int r = e / D, c = e % D;
            const bool in = kv0 + r < a.N;
            ks[r][c] = in ? kh[(size_t)(kv0 + r) * D + c] : 0.0f;
            vs[r][c] = in ? vh[(size_t)(kv0 + r) * D + c] : 0.0f;
        }
        __syncthreads();
        for (int kk = 0; kk < KT; ++kk) {
            float sp = 0.0f;
#pragma unroll
            for (int d = 0; d < 64; ++d) sp = __builtin_fmaf(qv[d], ks[kk][dp + d], sp);
            if (TPQ == 2) sp += __shfl_xor(sp, 1);
            const int key = kv0 + kk;
            if (key <= qi && qi < a.N) {
                const float s = sp * a.scale;
                const float mn = fmaxf(m, s);
                const float corr = expf(m - mn);
                const float p = expf(s - mn);
                l = l * corr + p;
#pragma unroll
                for (int d = 0; d < 64; ++d) ov[d] = __builtin_fmaf(p, vs[kk][dp + d], ov[d] * corr);
                m = mn;
            }
        }
    }
    if (qi < a.N) {
        float* oh = a.o + ((size_t)b * a.Hq + h) * (size_t)a.N * D + (size_t)qi * D + dp;
        const float inv = 1.0f / l;
#pragma unroll
        for (int d = 0; d < 64; ++d) oh[d] = ov[d] * inv;
        if (a.lse && lane % TPQ == 0) a.lse[((size_t)b * a.Hq + h) * a.N + qi] = m + logf(l);
    }
}

static int gcd_int(int x, int y) {
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return x;
}

}  // namespace

hipError_t launch_prefill_dense_bf16(const PrefillProblem& p, hipStream_t s) {
    constexpr int NW = kDenseWaves;
    DenseArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.o = static_cast<uint16_t*>(p.o);
    a.lse = p.lse;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.N = p.N;
    a.G = p.Hq / p.Hkv;
    a.HPW = gcd_int(a.G, NW);
    a.NHG = a.G / a.HPW;
    a.PPW = 32 * (NW / a.HPW);
    a.n_ptiles = (p.N + a.PPW - 1) / a.PPW;
    a.c2 = p.scale * kLog2e;
    const dim3 grid((unsigned)(a.n_ptiles * a.B * a.Hkv * a.NHG));
    if (p.D == 128)
        hipLaunchKernelGGL((prefill_dense_kernel<128>), grid, dim3(NW * 64), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_dense_kernel<64>), grid, dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prefill_paged(const PagedPrefillProblem& p, hipStream_t s) {
    constexpr int NW = kDenseWaves;
    PagedArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.kc = static_cast<const uint16_t*>(p.k_cache);
    a.vc = static_cast<const uint16_t*>(p.v_cache);
    a.o = static_cast<uint16_t*>(p.o);
    a.lse = p.lse;
    a.bt = p.block_table;
    a.lens = p.seq_lens;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.Nq = p.Nq;
    a.G = p.Hq / p.Hkv;
    a.max_pages = p.max_pages;
    a.num_pages = p.num_pages;
    a.window = p.window;
    a.HPW = gcd_int(a.G, NW);
    a.NHG = a.G / a.HPW;
    a.PPW = 32 * (NW / a.HPW);
    a.n_ptiles = (p.Nq + a.PPW - 1) / a.PPW;
    a.c2 = p.scale * kLog2e;
    a.splits = p.splits;
    a.opart = static_cast<float*>(p.workspace);
    a.lpart = a.opart + (size_t)p.splits * p.B * p.Hq * p.Nq * p.D;
    const dim3 grid((unsigned)(a.n_ptiles * a.B * a.Hkv * a.NHG), (unsigned)p.splits);
    // padded K with the scheduled products, except for sliding windows, whose short walks are bound by their loads
    // (windowed chunk: swizzled 0.1155 against padded 0.1199 ms; chunk closing a 32K sequence: padded 1.816 against
    // swizzled 1.862 ms, bit-identical)
    const bool padk = p.window <= 0;
    if (p.D == 128) {
        if (padk) hipLaunchKernelGGL((prefill_paged_kernel<128, true>), grid, dim3(NW * 64), 0, s, a);
        else hipLaunchKernelGGL((prefill_paged_kernel<128, false>), grid, dim3(NW * 64), 0, s, a);
    } else {
        if (padk) hipLaunchKernelGGL((prefill_paged_kernel<64, true>), grid, dim3(NW * 64), 0, s, a);
        else hipLaunchKernelGGL((prefill_paged_kernel<64, false>), grid, dim3(NW * 64), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    PagedCombineArgs c;
    c.opart = a.opart;
    c.lpart = a.lpart;
    c.o = static_cast<uint16_t*>(p.o);
    c.lse = p.lse;
    c.rows = (long)p.B * p.Hq * p.Nq;
    c.splits = p.splits;
    const long rows_per_wg = 4L * (256 / p.D);   // four waves of 256 / D rows
    const dim3 g2((unsigned)((c.rows + rows_per_wg - 1) / rows_per_wg));
    if (p.D == 128) hipLaunchKernelGGL((prefill_paged_combine_kernel<128>), g2, dim3(256), 0, s, c);
    else hipLaunchKernelGGL((prefill_paged_combine_kernel<64>), g2, dim3(256), 0, s, c);
    return hipGetLastError();
}

// Key-range splits for a chunk closing a long sequence: its work-groups all carry about the same number of tiles,
// so when there are too few of them to fill the last round the CUs idle for most of it. Each row set's tiles are
// then shared by `splits` work-groups, chosen to minimise rounds x tiles per work-group on 256 CUs at three
// work-groups each, counting a split only where every piece keeps at least 16 tiles. Chunks that are most of their
// sequence (Nq > half the longest) have causal, uneven work that heaviest-first issue already spreads, and
// windowed chunks have a few tiles per work-group: neither is split.
int paged_prefill_splits(int B, int Hq, int Hkv, int D, int Nq, int max_seq_len, int window) {
    constexpr int NW = kDenseWaves, kSlots = 256 * 3;
    (void)D;
    if (window > 0 || 2 * (long)Nq > max_seq_len) return 1;
    const int G = Hq / Hkv, HPW = gcd_int(G, NW), PPW = 32 * (NW / HPW);
    const long wgs = (long)((Nq + PPW - 1) / PPW) * B * Hkv * (G / HPW);
    const int tiles = (max_seq_len + kBN - 1) / kBN + 1;
    int best = 1;
    double best_cost = (double)((wgs + kSlots - 1) / kSlots) * tiles;
    for (int sp = 2; sp <= 8; ++sp) {
        if (tiles / sp < 16) break;
        const double cost = (double)((wgs * sp + kSlots - 1) / kSlots) * ((tiles + sp - 1) / sp) * 1.03;
        if (cost < best_cost) {
            best_cost = cost;
            best = sp;
        }
    }
    return best;
}

size_t paged_prefill_workspace_bytes(int B, int Hq, int D, int Nq, int splits) {
    if (splits <= 1) return 0;
    return (size_t)splits * B * Hq * Nq * (D + 1) * sizeof(float);
}

hipError_t launch_prefill_sparse_bf16(const PrefillProblem& p, int block, const int32_t* kv_count,
                                      const int32_t* kv_index, hipStream_t s) {
    SparseArgs a;
    a.q = static_cast<const uint16_t*>(p.q);
    a.k = static_cast<const uint16_t*>(p.k);
    a.v = static_cast<const uint16_t*>(p.v);
    a.o = static_cast<uint16_t*>(p.o);
    a.lse = p.lse;
    a.kv_count = kv_count;
    a.kv_index = kv_index;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.N = p.N;
    a.G = p.Hq / p.Hkv;
    a.block = block;
    a.nb = p.N / block;
    a.c2 = p.scale * kLog2e;
    const size_t lst_bytes = ((size_t)a.nb * sizeof(int32_t) + 15) / 16 * 16;   // the kept-block list in LDS
    // one wave per 32 rows: two waves for 64-row blocks; four for 128-row blocks, and for each half of a 256-row one
    if (block == 64) {
        const dim3 grid((unsigned)(a.nb * a.B * a.Hq));
        if (p.D == 128) hipLaunchKernelGGL((prefill_sparse_bf16_kernel<128, 2>), grid, dim3(128), lst_bytes, s, a);
        else hipLaunchKernelGGL((prefill_sparse_bf16_kernel<64, 2>), grid, dim3(128), lst_bytes, s, a);
    } else if (block == 128 || block == 256) {
        const dim3 grid((unsigned)(a.nb * (block / 128) * a.B * a.Hq));
        if (p.D == 128) hipLaunchKernelGGL((prefill_sparse_bf16_kernel<128, 4>), grid, dim3(256), lst_bytes, s, a);
        else hipLaunchKernelGGL((prefill_sparse_bf16_kernel<64, 4>), grid, dim3(256), lst_bytes, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_prefill_dense_f32(const PrefillProblem& p, hipStream_t s) {
    F32Args a;
    a.q = static_cast<const float*>(p.q);
    a.k = static_cast<const float*>(p.k);
    a.v = static_cast<const float*>(p.v);
    a.o = static_cast<float*>(p.o);
    a.lse = p.lse;
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.N = p.N;
    a.G = p.Hq / p.Hkv;
    a.scale = p.scale;
    const int qpb = 64 / (p.D / 64);
    a.n_qt = (p.N + qpb - 1) / qpb;
    const dim3 grid((unsigned)(a.n_qt * a.B * a.Hq));
    if (p.D == 128) hipLaunchKernelGGL((prefill_dense_f32_kernel<128>), grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL((prefill_dense_f32_kernel<64>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace lcattn
