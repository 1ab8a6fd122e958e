// Causal prefill kernels for gfx950: dense GQA (bf16 MFMA), block-sparse (same tile body walking a kept-block
// list) and a plain fp32 path.
//
// Method ("attention-kernel-optimization", section "FlashAttention (1 -> 2 -> 3)"): K/V are streamed through
// on-chip memory in tiles, each query row keeps a running max and sum, and earlier partial results are
// rescaled whenever the max moves, so the score matrix never leaves the chip and the result equals plain
// softmax attention up to rounding.
//
// bf16 tile body (one wave = 32 query rows of one head, one KV tile = 64 keys):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = K rows from LDS, B = the wave's Q rows held in VGPRs for
//   the whole kernel. In the 32x32 accumulator layout lane l owns query column l%32 and 16 keys, so a row
//   max/sum is 15 in-lane ops plus one exchange with lane l^32.
//   O^T += V^T P^T with the same MFMA: the bf16-rounded probabilities are already in B-operand order in the
//   lane that computed them (no LDS round trip); V is stored transposed in LDS when it is staged, with the
//   key order inside each 16-key group permuted so every A operand is one 16-byte LDS read.
//   The running max is refreshed lazily: only when a tile's max exceeds it by more than 2^8, which keeps
//   every exp2 argument <= 8 and skips the O rescale on almost every tile. The final normalisation uses the
//   same max, so the result is unchanged up to rounding.
//   The row sum adds the bf16-rounded probabilities (v_dot2_f32_bf16), i.e. exactly the weights the PV
//   product uses.
// Staging: K/V tiles for step j+1 are fetched into VGPRs while step j computes, then written to the other of
// two LDS buffers; one barrier per step.
#include "device_common.hpp"
#include "internal.hpp"

namespace lcattn {
namespace {

constexpr int kBN = 64;        // keys per KV tile
constexpr int kMaxBlocks = 4096;  // longest kept-block list of one block-sparse row
constexpr float kSlack = 8.0f; // lazy-rescale threshold, log2 units

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// K and V tiles (64 keys x D, bf16) live in LDS in their natural row-major layout without padding; 16-byte chunk c
// of row r sits at chunk position c ^ swz(r). The swizzle keeps both access patterns free of bank conflicts:
// the 16-byte K reads of 16 consecutive rows, and the 8-byte transposed V reads of four consecutive keys.
template <int D>
struct Lds {
    static constexpr int ROWB = D * 2;            // bytes per key row
    static constexpr int CPR = ROWB / 16;         // 16-byte chunks per row
    static constexpr int TILE = kBN * ROWB;       // one K or V tile
    static constexpr int LOADS = TILE / 1024;     // 64-lane x 16-byte direct loads per tile
    __device__ static __forceinline__ int swz(int r) {
        return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes, 0x00020000);
}

// Direct global->LDS staging of one tile by the work-group's NW waves: each 64-lane load moves 1 KiB into
// consecutive LDS bytes, lane l's 16 bytes to position l; the lane fetches the global chunk that the swizzle puts
// there. Buffer range checking returns zeros for keys outside [0, N) (including negative tile starts).
template <int D, int NW>
struct TileLoader {
    static constexpr int PER = (Lds<D>::LOADS + NW - 1) / NW;
    int voff[PER];
    int first;   // this wave's first load slot
    __device__ __forceinline__ void init(int w, int lane) {
        first = w * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int z = (first + i) * 64 + lane;           // 16-byte slot inside the tile
            const int r = z / Lds<D>::CPR, pc = z % Lds<D>::CPR;
            voff[i] = r * Lds<D>::ROWB + ((pc ^ Lds<D>::swz(r)) * 16);
        }
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, lds_char* tile, int kv0) const {
        const int soff = kv0 * Lds<D>::ROWB;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (Lds<D>::LOADS % NW == 0 || first + i < Lds<D>::LOADS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (first + i) * 1024),
                                                         16, voff[i], soff, 0, 0);
    }
};

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

template <int D>
struct RowState {
    f32x16 o[D / 32];
    float m;  // running max of scale*log2(e)*score (log2 units), -inf before the first key
    float l;  // this lane's share of the row sum
};

// S^T for a 64-key tile: two 32x32 blocks (keys x this wave's 32 query rows); the two accumulators alternate.
template <int D>
__device__ __forceinline__ void qk_tile(const lds_char* kl, const bf16x8 (&qf)[D / 16], f32x16 (&s)[2], int lane) {
    const int hi = lane >> 5, ln = lane & 31;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = 32 * t + ln;
            const bf16x8 kf = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
                kl + r * Lds<D>::ROWB + (((2 * ks + hi) ^ Lds<D>::swz(r)) * 16));
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[t], 0, 0, 0);
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

// Online-softmax update for one tile: row max (lazy refresh), probabilities rounded to bf16 and packed in the
// B-operand order of the PV product, row-sum share updated with the rounded values.
template <int D>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[2], uint32_t (&pw)[2][8], RowState<D>& st, float c2,
                                             bool diag, int kv0, int qrow, int lane) {
    const int hi = lane >> 5;
    if (diag) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (key > qrow) s[t][r] = -INFINITY;
            }
    }
    float c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = fmaxf(fmaxf(s[0][k], s[0][k + 4]), fmaxf(s[0][k + 8], s[0][k + 12]));
#pragma unroll
    for (int k = 0; k < 4; ++k)
        c[k] = fmaxf(c[k], fmaxf(fmaxf(s[1][k], s[1][k + 4]), fmaxf(s[1][k + 8], s[1][k + 12])));
    const float mx = pair_max(fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3])));
    const float mxs = mx * c2;
    if (mxs > st.m + kSlack) {
        const float alpha = __builtin_amdgcn_exp2f(st.m - mxs);
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) st.o[dt] *= alpha;
        st.m = mxs;
    }
    const float bias = (st.m == -INFINITY) ? 0.0f : -st.m;
    bf16x2 ones;
    ones[0] = (__bf16)1.0f;
    ones[1] = (__bf16)1.0f;
    float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * w], c2, bias));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * w + 1], c2, bias));
            pw[t][w] = pack_bf16x2(p0, p1);
            if (w & 1) l1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[t][w]), ones, l1, false);
            else l0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[t][w]), ones, l0, false);
        }
    st.l += l0 + l1;
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
        return key * Lds<D>::ROWB + (((d >> 3) ^ Lds<D>::swz(key)) * 16) + (d & 7) * 2;
    }
};

// O^T += V^T P^T over the tile's 64 keys.
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

// LDS of one work-group: two K and two V tiles.
template <int D>
struct Tiles {
    lds_char* k[2];
    lds_char* v[2];
};

// The KV loop of one work-group, software-pipelined inside every wave: while the VALU turns tile j's scores
// into probabilities, the matrix cores already compute tile j+1's scores; then tile j's PV product. K is staged
// one tile ahead of V so both are resident: during step j LDS holds K(j+1) and V(j), and the step's loads of
// K(j+2) and V(j+1) stream straight into the buffers step j-1 finished with. One barrier per step; the
// buffer parity is a compile-time constant inside each unrolled step.
// kv_of(t) gives tile t's first key; a wave skips tiles that start past its last row, and masks elements only on
// tiles that reach past its first row.
template <int D, int NW, int PAR, typename KvOf>
__device__ __forceinline__ void attend_step(const Tiles<D>& tl, const TileLoader<D, NW>& ld,
                                            __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, const VtAddr<D>& va,
                                            int j, int ntiles, KvOf kv_of, int& kv_cur, int& kv_nxt,
                                            const bf16x8 (&qf)[D / 16], f32x16 (&scur)[2], f32x16 (&snext)[2],
                                            RowState<D>& st, float c2, int q0, int wave_last, int lane) {
    const int qrow = q0 + (lane & 31);
    const bool has_next = j + 1 < ntiles;
    const bool act = kv_cur <= wave_last;
    const bool act_n = has_next && kv_nxt <= wave_last;
    const bool diag = kv_cur + kBN - 1 > q0;
    const int kv_2 = j + 2 < ntiles ? kv_of(j + 2) : 0;
    if (j + 2 < ntiles) ld.load(krs, tl.k[PAR], kv_2);
    if (has_next) ld.load(vrs, tl.v[1 - PAR], kv_nxt);
    uint32_t pw[2][8];
    if (act && act_n && !diag) {
        // steady state: one basic block so the scheduler can interleave the two MFMA streams with the VALU
        softmax_tile<D>(scur, pw, st, c2, false, kv_cur, qrow, lane);
        qk_tile<D>(tl.k[1 - PAR], qf, snext, lane);
        pv_tile<D>(tl.v[PAR], va, pw, st);
    } else {
        if (act) softmax_tile<D>(scur, pw, st, c2, diag, kv_cur, qrow, lane);
        if (act_n) qk_tile<D>(tl.k[1 - PAR], qf, snext, lane);
        if (act) pv_tile<D>(tl.v[PAR], va, pw, st);
    }
    wait_vmem();
    __syncthreads();
    kv_cur = kv_nxt;
    kv_nxt = kv_2;
}

template <int D, int NW, typename KvOf>
__device__ __forceinline__ void attend(const Tiles<D>& tl, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                       int ntiles, KvOf kv_of, const bf16x8 (&qf)[D / 16], RowState<D>& st, float c2,
                                       int q0, int wave_last, int w, int lane) {
    TileLoader<D, NW> ld;
    ld.init(w, lane);
    VtAddr<D> va;
    va.init(lane);
    int kv_cur = kv_of(0);
    int kv_nxt = ntiles > 1 ? kv_of(1) : 0;
    ld.load(krs, tl.k[0], kv_cur);
    ld.load(vrs, tl.v[0], kv_cur);
    if (ntiles > 1) ld.load(krs, tl.k[1], kv_nxt);
    wait_vmem();
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (kv_cur <= wave_last) qk_tile<D>(tl.k[0], qf, sa, lane);
    __syncthreads();
    int j = 0;
    for (; j + 1 < ntiles; j += 2) {
        attend_step<D, NW, 0>(tl, ld, krs, vrs, va, j, ntiles, kv_of, kv_cur, kv_nxt, qf, sa, sb, st, c2, q0,
                              wave_last, lane);
        attend_step<D, NW, 1>(tl, ld, krs, vrs, va, j + 1, ntiles, kv_of, kv_cur, kv_nxt, qf, sb, sa, st, c2, q0,
                              wave_last, lane);
    }
    if (j < ntiles)
        attend_step<D, NW, 0>(tl, ld, krs, vrs, va, j, ntiles, kv_of, kv_cur, kv_nxt, qf, sa, sb, st, c2, q0,
                              wave_last, lane);
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

// Work-group = HPW query heads of one kv group x PPW consecutive positions; waves = heads x 32-row slices.
// All waves share each staged K/V tile. Work-groups are issued heaviest (latest positions) first, and the kv
// head cycles fastest so that, with 8 XCDs dispatched round-robin, an XCD keeps seeing the same kv heads.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_dense_bf16_kernel(const DenseArgs a) {
    __shared__ __attribute__((aligned(1024))) char k0[Lds<D>::TILE];
    __shared__ __attribute__((aligned(1024))) char k1[Lds<D>::TILE];
    __shared__ __attribute__((aligned(1024))) char v0[Lds<D>::TILE];
    __shared__ __attribute__((aligned(1024))) char v1[Lds<D>::TILE];
    const Tiles<D> tl{{(lds_char*)k0, (lds_char*)k1}, {(lds_char*)v0, (lds_char*)v1}};
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
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
    const int wave_last = q0 < a.N ? min(q0 + 31, a.N - 1) : -1;
    attend<D, NW>(tl, krs, vrs, ntiles, [](int t) { return t * kBN; }, qf, st, a.c2, q0, wave_last, w, lane);
    finish_rows<D>(st, a.o + qoff, a.lse ? a.lse + ((size_t)b * a.Hq + h) * a.N : nullptr, qrow, a.N, lane);
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
// are never read. Rows are issued latest block first, as they tend to hold the longest lists.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_sparse_bf16_kernel(const SparseArgs a) {
    __shared__ __attribute__((aligned(1024))) char k0[Lds<D>::TILE];
    __shared__ __attribute__((aligned(1024))) char k1[Lds<D>::TILE];
    __shared__ __attribute__((aligned(1024))) char v0[Lds<D>::TILE];
    __shared__ __attribute__((aligned(1024))) char v1[Lds<D>::TILE];
    const Tiles<D> tl{{(lds_char*)k0, (lds_char*)k1}, {(lds_char*)v0, (lds_char*)v1}};
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int per = a.B * a.Hq;
    const int i = a.nb - 1 - (int)(blockIdx.x / per);
    const int rest = (int)(blockIdx.x % per);
    const int h = rest % a.Hq;
    const int b = rest / a.Hq;
    const int g = h / a.G;
    const int q0 = i * a.block + 32 * w;
    const int qrow = q0 + (lane & 31);
    const size_t row = ((size_t)b * a.Hq + h) * a.nb + i;
    const int cnt = a.kv_count[row];
    const int32_t* list = a.kv_index + row * a.nb;
    const int sub = a.block / kBN;
    const int ntiles = cnt * sub;

    const size_t qoff = ((size_t)b * a.Hq + h) * (size_t)a.N * D;
    const size_t kvoff = ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + kvoff, a.N * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + kvoff, a.N * D * 2);

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + qoff, qrow, a.N, lane);
    RowState<D> st;
    init_state<D>(st);
    if (ntiles == 0) return;  // every valid list holds the diagonal; an empty one leaves the rows unwritten
    // the row's block list goes to LDS once, so the tile loop reads the next tile's block in LDS latency instead
    // of a global round trip per tile
    __shared__ int lst[kMaxBlocks];
    for (int e = tid; e < cnt; e += NW * 64) lst[e] = list[e];
    __syncthreads();
    const int blk = a.block;
    attend<D, NW>(tl, krs, vrs, ntiles, [&](int t) { return lst[t / sub] * blk + (t % sub) * kBN; }, qf, st, a.c2,
                  q0, q0 + 31, w, lane);
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
    constexpr int NW = 8;
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
        hipLaunchKernelGGL((prefill_dense_bf16_kernel<128, NW>), grid, dim3(NW * 64), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_dense_bf16_kernel<64, NW>), grid, dim3(NW * 64), 0, s, a);
    return hipGetLastError();
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
    const dim3 grid((unsigned)(a.nb * a.B * a.Hq));
    // one wave per 32 rows of the query block
    if (block == 64) {
        if (p.D == 128) hipLaunchKernelGGL((prefill_sparse_bf16_kernel<128, 2>), grid, dim3(128), 0, s, a);
        else hipLaunchKernelGGL((prefill_sparse_bf16_kernel<64, 2>), grid, dim3(128), 0, s, a);
    } else if (block == 128) {
        if (p.D == 128) hipLaunchKernelGGL((prefill_sparse_bf16_kernel<128, 4>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((prefill_sparse_bf16_kernel<64, 4>), grid, dim3(256), 0, s, a);
    } else if (block == 256) {
        if (p.D == 128) hipLaunchKernelGGL((prefill_sparse_bf16_kernel<128, 8>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((prefill_sparse_bf16_kernel<64, 8>), grid, dim3(512), 0, s, a);
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
