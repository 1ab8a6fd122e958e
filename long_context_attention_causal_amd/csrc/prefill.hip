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
constexpr float kSlack = 8.0f; // lazy-rescale threshold, log2 units

template <int D>
struct Lds {
    static constexpr int KP = D * 2 + 16;   // K row pitch in bytes (padding spreads rows over the banks)
    static constexpr int VP = kBN * 2 + 16; // V^T row pitch in bytes
    static constexpr int KBYTES = kBN * KP;
    static constexpr int VBYTES = D * VP;
    static constexpr int STAGE = KBYTES + VBYTES;
};

// Column of key k (0..63) inside a V^T row: bits 2 and 3 of the key's index within its 16-key group are swapped,
// so the eight keys one MFMA lane group contracts over sit next to each other.
__device__ __forceinline__ int vt_pos(int k) {
    const int w = k & 15;
    return (k & ~15) | ((w & 4) << 1) | ((w & 8) >> 1) | (w & 3);
}

template <int D, int NT>
struct Stager {
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int KCH = kBN * CPR;              // K chunks per tile
    static constexpr int KPT = (KCH + NT - 1) / NT;
    static constexpr int VU = (kBN / 2) * CPR;         // (key pair, chunk) units per tile
    static constexpr int VPT = (VU + NT - 1) / NT;
    u32x4 kr[KPT];
    u32x4 vr[VPT][2];

    __device__ __forceinline__ void load(const uint16_t* kb, const uint16_t* vb, int kv0, int N, int tid) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            kr[i] = u32x4{0u, 0u, 0u, 0u};
            if (KCH % NT == 0 || idx < KCH) {
                const int key = kv0 + idx / CPR;
                if ((unsigned)key < (unsigned)N) kr[i] = load16(kb + (size_t)key * D + (idx % CPR) * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * NT;
            vr[i][0] = u32x4{0u, 0u, 0u, 0u};
            vr[i][1] = u32x4{0u, 0u, 0u, 0u};
            if (VU % NT == 0 || idx < VU) {
                const int key = kv0 + 2 * (idx / CPR);
                const int c = idx % CPR;
                if ((unsigned)key < (unsigned)N) vr[i][0] = load16(vb + (size_t)key * D + c * 8);
                if ((unsigned)(key + 1) < (unsigned)N) vr[i][1] = load16(vb + (size_t)(key + 1) * D + c * 8);
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int idx = tid + i * NT;
            if (KCH % NT == 0 || idx < KCH) store16(lds + (idx / CPR) * Lds<D>::KP + (idx % CPR) * 16, kr[i]);
        }
        char* vt = lds + Lds<D>::KBYTES;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + i * NT;
            if (VU % NT == 0 || idx < VU) {
                const int p = idx / CPR, c = idx % CPR;
                const int col = vt_pos(2 * p) * 2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t a = vr[i][0][e >> 1], b = vr[i][1][e >> 1];
                    const uint32_t w = (e & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
                    *reinterpret_cast<uint32_t*>(vt + (c * 8 + e) * Lds<D>::VP + col) = w;
                }
            }
        }
    }
};

template <int D>
struct RowState {
    f32x16 o[D / 32];
    float m;  // running max of scale*log2(e)*score (log2 units), -inf before the first key
    float l;  // this lane's share of the row sum
};

// One KV tile for one wave. `lds` points at a staged tile (K rows, then V^T rows).
template <int D>
__device__ __forceinline__ void tile_step(const char* lds, const bf16x8 (&qf)[D / 16], RowState<D>& st, float c2,
                                          bool diag, int kv0, int qrow, int lane) {
    const int hi = lane >> 5, ln = lane & 31;
    f32x16 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        s[t] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8*>(lds + (32 * t + ln) * Lds<D>::KP + (16 * ks + 8 * hi) * 2);
            s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[t], 0, 0, 0);
        }
    }
    if (diag) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * t + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (key > qrow) s[t][r] = -INFINITY;
            }
    }
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * c2;
    if (mxs > st.m + kSlack) {
        const float alpha = exp2f(st.m - mxs);
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) st.o[dt] *= alpha;
        st.m = mxs;
    }
    const float bias = (st.m == -INFINITY) ? 0.0f : -st.m;
    uint32_t pw[2][8];
    bf16x2 ones;
    ones[0] = (__bf16)1.0f;
    ones[1] = (__bf16)1.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * w], c2, bias));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][2 * w + 1], c2, bias));
            pw[t][w] = pack_bf16x2(p0, p1);
            st.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[t][w]), ones, st.l, false);
        }
    const char* vt = lds + Lds<D>::KBYTES;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (32 * dt + ln) * Lds<D>::VP +
                                                                  (32 * t + 16 * u + 8 * hi) * 2);
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, (u32x4{pw[t][4 * u], pw[t][4 * u + 1], pw[t][4 * u + 2], pw[t][4 * u + 3]}));
                st.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, st.o[dt], 0, 0, 0);
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
    const float lt = st.l + __shfl_xor(st.l, 32);
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

// Work-group = HPW query heads of one kv group x PPW consecutive positions; waves = heads x 32-row slices.
// All waves share each staged K/V tile. Work-groups are issued heaviest (latest positions) first, and the kv
// head cycles fastest so that, with 8 XCDs dispatched round-robin, an XCD keeps seeing the same kv heads.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_dense_bf16_kernel(const DenseArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2 * Lds<D>::STAGE];
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
    const int ln = lane & 31;
    const int qrow = q0 + ln;

    const size_t qoff = ((size_t)b * a.Hq + h) * (size_t)a.N * D;
    const uint16_t* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    const uint16_t* vb = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.N * D;

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + qoff, qrow, a.N, lane);
    RowState<D> st;
    init_state<D>(st);

    Stager<D, NW * 64> sg;
    sg.load(kb, vb, 0, a.N, tid);
    sg.store(lds, tid);
    __syncthreads();
    const int wave_last = min(q0 + 31, a.N - 1);
    for (int j = 0; j < ntiles; ++j) {
        if (j + 1 < ntiles) sg.load(kb, vb, (j + 1) * kBN, a.N, tid);
        const int kv0 = j * kBN;
        if (q0 < a.N && kv0 <= wave_last)
            tile_step<D>(lds + (j & 1) * Lds<D>::STAGE, qf, st, a.c2, kv0 + kBN - 1 > q0, kv0, qrow, lane);
        if (j + 1 < ntiles) sg.store(lds + ((j + 1) & 1) * Lds<D>::STAGE, tid);
        __syncthreads();
    }
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
__global__ __launch_bounds__(NW * 64) void prefill_sparse_bf16_kernel(const SparseArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2 * Lds<D>::STAGE];
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
    const uint16_t* kb = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.N * D;
    const uint16_t* vb = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.N * D;

    bf16x8 qf[D / 16];
    load_q<D>(qf, a.q + qoff, qrow, a.N, lane);
    RowState<D> st;
    init_state<D>(st);
    if (ntiles == 0) return;  // every valid list holds the diagonal; an empty one leaves the rows unwritten

    Stager<D, NW * 64> sg;
    int jb = list[0];
    sg.load(kb, vb, jb * a.block, a.N, tid);
    sg.store(lds, tid);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int kv0 = jb * a.block + (t % sub) * kBN;
        const bool diag = (jb == i);
        if (t + 1 < ntiles) {
            const int jn = list[(t + 1) / sub];
            sg.load(kb, vb, jn * a.block + ((t + 1) % sub) * kBN, a.N, tid);
            if ((t + 1) % sub == 0) jb = jn;
        }
        if (kv0 <= q0 + 31)
            tile_step<D>(lds + (t & 1) * Lds<D>::STAGE, qf, st, a.c2, diag && (kv0 + kBN - 1 > q0), kv0, qrow,
                         lane);
        if (t + 1 < ntiles) sg.store(lds + ((t + 1) & 1) * Lds<D>::STAGE, tid);
        __syncthreads();
    }
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
