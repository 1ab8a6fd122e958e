// Block-selection pre-pass for gfx950, all arithmetic in float64.
//
// Source: "Your 128K Context Is 6x Slower Than It Needs to Be", sections "Why block-sparse attention
// underperforms: the mean-dilution trap" (a block scored by its key centroid hides a single strong key) and
// "The rescue branch: two selection paths, one mask" (per key block the largest key-to-centroid distance; a
// threshold from the median and 90th percentile of those radii per kv head; the two branches thresholded on
// their own and OR-ed; the pre-pass is linear in sequence length).
//
// Four kernels on the caller's stream:
//   stats     one work-group per query block (mean of its rows) or key block (centroid, then radius): a
//             coalesced pass over Q and K with 16-byte loads, fp64 sums. The block sums of bf16 values are
//             exact in fp64 for ordinary data, so the means do not depend on summation order.
//   threshold one work-group per (batch, kv head): the needed order statistics of the radii by exact rank
//             counting, then type-7 interpolation and tau, evaluated in the same operation order as the
//             reference definition with contraction disabled; then the rescue flags.
//   scores    fp64 tiled product of the query-block means with the key centroids of the same kv head, lower
//             triangle only (the O(nb^2) block score matrix the page warns about lives in the workspace).
//   select    one wave per (batch, head, query block): the integer budget, top-k by a bitwise search over
//             order-preserving 64-bit keys of the scores (ties to the smaller block index), OR with rescue
//             flags and the diagonal, then the uint8 row and its ascending CSR list via ballots.
#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"

namespace lcattn {
namespace {

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) { return (double)bf16_to_f32(bits16); }

struct StatsArgs {
    const uint16_t* q;
    const uint16_t* k;     // bf16 keys, or
    const uint8_t* k8;     // E4M3 key codes (value = code value * k_scale) when set
    double k_scale;
    double* qbar;
    double* kbar;
    double* radius;
    int B, Hq, Hkv, N, block, nb;
    long nq_blocks;  // B * Hq * nb
};

// Eight keys of a row from E4M3 codes, widened exactly (fp8 -> f32 is exact) and scaled in f64 (one rounding).
__device__ __forceinline__ void fp8x8_to_f64(u32x2 w, double k_scale, double (&x)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[h], true);
        x[4 * h + 0] = (double)lo[0] * k_scale;
        x[4 * h + 1] = (double)lo[1] * k_scale;
        x[4 * h + 2] = (double)hi[0] * k_scale;
        x[4 * h + 3] = (double)hi[1] * k_scale;
    }
}

template <int D, bool K8>
__global__ __launch_bounds__(256) void mask_stats_kernel(const StatsArgs a) {
    constexpr int CPR = D / 8;        // 16-byte chunks per row
    constexpr int RPP = 256 / CPR;    // rows per pass
    __shared__ double part[RPP][D];
    __shared__ double cen[D];
    __shared__ double wmax[4];
    const int tid = threadIdx.x, c = tid % CPR, r0 = tid / CPR;
    long id = blockIdx.x;
    const bool isq = id < a.nq_blocks;
    const uint16_t* base;
    const uint8_t* base8 = nullptr;
    double* out;
    int b, hh, j;
    if (isq) {
        j = (int)(id % a.nb);
        const long bh = id / a.nb;
        hh = (int)(bh % a.Hq);
        b = (int)(bh / a.Hq);
        base = a.q + (((size_t)b * a.Hq + hh) * a.N + (size_t)j * a.block) * D;
        out = a.qbar + (((size_t)b * a.Hq + hh) * a.nb + j) * D;
    } else {
        id -= a.nq_blocks;
        j = (int)(id % a.nb);
        const long bg = id / a.nb;
        hh = (int)(bg % a.Hkv);
        b = (int)(bg / a.Hkv);
        const size_t row0 = (((size_t)b * a.Hkv + hh) * a.N + (size_t)j * a.block) * D;
        base = K8 ? nullptr : a.k + row0;
        base8 = K8 ? a.k8 + row0 : nullptr;
        out = a.kbar + (((size_t)b * a.Hkv + hh) * a.nb + j) * D;
    }
    // eight consecutive elements of row r (this lane's chunk), as f64
    auto elems = [&](int r, double (&x)[8]) {
        if (K8 && !isq) {
            fp8x8_to_f64(*reinterpret_cast<const u32x2*>(base8 + (size_t)r * D + c * 8), a.k_scale, x);
        } else {
            const u32x4 v = load16(base + (size_t)r * D + c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = bf16_to_f64((v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
        }
    };
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0;
    for (int r = r0; r < a.block; r += RPP) {
        double x[8];
        elems(r, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r0][c * 8 + e] = s[e];
    __syncthreads();
    if (tid < D) {
        double t = 0.0;
        for (int r = 0; r < RPP; ++r) t += part[r][tid];
        const double mean = t / (double)a.block;
        out[tid] = mean;
        cen[tid] = mean;
    }
    if (isq) return;  // uniform over the work-group
    __syncthreads();
    double cc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cc[e] = cen[c * 8 + e];
    double best = 0.0;
    for (int r = r0; r < a.block; r += RPP) {
        double xs[8];
        elems(r, xs);
        double d2 = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double x = xs[e] - cc[e];
            d2 += x * x;
        }
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) d2 += __shfl_xor(d2, o);   // the row's CPR lanes are adjacent
        best = fmax(best, d2);
    }
    best = wave_max_f64(best);
    if ((tid & 63) == 0) wmax[tid >> 6] = best;
    __syncthreads();
    if (tid == 0) {
        const double m = fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
        a.radius[((size_t)b * a.Hkv + hh) * a.nb + j] = sqrt(m);
    }
}

struct ThreshArgs {
    const double* radius;
    double* thresh;       // [B*Hkv][4]
    uint8_t* flags;       // [B*Hkv][nb]
    double* radius_stats; // optional [B*Hkv][nb+3]
    int nb, lo_pct, hi_pct;
    double alpha;
};

// Type-7 quantile value from the two order statistics around the position, in the reference operation order.
__device__ double interp7(double xlo, double xhi, long num, bool has_next) {
#pragma clang fp contract(off)
    const double f = (double)(num % 100) / 100.0;
    if (!has_next || f == 0.0) return xlo;
    return xlo + f * (xhi - xlo);
}

// The four order statistics around the two quantile positions, by exact rank counting: work-group (bg, y) ranks
// the 64 radii e = 64 y + lane against all n of its (batch, kv head), the four waves each counting a quarter of them.
// The radius of sorted position k is the one x with #{y < x} <= k < #{y <= x} (equal radii write equal values), and
// it lands in slot k of the (batch, kv head)'s four-double threshold record, which the threshold kernel then reads
// and overwrites.
__global__ __launch_bounds__(256) void mask_rank_kernel(const ThreshArgs a) {
    __shared__ double rs[4096];
    __shared__ int cnt[2][4][64];
    const int bg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, n = a.nb;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const double* r = a.radius + (size_t)bg * n;
    for (int e = tid; e < n; e += 256) rs[e] = r[e];
    __syncthreads();
    const int e = (int)blockIdx.y * 64 + lane;
    const double x = rs[min(e, n - 1)];
    const int q = (n + 3) / 4, t0 = w * q, t1 = min(n, t0 + q);
    int lt = 0, le = 0;
    for (int t = t0; t < t1; ++t) {
        const double y = rs[t];
        lt += (y < x);
        le += (y <= x);
    }
    cnt[0][w][lane] = lt;
    cnt[1][w][lane] = le;
    __syncthreads();
    if (w != 0 || e >= n) return;
    lt = cnt[0][0][lane] + cnt[0][1][lane] + cnt[0][2][lane] + cnt[0][3][lane];
    le = cnt[1][0][lane] + cnt[1][1][lane] + cnt[1][2][lane] + cnt[1][3][lane];
    const long num_lo = (long)(n - 1) * a.lo_pct, num_hi = (long)(n - 1) * a.hi_pct;
    const int want[4] = {(int)(num_lo / 100), (int)min((long)n - 1, num_lo / 100 + 1), (int)(num_hi / 100),
                         (int)min((long)n - 1, num_hi / 100 + 1)};
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (lt <= want[k] && want[k] < le) a.thresh[(size_t)bg * 4 + k] = x;
}

// One work-group per (batch, kv head): the quantiles from the ranked order statistics, tau and the flags.
__global__ __launch_bounds__(1024) void mask_threshold_kernel(const ThreshArgs a) {
#pragma clang fp contract(off)
    __shared__ double rs[4096];
    __shared__ double os[4];
    const int bg = blockIdx.x, tid = threadIdx.x, n = a.nb;
    const double* r = a.radius + (size_t)bg * n;
    for (int e = tid; e < n; e += 1024) rs[e] = r[e];
    if (tid < 4) os[tid] = a.thresh[(size_t)bg * 4 + tid];
    const long num_lo = (long)(n - 1) * a.lo_pct, num_hi = (long)(n - 1) * a.hi_pct;
    __syncthreads();
    __shared__ double tau_s;
    if (tid == 0) {
        const double med = interp7(os[0], os[1], num_lo, num_lo / 100 + 1 < n);
        const double hi = interp7(os[2], os[3], num_hi, num_hi / 100 + 1 < n);
        const double tau = isinf(a.alpha) ? INFINITY : med + a.alpha * (hi - med);
        double* t = a.thresh + (size_t)bg * 4;
        t[0] = med;
        t[1] = hi;
        t[2] = tau;
        t[3] = hi == 0.0 ? 0.0 : (hi - med) / hi;   // query-aware rescue coefficient
        if (a.radius_stats) {
            double* rsd = a.radius_stats + (size_t)bg * (n + 3);
            rsd[n] = med;
            rsd[n + 1] = hi;
            rsd[n + 2] = tau;
        }
        tau_s = tau;
    }
    __syncthreads();
    const double tau = tau_s;
    for (int e = tid; e < n; e += 1024) {
        a.flags[(size_t)bg * n + e] = rs[e] > tau ? 1 : 0;
        if (a.radius_stats) a.radius_stats[(size_t)bg * (n + 3) + e] = rs[e];
    }
}

struct ScoreArgs {
    const double* qbar;
    const double* kbar;
    double* scores;   // [B, Hq, nb, nb]
    int Hq, Hkv, G, nb, D;
    double scale;
};

// 128 x 128 output tile per work-group (rows: the kv head's query heads stacked, hl * nb + i; columns: key blocks) on
// the fp64 matrix cores: each wave owns a 64 x 64 quarter as 4 x 4 blocks of v_mfma_f64_16x16x4f64, the head dim
// in chunks of 16 staged through LDS, the next chunk loaded into registers while the current one is multiplied.
// Tiles wholly above the diagonal are skipped. The grid is one-dimensional over (kv group, row tile, column tile),
// and work-group L takes tile (L % 8) * (total / 8) + L / 8 when the tile count divides by 8: the hardware deals
// work-groups to the 8 XCDs round-robin, so each XCD then takes one contiguous eighth of the tiles, whose share of
// the lower triangle is even (with column tiles innermost, XCD x would take every tile of column x, from all rows
// for x = 0 down to the last row tile only for x = 7).
constexpr int kST = 128;      // tile edge
constexpr int kSC = 16;       // head-dim chunk (doubles)
constexpr int kSP = kSC + 1;  // LDS row stride in doubles
typedef double f64x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mask_scores_kernel(const ScoreArgs a) {
    __shared__ double As[kST * kSP];
    __shared__ double Bs[kST * kSP];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int R = a.G * a.nb;
    const int nct = (a.nb + kST - 1) / kST, nrt = (R + kST - 1) / kST;
    const int total = (int)gridDim.x, L = (int)blockIdx.x;
    const int T = total % 8 == 0 ? (L % 8) * (total / 8) + L / 8 : L;
    const int j0 = (T % nct) * kST, r0 = ((T / nct) % nrt) * kST;
    const int bg = T / (nct * nrt), b = bg / a.Hkv, g = bg % a.Hkv;
    const int rl = min(r0 + kST - 1, R - 1);
    const int imax = (r0 / a.nb == rl / a.nb) ? rl % a.nb : a.nb - 1;
    if (j0 > imax) return;
    const double* kb = a.kbar + ((size_t)b * a.Hkv + g) * a.nb * a.D;
    // loader: thread -> (row or key block lr = tid / 2, half lh = tid % 2 of the chunk: 8 doubles)
    const int lr = tid >> 1, lh = tid & 1;
    const int ra = r0 + lr, ja = j0 + lr;
    const double* qsrc = nullptr;
    if (ra < R) {
        const int hl = ra / a.nb, i = ra % a.nb;
        qsrc = a.qbar + (((size_t)b * a.Hq + g * a.G + hl) * a.nb + i) * a.D + 8 * lh;
    }
    const double* ksrc = ja < a.nb ? kb + (size_t)ja * a.D + 8 * lh : nullptr;
    double qa[8], ka[8];
    auto fetch = [&](int d0) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            const double2 x = qsrc ? *reinterpret_cast<const double2*>(qsrc + d0 + k) : double2{0.0, 0.0};
            const double2 y = ksrc ? *reinterpret_cast<const double2*>(ksrc + d0 + k) : double2{0.0, 0.0};
            qa[k] = x.x;
            qa[k + 1] = x.y;
            ka[k] = y.x;
            ka[k + 1] = y.y;
        }
    };
    const int wr = (w >> 1) * 64, wc = (w & 1) * 64;   // the wave's quarter
    const int fi = lane & 15, fk = lane >> 4;            // operand lane: row (column) fi, head dim fk of 4
    f64x4 acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f64x4{0.0, 0.0, 0.0, 0.0};
    fetch(0);
    for (int d0 = 0; d0 < a.D; d0 += kSC) {
        __syncthreads();   // every wave is done with the previous chunk
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            As[lr * kSP + 8 * lh + k] = qa[k];
            Bs[lr * kSP + 8 * lh + k] = ka[k];
        }
        __syncthreads();
        if (d0 + kSC < a.D) fetch(d0 + kSC);
#pragma unroll
        for (int ks = 0; ks < kSC / 4; ++ks) {
            double av[4], bv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) av[m] = As[(wr + 16 * m + fi) * kSP + 4 * ks + fk];
#pragma unroll
            for (int n = 0; n < 4; ++n) bv[n] = Bs[(wc + 16 * n + fi) * kSP + 4 * ks + fk];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[m], bv[n], acc[m][n], 0, 0, 0);
        }
    }
    // block (m, n) element v of lane l is row 16 m + l / 16 + 4 v, column 16 n + l % 16 of the quarter
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = r0 + wr + 16 * m + fk + 4 * v;
            if (r >= R) continue;
            const int hl = r / a.nb, i = r % a.nb;
            double* srow = a.scores + (((size_t)b * a.Hq + g * a.G + hl) * a.nb + i) * a.nb;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int j = j0 + wc + 16 * n + fi;
                if (j <= i && j < a.nb) srow[j] = __dmul_rn(a.scale, acc[m][n][v]);
            }
        }
}

struct SelectArgs {
    const double* scores;
    const uint8_t* flags;
    const double* qbar;    // query-aware mode: [B*Hq*nb][D]
    const double* radius;  // query-aware mode: [B*Hkv][nb]
    const double* thresh;  // query-aware mode: [B*Hkv][4] = (med, p_hi, tau, lambda)
    uint8_t* mask;
    int32_t* kv_count;
    int32_t* kv_index;
    int B, Hq, Hkv, G, nb, keep, D, mode;
    double scale;
};

// Order-preserving map of a double onto uint64 (after folding -0 onto +0, which compares equal).
__device__ __forceinline__ uint64_t order_key(double x) {
    if (x == 0.0) x = 0.0;
    const uint64_t u = __double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <int E>
__global__ __launch_bounds__(256) void mask_select_kernel(const SelectArgs a) {
    // wave-uniform row: its length, budget and the search's branches stay scalar
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + w;
    if (row >= (long)a.B * a.Hq * a.nb) return;   // no barriers in this kernel
    const int i = (int)(row % a.nb);
    const long bh = row / a.nb;
    const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
    const int g = h / a.G;
    const double* srow = a.scores + (size_t)row * a.nb;
    const uint8_t* fl = a.flags + ((size_t)b * a.Hkv + g) * a.nb;
    const int cand = i + 1;
    const int budget = min(cand, (int)(((long)cand * a.keep + 999) / 1000));
    // slots e with 64 e > i hold no candidate in any lane: the counting loops skip them (a uniform branch).
    // Every lane loads its scores and flags at a clamped index (always inside the row), so the loads issue
    // back to back instead of one guarded load and wait per slot.
    uint64_t key[E];
    bool kept[E];
    uint8_t fv[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = lane + 64 * e;
        const double x = srow[min(j, i)];
        fv[e] = fl[min(j, i)];
        key[e] = order_key(x) & (0ull - (uint64_t)(j <= i));   // arithmetic, so the load stays unconditional
        kept[e] = false;
    }
    if (budget >= cand) {
#pragma unroll
        for (int e = 0; e < E; ++e) kept[e] = (lane + 64 * e) <= i;
    } else if (budget > 0) {
        uint64_t T = 0;
        bool exact = false;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t c = T | (1ull << bit);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (64 * e <= i) cnt += __popcll(__ballot((lane + 64 * e) <= i && key[e] >= c));
            if (cnt >= budget) {
                T = c;
                if (cnt == budget) {
                    exact = true;
                    break;
                }
            }
        }
        if (exact) {
#pragma unroll
            for (int e = 0; e < E; ++e) kept[e] = (lane + 64 * e) <= i && key[e] >= T;
        } else {
            // T is the budget-th largest key and is shared by several candidates: take all above it, then the
            // tied ones in ascending block order until the budget is met
            int have = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                kept[e] = (lane + 64 * e) <= i && key[e] > T;
                have += __popcll(__ballot(kept[e]));
            }
            int need = budget - have;
            const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool tie = (lane + 64 * e) <= i && key[e] == T;
                const uint64_t bal = __ballot(tie);
                const int before = __popcll(bal & below);
                if (tie && before < need) kept[e] = true;
                need -= min(need, __popcll(bal));
            }
        }
    }
    // Query-aware rescue: a flagged block j stays a rescue only where its centroid score plus the allowance
    // lambda * scale * |qbar_i| * (r_j - med) beats this row's centroid cutoff (the smallest kept score). When the
    // budget covers every candidate the row is full anyway; with no budget there is no cutoff to beat.
    const bool aware = a.mode == 1 && budget < cand;
    double cut = INFINITY, coef = 0.0, med = 0.0;
    const double* rad = nullptr;
    if (aware) {
#pragma clang fp contract(off)
        if (budget > 0) {
            uint64_t lo = ~0ull;
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (kept[e]) lo = min(lo, key[e]);
            for (int o = 32; o >= 1; o >>= 1) lo = min(lo, (uint64_t)__shfl_xor((unsigned long long)lo, o));
            cut = __longlong_as_double((long long)((lo >> 63) ? (lo & 0x7fffffffffffffffull) : ~lo));
        }
        const double* qr = a.qbar + (size_t)row * a.D;
        double ss = 0.0;
        for (int d = lane; d < a.D; d += 64) ss += qr[d] * qr[d];
        for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
        const double* th = a.thresh + ((size_t)b * a.Hkv + g) * 4;
        med = th[0];
        coef = th[3] * a.scale * sqrt(ss);
        rad = a.radius + ((size_t)b * a.Hkv + g) * a.nb;
    }
    uint8_t* mrow = a.mask + (size_t)row * a.nb;
    int32_t* irow = a.kv_index + (size_t)row * a.nb;
    const uint64_t below = (1ull << lane) - 1ull;
    int count = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int j = lane + 64 * e;
        bool resc = j <= i && fv[e] != 0;
        if (aware && resc && !kept[e]) {
#pragma clang fp contract(off)
            resc = srow[j] + coef * (rad[j] - med) > cut;
        }
        const bool m = j <= i && (kept[e] || resc || j == i);
        if (j < a.nb) mrow[j] = m ? 1 : 0;
        const uint64_t bal = __ballot(m);
        if (m) irow[count + __popcll(bal & below)] = j;
        count += __popcll(bal);
    }
    if (lane == 0) a.kv_count[row] = count;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

MaskWorkspace mask_workspace_layout(int B, int Hq, int Hkv, int nb, int D, char* base) {
    MaskWorkspace w;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += align256(bytes);
        return p;
    };
    w.qbar = reinterpret_cast<double*>(take((size_t)B * Hq * nb * D * 8));
    w.kbar = reinterpret_cast<double*>(take((size_t)B * Hkv * nb * D * 8));
    w.radius = reinterpret_cast<double*>(take((size_t)B * Hkv * nb * 8));
    w.thresh = reinterpret_cast<double*>(take((size_t)B * Hkv * 4 * 8));
    w.flags = reinterpret_cast<uint8_t*>(take((size_t)B * Hkv * nb));
    w.scores = reinterpret_cast<double*>(take((size_t)B * Hq * nb * nb * 8));
    w.total = off;
    return w;
}

hipError_t launch_block_mask(const MaskProblem& p, const MaskWorkspace& ws, hipStream_t s) {
    StatsArgs sa;
    sa.q = static_cast<const uint16_t*>(p.q);
    sa.k = p.k8 ? nullptr : static_cast<const uint16_t*>(p.k);
    sa.k8 = p.k8;
    sa.k_scale = p.k_scale;
    sa.qbar = ws.qbar;
    sa.kbar = ws.kbar;
    sa.radius = ws.radius;
    sa.B = p.B;
    sa.Hq = p.Hq;
    sa.Hkv = p.Hkv;
    sa.N = p.N;
    sa.block = p.block;
    sa.nb = p.nb;
    sa.nq_blocks = (long)p.B * p.Hq * p.nb;
    const unsigned nstat = (unsigned)(sa.nq_blocks + (long)p.B * p.Hkv * p.nb);
    if (p.k8) {
        if (p.D == 128) hipLaunchKernelGGL((mask_stats_kernel<128, true>), dim3(nstat), dim3(256), 0, s, sa);
        else hipLaunchKernelGGL((mask_stats_kernel<64, true>), dim3(nstat), dim3(256), 0, s, sa);
    } else {
        if (p.D == 128) hipLaunchKernelGGL((mask_stats_kernel<128, false>), dim3(nstat), dim3(256), 0, s, sa);
        else hipLaunchKernelGGL((mask_stats_kernel<64, false>), dim3(nstat), dim3(256), 0, s, sa);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    ThreshArgs ta;
    ta.radius = ws.radius;
    ta.thresh = ws.thresh;
    ta.flags = ws.flags;
    ta.radius_stats = p.radius_stats;
    ta.nb = p.nb;
    ta.lo_pct = p.lo_pct;
    ta.hi_pct = p.hi_pct;
    ta.alpha = p.alpha;
    hipLaunchKernelGGL(mask_rank_kernel, dim3((unsigned)(p.B * p.Hkv), (unsigned)((p.nb + 63) / 64)), dim3(256), 0, s,
                       ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(mask_threshold_kernel, dim3((unsigned)(p.B * p.Hkv)), dim3(1024), 0, s, ta);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    ScoreArgs sc;
    sc.qbar = ws.qbar;
    sc.kbar = ws.kbar;
    sc.scores = ws.scores;
    sc.Hq = p.Hq;
    sc.Hkv = p.Hkv;
    sc.G = p.Hq / p.Hkv;
    sc.nb = p.nb;
    sc.D = p.D;
    sc.scale = p.scale;
    const long ntiles = (long)((p.nb + kST - 1) / kST) * ((sc.G * p.nb + kST - 1) / kST) * p.B * p.Hkv;
    if (ntiles > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const dim3 sgrid((unsigned)ntiles);
    hipLaunchKernelGGL(mask_scores_kernel, sgrid, dim3(256), 0, s, sc);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    SelectArgs se;
    se.scores = ws.scores;
    se.flags = ws.flags;
    se.mask = p.mask;
    se.kv_count = p.kv_count;
    se.kv_index = p.kv_index;
    se.B = p.B;
    se.Hq = p.Hq;
    se.Hkv = p.Hkv;
    se.G = p.Hq / p.Hkv;
    se.nb = p.nb;
    se.keep = p.keep_permille;
    se.qbar = ws.qbar;
    se.radius = ws.radius;
    se.thresh = ws.thresh;
    se.D = p.D;
    se.mode = p.rescue_mode;
    se.scale = p.scale;
    const long rows = (long)p.B * p.Hq * p.nb;
    const dim3 grid((unsigned)((rows + 3) / 4));
    const int E = (p.nb + 63) / 64;
    if (E <= 1) hipLaunchKernelGGL((mask_select_kernel<1>), grid, dim3(256), 0, s, se);
    else if (E <= 2) hipLaunchKernelGGL((mask_select_kernel<2>), grid, dim3(256), 0, s, se);
    else if (E <= 4) hipLaunchKernelGGL((mask_select_kernel<4>), grid, dim3(256), 0, s, se);
    else if (E <= 8) hipLaunchKernelGGL((mask_select_kernel<8>), grid, dim3(256), 0, s, se);
    else if (E <= 16) hipLaunchKernelGGL((mask_select_kernel<16>), grid, dim3(256), 0, s, se);
    else if (E <= 32) hipLaunchKernelGGL((mask_select_kernel<32>), grid, dim3(256), 0, s, se);
    else hipLaunchKernelGGL((mask_select_kernel<64>), grid, dim3(256), 0, s, se);
    return hipGetLastError();
}

}  // namespace lcattn
