// score_fused.hip -- steps a5-a6 for many rows: block scores on bf16 MFMA with
// the top-k filter fused into the GEMM, then an exact per-row merge.
//
// "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
// Attention": s_{t,b} = 1/sqrt(128) * sum over 4 index heads of
// ReLU(<q_{t,h}, kbar_b>) over the visible blocks, and the best 512 blocks are
// kept.  Readings: ties go to the lower block id; the selection ranks the
// un-scaled sum.
//
// Materializing every score would cost 4 bytes per (row, block) pair of HBM
// traffic, more than the GEMM's own time at MFMA rate, so the GEMM keeps per
// row a lower bound tau on the row's k-th best score and writes out only the
// pairs with score >= tau.  tau is valid whenever at least k already written
// pairs of the row score >= tau (then the k-th best of all visible blocks is
// >= tau, and a pair below it cannot be kept).  Each row counts its written
// pairs in a 256-bin histogram over key space -- 1/32 octave per bin, 4
// octaves either side of an anchor (the row's best score in its first 64
// blocks), everything above or below lumped into the end bins -- and after
// every 64-block step a row that received pairs raises tau to the lowest key
// of the highest bin at which k pairs are reached.
//
// Workgroup: 4 waves x 16 query rows (MFMA row m of tile mt = query row
// 4*mt + m/4, index head m%4, so a lane's 4 accumulators are the 4 heads of
// one (row, block) pair), one split of the block range.  The 64-block key
// tile is staged through LDS (double buffered) and shared by the 4 waves.
// The merge kernel takes, per row, the pairs of every split at or above the
// best split's tau, picks the exact top k with a radix select on the unique
// composite (key, ~block), and emits them sorted by block.  A row whose pair
// buffer overflowed (e.g. massive exact ties) is redone by the merge kernel
// from recomputed scores.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

constexpr int kFRows = 64;            // rows per workgroup
constexpr int kFStep = 64;            // blocks per step
constexpr int kFKRow = kDim + 8;      // LDS key row stride (bf16): conflict-free b128 reads
constexpr int kTauBins = 256;
constexpr int kTauShift = 18;         // 2^18 key units = 1/32 octave
constexpr int64_t kTauHalf = 1ll << 25;  // 4 octaves
constexpr int kMergeThreads = 256;
constexpr int kMergeLds = 4096;       // pairs a merge workgroup stages in LDS

__device__ __forceinline__ float relu_sum4f(f32x4_t a)
{
    return ((fmaxf(a[0], 0.0f) + fmaxf(a[1], 0.0f)) + fmaxf(a[2], 0.0f)) + fmaxf(a[3], 0.0f);
}

__device__ __forceinline__ int tau_bin(uint32_t key, uint32_t anchor)
{
    const int64_t d = (int64_t)anchor + kTauHalf - (int64_t)key;
    if (d < 0) return 0;
    const int64_t b = d >> kTauShift;
    return b >= kTauBins - 1 ? kTauBins - 1 : (int)b;
}

// Threshold key -> float for `score >= tau` (key 0: no threshold yet).
__device__ __forceinline__ float tau_float(uint32_t key) { return key == 0u ? -INFINITY : key_score(key); }

// Lowest key of bin b (the last bin reaches down to every key).
__device__ __forceinline__ uint32_t tau_bin_floor(int b, uint32_t anchor)
{
    if (b >= kTauBins - 1) return 0u;
    const int64_t k = (int64_t)anchor + kTauHalf - ((int64_t)(b + 1) << kTauShift) + 1;
    return k <= 0 ? 0u : (k >= 0xffffffffll ? 0xffffffffu : (uint32_t)k);
}

}  // namespace

__global__ __launch_bounds__(256) void score_filter_kernel(FusedScoreArgs a)
{
    const bf16_t *__restrict__ qrot = (const bf16_t *)a.qrot;
    const bf16_t *__restrict__ pooled = (const bf16_t *)a.pooled;
    __shared__ bf16_t keys[2][kFStep][kFKRow];
    __shared__ uint32_t hist[kFRows][kTauBins / 2];  // two 16-bit bins per word
    __shared__ uint32_t cnt[kFRows], tau[kFRows], anchor[kFRows], dirty[kFRows];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * kFRows;
    const int nrows = (int)min((int64_t)kFRows, (int64_t)a.rows - row0);
    const int split = blockIdx.y;
    const int64_t split_lo = (int64_t)split * a.split_len;
    const int64_t split_hi = min((int64_t)a.max_nb, split_lo + a.split_len);
    for (int i = t; i < kFRows * kTauBins / 2; i += 256) (&hist[0][0])[i] = 0u;
    if (t < kFRows) {
        cnt[t] = 0u;
        tau[t] = 0u;
        anchor[t] = 0x80000000u;
        dirty[t] = 0u;
    }
    // A operands: this wave's 16 rows x 4 heads
    bf16x8_t qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + (m >> 2);
        const bool ok = rw < nrows;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[mt][s] = ok ? as_bf16x8(*(const uint4 *)(qrot + ((row0 + rw) * kIdxHeads + (m & 3)) * kDim + 32 * g + 8 * s))
                           : zero_bf16x8();
    }
    // the 4 rows whose scores this lane receives: 16*wave + 4*mt + g
    int64_t my_nc[4];
    int32_t my_seq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + g;
        my_nc[mt] = rw < nrows ? min(visible_blocks(a.row_pos[row0 + rw]), (int64_t)a.max_nb) : 0;
        my_seq[mt] = rw < nrows ? a.row_seq[row0 + rw] : -1;
    }
    __syncthreads();
    uint64_t todo = nrows >= 64 ? ~0ull : ((1ull << nrows) - 1ull);
    while (todo) {  // rows of one sequence at a time (uniform across the workgroup)
        const int first = __builtin_ctzll(todo);
        const int32_t seq = a.row_seq[row0 + first];
        int64_t nb_hi = 0;
        uint64_t active = 0;
        for (int r = first; r < nrows; ++r)
            if (((todo >> r) & 1ull) && a.row_seq[row0 + r] == seq) {
                active |= 1ull << r;
                nb_hi = max(nb_hi, min(visible_blocks(a.row_pos[row0 + r]), (int64_t)a.max_nb));
            }
        todo &= ~active;
        int64_t lim[4];  // visible bound of the lane's rows in this pass (0: not in it)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) lim[mt] = my_seq[mt] == seq ? my_nc[mt] : 0;
        const int64_t lo = split_lo, hi = min(split_hi, nb_hi);
        if (lo >= hi) continue;
        const bf16_t *kb = pooled + (int64_t)seq * a.pooled_stride;
        // key tile loader: thread -> block t/4 of the step, 64 bytes at dim 32*(t%4)
        const int lrow = t >> 2, ldim = (t & 3) * 32;
        uint4 pre[4];
        auto load_tile = [&](int64_t base) {
            const int64_t b = min(base + lrow, hi - 1);
            const uint4 *src = (const uint4 *)(kb + b * kDim + ldim);
#pragma unroll
            for (int i = 0; i < 4; ++i) pre[i] = src[i];
        };
        auto store_tile = [&](int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) *(uint4 *)&keys[buf][lrow][ldim + 8 * i] = pre[i];
        };
        load_tile(lo);
        store_tile(0);
        __syncthreads();
        float tauf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) tauf[mt] = tau_float(tau[16 * wave + 4 * mt + g]);
        int cur = 0;
        bool first_step = true;
        for (int64_t base = lo; base < hi; base += kFStep) {
            const bool more = base + kFStep < hi;
            if (more) load_tile(base + kFStep);
            // ---- scores of the step: 4 row tiles x 4 block tiles ----
            float sc[4][4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                bf16x8_t bk[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) bk[s] = as_bf16x8(*(const uint4 *)&keys[cur][nt * 16 + m][32 * g + 8 * s]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], bk[s], acc, 0, 0, 0);
                    sc[mt][nt] = relu_sum4f(acc);
                }
            }
            if (more) store_tile(cur ^ 1);
            // ---- anchors: each row's best score in its first step ----
            if (first_step) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    float mx = 0.0f;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        if (base + nt * 16 + m < lim[mt]) mx = fmaxf(mx, sc[mt][nt]);
                    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
                    if (m == 0 && lim[mt] > 0) anchor[16 * wave + 4 * mt + g] = score_key(mx);
                }
                first_step = false;
            }
            // ---- filter: pairs at or above the row's tau are written out ----
            bool pass[4][4];
            bool any = false;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    pass[mt][nt] = sc[mt][nt] >= tauf[mt] && base + nt * 16 + m < lim[mt];
                    any |= pass[mt][nt];
                }
            if (__ballot(any)) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int rw = 16 * wave + 4 * mt + g;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        if (!pass[mt][nt]) continue;
                        const uint32_t key = score_key(sc[mt][nt]);
                        const uint32_t slot = atomicAdd(&cnt[rw], 1u);
                        if (slot < (uint32_t)a.cap) {
                            a.buf[((row0 + rw) * a.nsplit + split) * (int64_t)a.cap + slot] =
                                make_uint2(key, (uint32_t)(base + nt * 16 + m));
                            const int bin = tau_bin(key, anchor[rw]);
                            atomicAdd(&hist[rw][bin >> 1], (bin & 1) ? 0x10000u : 1u);
                            dirty[rw] = 1u;
                        }
                    }
                }
                // ---- raise tau of the wave's rows that received pairs ----
                bool changed = false;
                for (int i = 0; i < 16; ++i) {
                    const int rw = 16 * wave + i;
                    if (!dirty[rw]) continue;  // wave-uniform (LDS broadcast)
                    const uint32_t c = cnt[rw];
                    if (lane == 0) dirty[rw] = 0u;
                    if (c < (uint32_t)a.top_k || c > (uint32_t)a.cap) continue;
                    const uint32_t w0 = hist[rw][2 * lane], w1 = hist[rw][2 * lane + 1];
                    const uint32_t h4[4] = {w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16};
                    const uint32_t sum = h4[0] + h4[1] + h4[2] + h4[3];
                    uint32_t incl = sum;
                    for (int o = 1; o < 64; o <<= 1) {
                        const uint32_t y = __shfl_up(incl, o);
                        if (lane >= o) incl += y;
                    }
                    const uint64_t reach = __ballot(incl >= (uint32_t)a.top_k);
                    const int l_star = __ffsll((unsigned long long)reach) - 1;  // exists: total >= top_k
                    int b_star = kTauBins - 1;
                    if (lane == l_star) {
                        uint32_t acc = incl - sum;
                        for (int j = 0; j < 4; ++j) {
                            acc += h4[j];
                            if (acc >= (uint32_t)a.top_k) {
                                b_star = 4 * lane + j;
                                break;
                            }
                        }
                    }
                    b_star = __shfl(b_star, l_star);
                    const uint32_t nt_key = tau_bin_floor(b_star, anchor[rw]);
                    if (nt_key > tau[rw]) {
                        if (lane == 0) tau[rw] = nt_key;
                        changed = true;
                    }
                }
                if (changed) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) tauf[mt] = tau_float(tau[16 * wave + 4 * mt + g]);
                }
            }
            __syncthreads();
            cur ^= 1;
        }
        __syncthreads();
    }
    if (t < nrows) {
        a.cnt[(row0 + t) * a.nsplit + split] = cnt[t];
        a.tau[(row0 + t) * a.nsplit + split] = tau[t];
    }
}

// ---------------------------------------------------------------------------
// Merge: one workgroup per row.
// ---------------------------------------------------------------------------
namespace {

template <int NT>
__device__ __forceinline__ uint32_t incl_scan(uint32_t v, uint32_t *wtot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wtot[w];
    __syncthreads();
    return before + x;
}

template <int NT>
__device__ __forceinline__ uint32_t rank_of(bool pred, uint32_t *wtot, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t msk = __ballot(pred);
    const uint32_t in_wave = (uint32_t)__popcll(msk & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[wave] = (uint32_t)__popcll(msk);
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int w = 0; w < NT / kWave; ++w) {
        before += w < wave ? wtot[w] : 0u;
        tot += wtot[w];
    }
    __syncthreads();
    total = tot;
    return before + in_wave;
}

__device__ __forceinline__ uint64_t composite32(uint2 e) { return ((uint64_t)e.x << 32) | (uint64_t)(~e.y); }

// Raw score of (row, block) recomputed on the VALU (bf16 operands, fp32 sums).
__device__ __forceinline__ float recompute_score(const bf16_t *__restrict__ q4, const bf16_t *__restrict__ key)
{
    float d[kIdxHeads] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 0; i < kDim; i += 8) {
        float kv[8];
        load8(key + i, kv);
#pragma unroll
        for (int h = 0; h < kIdxHeads; ++h) {
            float qv[8];
            load8(q4 + h * kDim + i, qv);
#pragma unroll
            for (int e = 0; e < 8; ++e) d[h] = fmaf(qv[e], kv[e], d[h]);
        }
    }
    return ((fmaxf(d[0], 0.0f) + fmaxf(d[1], 0.0f)) + fmaxf(d[2], 0.0f)) + fmaxf(d[3], 0.0f);
}

}  // namespace

__global__ __launch_bounds__(kMergeThreads) void select_merge_kernel(FusedScoreArgs a, int32_t *__restrict__ sel_blocks,
                                                                   int32_t *__restrict__ sel_count,
                                                                   float *__restrict__ sel_scores)
{
    __shared__ uint2 stage[kMergeLds];
    __shared__ uint64_t kept[QSA_MAX_TOP_K];
    __shared__ uint32_t dh[256];
    __shared__ uint32_t wtot[kMergeThreads / kWave];
    __shared__ uint32_t s_n, s_digit, s_above, s_cnt, s_fill;
    const int t = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int32_t nc = (int32_t)min(visible_blocks(a.row_pos[r]), (int64_t)a.max_nb);
    const int32_t kk = min(a.top_k, nc);
    int32_t *out = sel_blocks + r * a.top_k;
    float *osc = sel_scores ? sel_scores + r * a.top_k : nullptr;
    if (nc <= 0) {  // no visible block (the scorer may not have run at all)
        if (t == 0) sel_count[r] = 0;
        for (int32_t i = t; i < a.top_k; i += kMergeThreads) {
            out[i] = -1;
            if (osc) osc[i] = 0.0f;
        }
        return;
    }
    // pairs of every split; the best split's tau bounds the row's k-th best
    bool overflow = false;
    uint32_t tau_max = 0, total = 0;
    for (int s = 0; s < a.nsplit; ++s) {
        const uint32_t c = a.cnt[r * a.nsplit + s];
        overflow |= c > (uint32_t)a.cap;
        total += min(c, (uint32_t)a.cap);
        tau_max = max(tau_max, a.tau[r * a.nsplit + s]);
    }
    if (t == 0) sel_count[r] = kk;
    if (!overflow) {
        // stage the pairs >= tau_max (LDS when they fit, else they are re-read)
        if (t == 0) s_n = 0;
        __syncthreads();
        for (int s = 0; s < a.nsplit; ++s) {
            const uint32_t c = min(a.cnt[r * a.nsplit + s], (uint32_t)a.cap);
            const uint2 *src = a.buf + (r * a.nsplit + s) * (int64_t)a.cap;
            for (uint32_t i0 = 0; i0 < c; i0 += kMergeThreads) {
                const uint32_t i = i0 + t;
                const uint2 e = i < c ? src[i] : make_uint2(0u, 0u);
                const bool keep = i < c && e.x >= tau_max;
                uint32_t tot;
                const uint32_t rk = rank_of<kMergeThreads>(keep, wtot, tot);
                if (keep && s_n + rk < (uint32_t)kMergeLds) stage[s_n + rk] = e;
                __syncthreads();
                if (t == 0) s_n += tot;
                __syncthreads();
            }
        }
        const uint32_t n = s_n;
        if (n <= (uint32_t)kMergeLds) {
            // radix select of the kk-th largest composite among stage[0..n)
            uint32_t need = (uint32_t)kk;
            uint64_t prefix = 0, pmask = 0;
            if (need < n) {
                for (int sh = 56; sh >= 0; sh -= 8) {
                    dh[t] = 0u;
                    __syncthreads();
                    for (uint32_t i = t; i < n; i += kMergeThreads) {
                        const uint64_t c = composite32(stage[i]);
                        if ((c & pmask) == prefix) atomicAdd(&dh[(uint32_t)(c >> sh) & 0xffu], 1u);
                    }
                    __syncthreads();
                    const uint32_t hv = dh[255 - t];
                    const uint32_t incl = incl_scan<kMergeThreads>(hv, wtot);
                    if (hv && incl - hv < need && incl >= need) {
                        s_digit = 255u - (uint32_t)t;
                        s_above = incl - hv;
                        s_cnt = hv;
                    }
                    __syncthreads();
                    prefix |= (uint64_t)s_digit << sh;
                    pmask |= 0xffull << sh;
                    need -= s_above;
                    const bool done = s_cnt == need;
                    __syncthreads();
                    if (done) break;
                }
            }
            if (t == 0) s_fill = 0;
            __syncthreads();
            for (uint32_t i = t; i < n; i += kMergeThreads) {
                const uint2 e = stage[i];
                if ((composite32(e) & pmask) >= prefix) {
                    const uint32_t at = atomicAdd(&s_fill, 1u);
                    if (at < (uint32_t)QSA_MAX_TOP_K) kept[at] = ((uint64_t)e.y << 32) | e.x;
                }
            }
            __syncthreads();
            const uint32_t nk = min(s_fill, (uint32_t)kk);
            uint32_t n2 = 1;
            while (n2 < nk) n2 <<= 1;
            for (uint32_t i = nk + t; i < n2; i += kMergeThreads) kept[i] = ~0ull;
            __syncthreads();
            for (uint32_t size = 2; size <= n2; size <<= 1) {
                for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
                    for (uint32_t i = t; i < n2 / 2; i += kMergeThreads) {
                        const uint32_t lo = 2 * i - (i & (stride - 1));
                        const uint32_t hi = lo + stride;
                        const bool up = (lo & size) == 0;
                        const uint64_t x = kept[lo], y = kept[hi];
                        if ((x > y) == up) {
                            kept[lo] = y;
                            kept[hi] = x;
                        }
                    }
                    __syncthreads();
                }
            }
            for (int32_t i = t; i < a.top_k; i += kMergeThreads) {
                const bool k_ = (uint32_t)i < nk;
                const uint64_t e = k_ ? kept[i] : 0ull;
                out[i] = k_ ? (int32_t)(e >> 32) : -1;
                if (osc) osc[i] = k_ ? (float)((double)key_score((uint32_t)e) / sqrt((double)kDim)) : 0.0f;
            }
            return;
        }
    }
    // ---- fallback: radix select over recomputed scores of every visible block,
    // in block order (too many pairs for the staged merge) ----
    const int32_t seq = a.row_seq[r];
    const bf16_t *q4 = (const bf16_t *)a.qrot + r * kIdxHeads * kDim;
    const bf16_t *kb = (const bf16_t *)a.pooled + (int64_t)seq * a.pooled_stride;
    uint32_t need = (uint32_t)kk;
    uint32_t prefix = 0;
    int sh = 32;
    const int widths[4] = {8, 8, 8, 8};
    for (int pass = 0; pass < 4 && need > 0; ++pass) {
        const int nsh = sh - widths[pass];
        dh[t] = 0u;
        __syncthreads();
        for (int32_t b = t; b < nc; b += kMergeThreads) {
            const uint32_t key = score_key(recompute_score(q4, kb + (int64_t)b * kDim));
            if (sh == 32 || (key >> sh) == prefix) atomicAdd(&dh[(key >> nsh) & 0xffu], 1u);
        }
        __syncthreads();
        const uint32_t hv = dh[255 - t];
        const uint32_t incl = incl_scan<kMergeThreads>(hv, wtot);
        if (hv && incl - hv < need && incl >= need) {
            s_digit = 255u - (uint32_t)t;
            s_above = incl - hv;
            s_cnt = hv;
        }
        __syncthreads();
        need -= s_above;
        prefix = (sh == 32 ? 0u : (prefix << 8)) | s_digit;
        sh = nsh;
        const bool done = s_cnt == need;
        __syncthreads();
        if (done) break;
    }
    uint32_t eq_before = 0, out_before = 0;
    for (int32_t b0 = 0; b0 < nc; b0 += kMergeThreads) {
        const int32_t b = b0 + t;
        const bool valid = b < nc;
        const float sc = valid ? recompute_score(q4, kb + (int64_t)b * kDim) : 0.0f;
        const uint32_t top = valid ? (score_key(sc) >> sh) : 0u;
        const bool gt = valid && top > prefix;
        const bool eq = valid && top == prefix;
        uint32_t eq_total, take_total;
        const uint32_t eq_rank = eq_before + rank_of<kMergeThreads>(eq, wtot, eq_total);
        const bool take = gt || (eq && eq_rank < need);
        const uint32_t pos = out_before + rank_of<kMergeThreads>(take, wtot, take_total);
        if (take && pos < (uint32_t)kk) {
            out[pos] = b;
            if (osc) osc[pos] = (float)((double)sc / sqrt((double)kDim));
        }
        eq_before += eq_total;
        out_before += take_total;
    }
    for (int32_t i = kk + t; i < a.top_k; i += kMergeThreads) {
        out[i] = -1;
        if (osc) osc[i] = 0.0f;
    }
}

// Split of the block range: enough workgroups to fill the chip, each split a
// multiple of the step.
int32_t fused_score_splits(int32_t rows, int32_t max_nb)
{
    const int64_t tiles = ((int64_t)rows + kFRows - 1) / kFRows;
    int64_t s = (512 + tiles - 1) / tiles;
    s = min(s, ((int64_t)max_nb + 4095) / 4096);  // at least 4096 blocks per split
    return (int32_t)max((int64_t)1, s);
}

int32_t fused_score_split_len(int32_t max_nb, int32_t nsplit)
{
    const int64_t len = ((int64_t)max_nb + nsplit - 1) / nsplit;
    return (int32_t)((len + kFStep - 1) / kFStep * kFStep);
}

int32_t fused_score_cap(int32_t top_k) { return max(4096, 8 * top_k); }

void launch_score_fused(const FusedScoreArgs &a, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                        hipStream_t stream)
{
    if (a.max_nb > 0) {
        const dim3 grid((unsigned)((a.rows + kFRows - 1) / kFRows), (unsigned)a.nsplit), block(256);
        QSA_LAUNCH("score_filter", score_filter_kernel, grid, block, 0, stream, a);
    }
    QSA_LAUNCH("select_merge", select_merge_kernel, dim3((unsigned)a.rows), dim3(kMergeThreads), 0, stream, a,
               sel_blocks, sel_count, sel_scores);
}

}  // namespace qsa
