// select.hip -- step a6: exact top-k block selection per query row.
//
// "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
// Attention": QSA keeps the best 512 blocks ("up to 512" when fewer are
// visible).  Readings: ties go to the lower block index; the kept blocks are
// listed in ascending order, padded with -1.
//
// Scores are compared through an order-preserving uint32 key.  One workgroup
// per row runs a radix select over the row's materialized scores:
//   A. histogram of key bits [31:20] -> the bin holding the k-th best key;
//   B. histogram of bits [19:8] inside that bin;
//   C. histogram of bits [7:0] inside the refined bin -> the exact k-th key T
//      and how many keys equal to T are kept;
//   D. one pass in block order keeps every key above T and the first `need`
//      keys equal to T (lowest block ids win); a workgroup-wide ballot scan
//      gives each kept block its output slot, so the list comes out ascending.
// A pass is skipped as soon as the whole bin is kept.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;

// Reported score s = raw / sqrt(128) (the score equation's scale), divided in
// double and rounded once to float.
__device__ __forceinline__ float scaled_score(float raw) { return (float)((double)raw / sqrt((double)kDim)); }

// Exclusive rank of `pred` among the workgroup's threads (thread order) and
// the workgroup-wide count.  Every thread must call it.
__device__ __forceinline__ uint32_t wg_rank(bool pred, uint32_t *wtot, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t m = __ballot(pred);
    const uint32_t in_wave = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t c = wtot[w];
        before += w < wave ? c : 0u;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + in_wave;
}

// Inclusive scan of a per-thread count over the workgroup (thread order).
__device__ __forceinline__ uint32_t wg_inclusive_scan(uint32_t v, uint32_t *wtot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wtot[wave] = x;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) before += w < wave ? wtot[w] : 0u;
    __syncthreads();
    return before + x;
}

// Bin b* of `hist` (nbins = 4096 or 256, scanned from the top) such that
// above(b*) < need <= above(b*) + hist[b*]; writes b* and above(b*) to LDS.
__device__ __forceinline__ void find_bin(const uint32_t *hist, int nbins, uint32_t need, uint32_t *wtot,
                                         uint32_t *out_bin, uint32_t *out_above)
{
    const int per = nbins / kSelThreads > 0 ? nbins / kSelThreads : 1;
    const int owned = (int)threadIdx.x * per < nbins ? per : 0;
    const int hi = nbins - (int)threadIdx.x * per;  // this thread owns [hi - owned, hi)
    uint32_t sum = 0;
    for (int i = 0; i < owned; ++i) sum += hist[hi - 1 - i];
    const uint32_t incl = wg_inclusive_scan(sum, wtot);
    const uint32_t before = incl - sum;
    if (owned && before < need && incl >= need) {
        uint32_t acc = before;
        for (int i = 0; i < owned; ++i) {
            const uint32_t c = hist[hi - 1 - i];
            if (acc + c >= need) {
                *out_bin = (uint32_t)(hi - 1 - i);
                *out_above = acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(const float *__restrict__ scores, int64_t sc_stride,
                                                                  const int32_t *__restrict__ row_pos, int32_t max_nb,
                                                                  int32_t top_k,
                                                                  int32_t *__restrict__ sel_blocks,
                                                                  int32_t *__restrict__ sel_count,
                                                                  float *__restrict__ sel_scores)
{
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t wtot[kSelWaves];
    __shared__ uint32_t s_bin, s_above;
    const int64_t r = blockIdx.x;
    const int32_t nc = (int32_t)min(visible_blocks(row_pos[r]), (int64_t)max_nb);  // max_nb: caller's bound
    const float *srow = scores + r * sc_stride;
    int32_t *out = sel_blocks + r * top_k;
    float *osc = sel_scores ? sel_scores + r * top_k : nullptr;
    const int32_t kk = min(top_k, nc);
    if (threadIdx.x == 0) sel_count[r] = kk;
    for (int32_t i = kk + threadIdx.x; i < top_k; i += kSelThreads) {
        out[i] = -1;
        if (osc) osc[i] = 0.0f;
    }
    if (nc <= top_k) {  // every visible block is kept
        for (int32_t b = threadIdx.x; b < nc; b += kSelThreads) {
            out[b] = b;
            if (osc) osc[b] = scaled_score(srow[b]);
        }
        return;
    }
    // ---- A/B/C: radix passes narrowing to the k-th key ----
    uint32_t need = (uint32_t)kk;
    uint32_t prefix = 0;  // resolved top bits of the k-th key
    int sh = 32;          // key >> sh == prefix marks the current bin
    const int widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
        const int w = widths[pass];
        const int nsh = sh - w;
        const int nbins = 1 << w;
        for (int i = threadIdx.x; i < nbins; i += kSelThreads) hist[i] = 0u;
        __syncthreads();
        for (int32_t b = threadIdx.x; b < nc; b += kSelThreads) {
            const uint32_t key = score_key(srow[b]);
            if (sh == 32 || (key >> sh) == prefix) atomicAdd(&hist[(key >> nsh) & (uint32_t)(nbins - 1)], 1u);
        }
        __syncthreads();
        find_bin(hist, nbins, need, wtot, &s_bin, &s_above);
        const uint32_t bin = s_bin, above = s_above;
        const uint32_t cnt = hist[bin];
        __syncthreads();
        need -= above;
        prefix = (sh == 32 ? 0u : (prefix << w)) | bin;
        sh = nsh;
        if (cnt == need) break;  // the whole bin is kept
    }
    // ---- D: keys above the bin, and the first `need` keys inside it ----
    uint32_t eq_before = 0, out_before = 0;
    for (int32_t b0 = 0; b0 < nc; b0 += kSelThreads) {
        const int32_t b = b0 + threadIdx.x;
        const bool valid = b < nc;
        const float sc = valid ? srow[b] : 0.0f;
        const uint32_t top = valid ? (score_key(sc) >> sh) : 0u;
        const bool gt = valid && top > prefix;
        const bool eq = valid && top == prefix;
        uint32_t eq_total, take_total;
        const uint32_t eq_rank = eq_before + wg_rank(eq, wtot, eq_total);
        const bool take = gt || (eq && eq_rank < need);
        const uint32_t pos = out_before + wg_rank(take, wtot, take_total);
        if (take && pos < (uint32_t)kk) {
            out[pos] = b;
            if (osc) osc[pos] = scaled_score(sc);
        }
        eq_before += eq_total;
        out_before += take_total;
    }
}

void launch_select_rows(const float *scores, int64_t sc_stride, const int32_t *row_pos, int32_t rows, int32_t max_nb,
                        int32_t top_k, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores, hipStream_t stream)
{
    QSA_LAUNCH("select_rows", select_rows_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, stream, scores,
               sc_stride, row_pos, max_nb, top_k, sel_blocks, sel_count, sel_scores);
}

}  // namespace qsa
