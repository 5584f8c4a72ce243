// qsa_wg.h -- workgroup-wide scans and the radix-select bin search shared by
// the selection kernels.  Every thread of the workgroup must call them.
#pragma once

#include "qsa_device.h"

namespace qsa {

// Exclusive rank of `pred` among the workgroup's threads (thread order) and
// the workgroup-wide count.  Every thread must call it.
template <int NT>
__device__ __forceinline__ uint32_t wg_rank(bool pred, uint32_t *wtot, uint32_t &total)
{
    constexpr int kSelWaves = NT / kWave;
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
template <int NT>
__device__ __forceinline__ uint32_t wg_inclusive_scan(uint32_t v, uint32_t *wtot)
{
    constexpr int kSelWaves = NT / kWave;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);  // DPP row shifts and broadcasts: no LDS round trips
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
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t *hist, int nbins, uint32_t need, uint32_t *wtot,
                                         uint32_t *out_bin, uint32_t *out_above)
{
    const int per = nbins / NT > 0 ? nbins / NT : 1;
    const int owned = (int)threadIdx.x * per < nbins ? per : 0;
    const int hi = nbins - (int)threadIdx.x * per;  // this thread owns [hi - owned, hi)
    uint32_t sum = 0;
    for (int i = 0; i < owned; ++i) sum += hist[hi - 1 - i];
    const uint32_t incl = wg_inclusive_scan<NT>(sum, wtot);
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

}  // namespace qsa
