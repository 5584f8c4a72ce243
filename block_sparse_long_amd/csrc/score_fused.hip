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
// traffic, more than the GEMM's own time at MFMA rate.  Instead:
//   1. sample: every row is scored against one block in 32 (a fixed
//      pseudo-random pick inside each group of 32), about 3% of the GEMM;
//      each lane keeps its 4 best sampled scores per row;
//   2. threshold: tau = the j-th best of those candidates, j = ceil(2.5k/32),
//      which is at most the row's j-th best sampled score (so about 2.5k of
//      the row's blocks are expected to score >= tau);
//   3. filter: the full GEMM writes out only the (key, block) pairs with
//      score >= tau, each lane into its own list (no atomics, no cross-lane
//      work in the MFMA loop);
//   4. merge: a row is exact when at least min(k, nc) of its pairs reached
//      tau -- then the k-th best of all visible blocks is >= tau and every
//      block it keeps is among the pairs -- and the merge finds the k-th
//      best key T among them (radix select), sorts the pairs >= T by block,
//      and keeps those above T and the lowest-block ones equal to it.  A row
//      whose count fell short, or whose list overflowed, is redone from
//      recomputed scores of every visible block.
// Workgroup of the GEMMs: 4 waves x 16 query rows; MFMA row m of tile mt is
// query row 4*mt + m/4, index head m%4, so a lane's 4 accumulators are the 4
// heads of one (row, block) pair and the ReLU-sum stays in the lane.  The
// 64-block key tile is staged through LDS (double buffered) and shared by the
// 4 waves.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_wg.h"

namespace qsa {

namespace {

constexpr int kFRows = 64;            // rows per GEMM workgroup
constexpr int kFStep = 64;            // blocks per step
constexpr int kFKRow = kDim + 8;      // LDS key row stride (bf16): conflict-free b128 reads
constexpr int kSampleStride = 32;     // one sampled block per 32
constexpr int kMergeWaves = 4;        // merge: rows per workgroup, one wave each
constexpr int kStage = 2048;          // merge: pairs a wave stages in LDS

// tau is the j-th best sampled score of a row, j = ceil(2.5 k / 32): about
// 2.5 k of the row's blocks reach it.  The row's k-th best block is below tau
// only if at least j of its k best blocks were sampled; for k = 512 that
// takes 40 of an expected 16 (binomial tail 1.8e-7 per row when the best
// blocks fall at random, less when they cluster).  Such a row is still
// exact: the merge recomputes it.
__host__ __device__ __forceinline__ int32_t sample_j(int32_t top_k)
{
    return (5 * top_k + 2 * kSampleStride - 1) / (2 * kSampleStride);
}

// Block of sample i: group i of 32 blocks, a fixed pseudo-random offset in it.
__device__ __forceinline__ int64_t sample_block(int64_t i)
{
    const uint32_t h = (uint32_t)i * 2654435761u;  // Knuth's multiplicative hash
    return i * kSampleStride + (h >> 27);
}

__device__ __forceinline__ float relu_sum4f(f32x4_t a)
{
    return ((relu(a[0]) + relu(a[1])) + relu(a[2])) + relu(a[3]);
}

// Order key of a non-negative score (a sum of ReLUs; -0 and +0 map to one key).
__device__ __forceinline__ uint32_t pos_key(float s) { return __float_as_uint(s) | 0x80000000u; }

__device__ __forceinline__ float tau_float(uint32_t key) { return key == 0u ? -INFINITY : key_score(key); }

__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

// A row's pair lists: 16 per split.  With the block range split (short lists,
// many rows' lists growing at once) the 16 lists of a split are interleaved slot
// by slot (pair j of list m at 16 j + m): an append instruction's lanes of one
// row at the same slot share a line, and the merge reads a row's lists in whole
// lines.  With one split (long lists that fill out of step) each list is
// contiguous (pair j of list m at subcap m + j) and fills its own lines.
__host__ __device__ __forceinline__ bool lists_interleaved(int32_t nsplit) { return nsplit >= 2; }
__device__ __forceinline__ int64_t list_slot(int li, uint32_t j, int32_t subcap, bool inter)
{
    return inter ? (int64_t)(li >> 4) * 16 * subcap + (int64_t)j * 16 + (li & 15) : (int64_t)li * subcap + j;
}

// The 16 x 4 x 128 query tile of a wave as MFMA A operands.
__device__ __forceinline__ void load_query_tile(const bf16_t *__restrict__ qrot, int64_t row0, int nrows, int wave,
                                                bf16x8_t (&qa)[4][4])
{
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + (m >> 2);
        // a row slot past the tile's rows takes the last row's query (clamped, so every load
        // is issued together with no branch): its scores are finite and never used, since the
        // slot belongs to no sequence and has tau = +inf
        const int rc = min(rw, nrows - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qa[mt][s] = as_bf16x8(*(const uint4 *)(qrot + ((row0 + rc) * kIdxHeads + (m & 3)) * kDim + 32 * g + 8 * s));
    }
}

// Scores of one 64-block tile in LDS: sc[mt][nt] = raw(row 16*wave + 4*mt + g,
// block nt*16 + m of the tile).  Four independent accumulator chains per
// 16-block slice; a slice's ReLU-sums are interleaved with the next slice's
// MFMAs.
__device__ __forceinline__ void tile_scores(const bf16_t (*keys)[kFKRow], const bf16x8_t (&qa)[4][4],
                                            float (&sc)[4][4])
{
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    f32x4_t acc[2][4];  // slice nt's accumulators; slice nt-1's ReLU-sums run between its MFMAs
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        bf16x8_t bk[4];  // the slice's 4 key operands are read together, before its MFMAs
#pragma unroll
        for (int s = 0; s < 4; ++s) bk[s] = as_bf16x8(*(const uint4 *)&keys[nt * 16 + m][32 * g + 8 * s]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[nt & 1][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[nt & 1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], bk[s], acc[nt & 1][mt], 0, 0, 0);
            if (nt > 0) sc[s][nt - 1] = relu_sum4f(acc[(nt - 1) & 1][s]);  // row tile s of the previous slice
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) sc[mt][3] = relu_sum4f(acc[1][mt]);
}

// Row r of a 64-row tile as lane r of every wave holds it: its sequence (-1
// past the tile's rows) and its visible-block count, read once, in parallel.
struct TileRows {
    int32_t seq;
    int32_t nb;
};
__device__ __forceinline__ TileRows tile_rows(const FusedScoreArgs &a, int64_t row0, int nrows)
{
    static_assert(kFRows == kWave, "one tile row per lane");
    const int lane = threadIdx.x & 63;
    const int32_t okm = lane < nrows ? -1 : 0;
    const int rc = min(lane, nrows - 1);  // loads issued unconditionally (clamped), then masked
    const int32_t sq = a.row_seq[row0 + rc], p = a.row_pos[row0 + rc];
    TileRows tr;
    tr.seq = sq | ~okm;
    tr.nb = (int32_t)min(visible_blocks(p), (int64_t)a.max_nb) & okm;
    return tr;
}

// Rows of one sequence at a time: the next group of the workgroup's rows
// (uniform across the workgroup), found with one ballot.  Returns the
// sequence and the largest visible-block count of the group; clears the
// group's bits from `todo`.
__device__ __forceinline__ int32_t next_seq_group(const TileRows &tr, uint64_t &todo, int64_t &nb_hi)
{
    const int lane = threadIdx.x & 63;
    const int first = __builtin_ctzll(todo);
    const int32_t seq = (int32_t)lane_value((uint32_t)tr.seq, first);
    const bool in = ((todo >> lane) & 1ull) && tr.seq == seq;
    todo &= ~__ballot(in);
    const uint32_t nbmax =
        wave_incl_scan_op((uint32_t)(in ? tr.nb : 0), [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    nb_hi = (int64_t)lane_value(nbmax, 63);
    return seq;
}

// One thread's share of a 64-block key tile (block b of sequence seq, dims
// ldim .. ldim + 31) on its way to LDS as bf16.  FP8 keys are read as 32
// codes and converted when stored (exactly); their scale goes to the tile's
// scale row, written by the first of the block's 4 threads.
template <bool FP8> struct TileShare;
template <> struct TileShare<false> {
    uint4 p0, p1, p2, p3;
    // element-wise vector loads: a plain 64-byte copy into the struct would be
    // turned into a block copy and kept in scratch memory
    // pg: the table entry of b's page (paged pools)
    __device__ __forceinline__ void load(const FusedScoreArgs &a, int32_t seq, int64_t b, int ldim, int32_t pg)
    {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const int64_t off = a.kp.table ? key_at(a.kp, 0, seq, b, pg) * kDim : seq * a.pooled_stride + b * kDim;
        const u32x4_t *src = (const u32x4_t *)((const bf16_t *)a.pooled + off + ldim);
        const u32x4_t x0 = src[0], x1 = src[1], x2 = src[2], x3 = src[3];
        p0 = make_uint4(x0.x, x0.y, x0.z, x0.w);
        p1 = make_uint4(x1.x, x1.y, x1.z, x1.w);
        p2 = make_uint4(x2.x, x2.y, x2.z, x2.w);
        p3 = make_uint4(x3.x, x3.y, x3.z, x3.w);
    }
    __device__ __forceinline__ void store(bf16_t *row, float *, bool) const
    {
        uint4 *dst = (uint4 *)row;
        dst[0] = p0;
        dst[1] = p1;
        dst[2] = p2;
        dst[3] = p3;
    }
};
template <> struct TileShare<true> {
    uint4 c[2];  // indexed with constants only
    float s;
    __device__ __forceinline__ void load(const FusedScoreArgs &a, int32_t seq, int64_t b, int ldim, int32_t pg)
    {
        const int64_t key = key_at(a.kp, a.pooled_stride, seq, b, pg);
        const uint4 *src = (const uint4 *)(a.codes + key * kDim + ldim);
        c[0] = src[0];
        c[1] = src[1];
        s = a.scales[key];
    }
    __device__ __forceinline__ void store(bf16_t *row, float *scale, bool first) const
    {
        uint4 *dst = (uint4 *)row;
        dst[0] = __builtin_bit_cast(uint4, fp8x8_to_bf16x8(c[0].x, c[0].y));
        dst[1] = __builtin_bit_cast(uint4, fp8x8_to_bf16x8(c[0].z, c[0].w));
        dst[2] = __builtin_bit_cast(uint4, fp8x8_to_bf16x8(c[1].x, c[1].y));
        dst[3] = __builtin_bit_cast(uint4, fp8x8_to_bf16x8(c[1].z, c[1].w));
        if (first) *scale = s;
    }
};

// FP8 keys: a block's ReLU-sum times its scale (column m of slice nt is block
// nt*16 + m of the tile).
template <bool FP8>
__device__ __forceinline__ void apply_scales(const float *tile_scale, float (&sc)[4][4])
{
    if (!FP8) return;
    const int m = threadIdx.x & 15;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const float f = tile_scale[nt * 16 + m];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sc[mt][nt] *= f;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. sample: grid (row tiles, sample-range splits).  Lane (mt, g, m) keeps the
//    4 best scores of row 16*wave + 4*mt + g among the samples it computes
//    (samples i with i % 16 == m of each 64-sample step) and writes their
//    keys to cand[row][split][m][0..3] (0: fewer than 4).
// ---------------------------------------------------------------------------
template <bool FP8>
__global__ __launch_bounds__(256, 2) void score_sample_kernel(FusedScoreArgs a)
{
    __shared__ bf16_t keys[kFStep][kFKRow];
    __shared__ float tile_scale[kFStep];
    const bf16_t *__restrict__ qrot = (const bf16_t *)a.qrot;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * kFRows;
    const int nrows = (int)min((int64_t)kFRows, (int64_t)a.rows - row0);
    const int split = blockIdx.y;
    const int64_t slen = ((int64_t)a.nsample + a.ssplit - 1) / a.ssplit;
    const int64_t s_lo = split * slen, s_hi = min((int64_t)a.nsample, s_lo + slen);
    bf16x8_t qa[4][4];
    load_query_tile(qrot, row0, nrows, wave, qa);
    const TileRows trow = tile_rows(a, row0, nrows);
    int64_t my_nc[4];
    int32_t my_seq[4];
    float top[4][4];  // per row: the lane's 4 best sampled scores, descending (-1: none)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + g;  // its sequence and bound: lane rw of the tile's rows
        my_nc[mt] = __shfl(trow.nb, rw);
        my_seq[mt] = __shfl(trow.seq, rw);
#pragma unroll
        for (int q = 0; q < 4; ++q) top[mt][q] = -1.0f;
    }
    uint64_t todo = nrows >= 64 ? ~0ull : ((1ull << nrows) - 1ull);
    while (todo) {
        int64_t nb_hi;
        const int32_t seq = next_seq_group(trow, todo, nb_hi);
        const int64_t hi = min(s_hi, (nb_hi + kSampleStride - 1) / kSampleStride);  // samples that can be visible
        // smallest visible bound over the wave's rows of this group
        int64_t lim_min = INT64_MAX;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            if (my_seq[mt] == seq) lim_min = min(lim_min, my_nc[mt]);
        lim_min = min(lim_min, (int64_t)__shfl_xor((long long)lim_min, 16));
        lim_min = min(lim_min, (int64_t)__shfl_xor((long long)lim_min, 32));
        const int lrow = t >> 2, ldim = (t & 3) * 32;
        TileShare<FP8> ts;
        auto fetch = [&](int64_t i0) {
            const int64_t b = min(sample_block(min(i0 + lrow, hi - 1)), nb_hi - 1);
            ts.load(a, seq, b, ldim, page_entry(a.kp, seq, b));
        };
        if (s_lo < hi) fetch(s_lo);
        for (int64_t i0 = s_lo; i0 < hi; i0 += kFStep) {
            ts.store(&keys[lrow][ldim], &tile_scale[lrow], (t & 3) == 0);
            __syncthreads();
            if (i0 + kFStep < hi) fetch(i0 + kFStep);
            float sc[4][4];
            tile_scores(keys, qa, sc);
            apply_scales<FP8>(tile_scale, sc);
            // every sample of the step visible to every row of the wave: no
            // per-sample test (sample i's block is below 32 i + 32)
            const bool all_vis = i0 + kFStep <= hi && (i0 + kFStep) * kSampleStride <= lim_min;
            // insert v into the lane's descending top-4 of row tile mt: the new q-th best of
            // {top[0..q], v} is the median of top[q-1], top[q] and v.  The lists start at -1
            // and scores are >= 0, so inserting -1 (a row of another sequence, a sample past
            // the row's visible blocks) changes nothing: the insertions stay straight-line code.
            auto insert = [&](int mt, float v) {
                float *tp = top[mt];
                const float t0 = tp[0], t1 = tp[1], t2 = tp[2];
                tp[0] = fmaxf(t0, v);
                tp[1] = __builtin_amdgcn_fmed3f(t0, t1, v);
                tp[2] = __builtin_amdgcn_fmed3f(t1, t2, v);
                tp[3] = __builtin_amdgcn_fmed3f(t2, tp[3], v);
            };
            if (all_vis) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) insert(mt, my_seq[mt] == seq ? sc[mt][nt] : -1.0f);
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt) {
                        const int64_t i = i0 + nt * 16 + m;
                        const bool vis = my_seq[mt] == seq && i < hi && sample_block(i) < my_nc[mt];
                        insert(mt, vis ? sc[mt][nt] : -1.0f);
                    }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + g;
        if (rw >= nrows) continue;
        uint4 k;
        k.x = top[mt][0] >= 0.0f ? pos_key(top[mt][0]) : 0u;
        k.y = top[mt][1] >= 0.0f ? pos_key(top[mt][1]) : 0u;
        k.z = top[mt][2] >= 0.0f ? pos_key(top[mt][2]) : 0u;
        k.w = top[mt][3] >= 0.0f ? pos_key(top[mt][3]) : 0u;
        *(uint4 *)(a.cand + (((row0 + rw) * a.ssplit + split) * 16 + m) * 4) = k;
    }
}

// ---------------------------------------------------------------------------
// 2. threshold: one wave per row.  tau[row] = the j-th best key among the
//    row's candidates (at most the j-th best sampled score), or 0 (no
//    threshold) when fewer than j candidates exist.
// ---------------------------------------------------------------------------
template <int kMaxPer>  // ssplit <= kMaxPer: at most kMaxPer candidates per lane
__global__ __launch_bounds__(256) void sample_threshold_kernel(FusedScoreArgs a)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * 4 + w;
    if (r >= a.rows) return;
    const int n = a.ssplit * 64;
    const uint32_t *crow = a.cand + r * n;
    uint32_t v[kMaxPer];
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) v[q] = q * 64 + lane < n ? crow[q * 64 + lane] : 0u;
    uint32_t valid = 0;
#pragma unroll
    for (int q = 0; q < kMaxPer; ++q) valid += (uint32_t)__popcll(__ballot(v[q] != 0u));
    const uint32_t j = (uint32_t)sample_j(a.top_k);
    if (valid < j) {
        if (lane == 0) a.tau[r] = 0u;
        return;
    }
    // the j-th largest key T is the largest t with #{keys >= t} >= j: fixed
    // bit by bit from the top, each count from ballots of the 64 lanes
    uint32_t tkey = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = tkey | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int q = 0; q < kMaxPer; ++q) cnt += (uint32_t)__popcll(__ballot(v[q] >= c));
        if (cnt >= j) tkey = c;
    }
    if (lane == 0) a.tau[r] = tkey;
}

// ---------------------------------------------------------------------------
// 3. filter: grid (row tiles, splits).  Lane (mt, g, m) owns list m of row
//    16*wave + 4*mt + g in this split and appends its pairs >= tau there.
// ---------------------------------------------------------------------------
template <bool FP8, bool INTER>  // INTER: lists_interleaved(a.nsplit)
__global__ __launch_bounds__(256, 2) void score_filter_kernel(FusedScoreArgs a)
{
    __shared__ bf16_t keys[2][kFStep][kFKRow];
    __shared__ float tile_scale[2][kFStep];
    const bf16_t *__restrict__ qrot = (const bf16_t *)a.qrot;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.x * kFRows;
    const int nrows = (int)min((int64_t)kFRows, (int64_t)a.rows - row0);
    const int split = blockIdx.y;
    const int64_t split_lo = (int64_t)split * a.split_len;
    const int64_t split_hi = min((int64_t)a.max_nb, split_lo + a.split_len);
    bf16x8_t qa[4][4];
    load_query_tile(qrot, row0, nrows, wave, qa);
    int64_t my_nc[4];
    int32_t my_seq[4];
    uint2 *my_list[4];
    // the next slot of each list (kept while the lists have room), a global
    // address so its stores stay global stores (a flat store would also count
    // against the LDS waits)
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(1))) u32x2_t global_pair;
    global_pair *my_ptr[4];
    uint32_t my_cnt[4];
    float tauf[4];
    const TileRows trow = tile_rows(a, row0, nrows);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + g;  // its sequence and bound: lane rw of the tile's rows
        const uint32_t okm = rw < nrows ? ~0u : 0u;
        const int rc = min(rw, nrows - 1);
        const uint32_t tk = a.tau[row0 + rc];  // issued unconditionally (clamped), then masked
        my_nc[mt] = __shfl(trow.nb, rw);
        my_seq[mt] = __shfl(trow.seq, rw);
        my_list[mt] = a.buf + ((row0 + rc) * a.nsplit + split) * 16 * (int64_t)a.subcap +
                      (INTER ? m : m * (int64_t)a.subcap);  // pair j at [16 j] or [j]
        my_ptr[mt] = (global_pair *)my_list[mt];
        my_cnt[mt] = 0;
        // an empty row slot gets tau = +inf, so it never appends
        tauf[mt] = __uint_as_float((__float_as_uint(tau_float(tk)) & okm) | (0x7f800000u & ~okm));
    }
    const uint32_t cap_last = (uint32_t)a.subcap - 1u;
    uint64_t todo = nrows >= 64 ? ~0ull : ((1ull << nrows) - 1ull);
    while (todo) {
        int64_t nb_hi;
        const int32_t seq = next_seq_group(trow, todo, nb_hi);
        int64_t lim[4];  // visible bound of the lane's rows in this group (0: not in it)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) lim[mt] = my_seq[mt] == seq ? my_nc[mt] : 0;
        // smallest bound over the wave's 16 rows (an empty row slot has tau = +inf, so it never appends)
        int64_t lim_min = INT64_MAX;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int rw = 16 * wave + 4 * mt + g;
            if (rw < nrows) lim_min = min(lim_min, lim[mt]);
        }
        lim_min = min(lim_min, (int64_t)__shfl_xor((long long)lim_min, 16));
        lim_min = min(lim_min, (int64_t)__shfl_xor((long long)lim_min, 32));
        const int64_t lo = split_lo, hi = min(split_hi, nb_hi);
        if (lo >= hi) continue;
        const int lrow = t >> 2, ldim = (t & 3) * 32;
        TileShare<FP8> ts;  // the next tile's share of this thread
        {
            const int64_t b = min(lo + lrow, hi - 1);
            ts.load(a, seq, b, ldim, page_entry(a.kp, seq, b));
        }
        // paged pools: the table entry of this thread's row of the next tile,
        // read a step ahead of its key
        int32_t pg_next = page_entry(a.kp, seq, min(lo + kFStep + lrow, hi - 1));
        ts.store(&keys[0][lrow][ldim], &tile_scale[0][lrow], (t & 3) == 0);
        __syncthreads();
        int cur = 0;
        for (int64_t base = lo; base < hi; base += kFStep) {
            const bool more = base + kFStep < hi;
            if (more) {
                ts.load(a, seq, min(base + kFStep + lrow, hi - 1), ldim, pg_next);
                pg_next = page_entry(a.kp, seq, min(base + 2 * kFStep + lrow, hi - 1));
            }
            float sc[4][4];
            tile_scores(keys[cur], qa, sc);
            apply_scales<FP8>(tile_scale[cur], sc);
            if (more) ts.store(&keys[cur ^ 1][lrow][ldim], &tile_scale[cur ^ 1][lrow], (t & 3) == 0);
            // a pair >= tau goes to the lane's list; past the list's capacity
            // the last slot is overwritten but the count goes on, so the
            // merge sees the overflow (and recomputes the row)
            // A lane appends at most 4 pairs per list in a step: while every list
            // of the wave has room for 4 more, the appends go to a running slot
            // pointer with no capacity clamp.
            const uint32_t cnt_hi = max(max(my_cnt[0], my_cnt[1]), max(my_cnt[2], my_cnt[3]));
            const bool roomy = __ballot(cnt_hi + 4u > (uint32_t)a.subcap) == 0ull;
            if (roomy && base + kFStep <= lim_min) {  // and every block of the step is visible to every row
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        if (sc[mt][nt] >= tauf[mt]) {
                            *my_ptr[mt] = u32x2_t{pos_key(sc[mt][nt]), (uint32_t)(base + nt * 16 + m)};
                            my_ptr[mt] += INTER ? 16 : 1;
                            ++my_cnt[mt];
                        }
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    // block base + 16*nt + m is visible iff 16*nt < lr
                    const int32_t lr = (int32_t)max(min(lim[mt] - base - m, (int64_t)kFStep), (int64_t)-1);
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        if (sc[mt][nt] >= tauf[mt] && 16 * nt < lr) {
                            my_list[mt][(INTER ? 16 : 1) * min(my_cnt[mt], cap_last)] =
                                make_uint2(pos_key(sc[mt][nt]), (uint32_t)(base + nt * 16 + m));
                            ++my_cnt[mt];
                        }
                    my_ptr[mt] = (global_pair *)(my_list[mt] + (INTER ? 16 : 1) * min(my_cnt[mt], cap_last));
                }
            }
            __syncthreads();
            cur ^= 1;
        }
        __syncthreads();
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + g;
        if (rw < nrows) a.cnt[((row0 + rw) * a.nsplit + split) * 16 + m] = my_cnt[mt];
    }
}

// ---------------------------------------------------------------------------
// 4. merge: one wave per row, four rows per workgroup; no workgroup barriers.
// ---------------------------------------------------------------------------
namespace {

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

// The same for an FP8 key: codes converted exactly, the sum times the scale.
__device__ __forceinline__ float recompute_score_fp8(const bf16_t *__restrict__ q4, const uint8_t *__restrict__ code,
                                                     float scale)
{
    float d[kIdxHeads] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i = 0; i < kDim; i += 8) {
        const uint2 w = *(const uint2 *)(code + i);
        const auto k01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false), k23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
        const auto k45 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false), k67 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
        const float kv[8] = {k01[0], k01[1], k23[0], k23[1], k45[0], k45[1], k67[0], k67[1]};
#pragma unroll
        for (int h = 0; h < kIdxHeads; ++h) {
            float qv[8];
            load8(q4 + h * kDim + i, qv);
#pragma unroll
            for (int e = 0; e < 8; ++e) d[h] = fmaf(qv[e], kv[e], d[h]);
        }
    }
    return (((fmaxf(d[0], 0.0f) + fmaxf(d[1], 0.0f)) + fmaxf(d[2], 0.0f)) + fmaxf(d[3], 0.0f)) * scale;
}

template <bool FP8>
__device__ __forceinline__ float recompute_block(const FusedScoreArgs &a, const bf16_t *q4, int32_t seq, int64_t b)
{
    if (FP8) {
        const int64_t key = key_index(a.kp, a.pooled_stride, seq, b);
        return recompute_score_fp8(q4, a.codes + key * kDim, a.scales[key]);
    }
    return recompute_score(q4, (const bf16_t *)a.pooled + key_offset(a.kp, a.pooled_stride, seq, b));
}

__device__ __forceinline__ float scaled(float raw) { return (float)((double)raw / sqrt((double)kDim)); }

// The merge of one row whose n <= kStage pairs sit in the wave's LDS stage.
// The pairs move to registers (kStage / 64 per lane; an empty slot holds key
// 0, which no pair has: pair keys always carry the top bit).  A radix select
// over the keys finds the kk-th largest key T; when T is shared by more pairs
// than still needed, a second radix select over the blocks of those pairs
// keeps the lowest ones.  The kept blocks are then written in block order:
// marked in a bitmap of the visible range (one 65,536-block window at a time,
// in the stage's LDS), whose per-word prefix counts give each one its slot.
constexpr int kRegPairs = kStage / kWave;
constexpr int kWinWords = 2048;  // bitmap window: 65,536 blocks
// Lane l owns bitmap words [32l, 32l + 32).  Word w is stored at w + 4(w/32)
// and its u16 prefix count at w + 8(w/32): a lane's run is 16-byte aligned,
// so it is cleared, read and its counts written 16 bytes at a time, and the
// runs' strides (144 and 80 bytes) put the 16 lanes of an access on distinct
// LDS bank groups.
__device__ __forceinline__ uint32_t bm_slot(uint32_t w) { return w + 4u * (w >> 5); }
__device__ __forceinline__ uint32_t pre_slot(uint32_t w) { return w + 8u * (w >> 5); }
constexpr int kBmSlots = kWinWords + 4 * (kWinWords / 32);
constexpr int kPreSlots = kWinWords + 8 * (kWinWords / 32);
static_assert(kBmSlots * 4 + kPreSlots * 2 <= kStage * 8, "bitmap + prefix fit the stage");

// The pick step of one radix pass (of `width` <= 8 bits) of a descending
// select in the wave: `h` holds the counts of the digits of the values whose
// higher bits match `prefix`; narrows (prefix, need) to the bin holding the
// need-th largest (prefix restarts on the first pass) and returns that bin's
// count.
__device__ __forceinline__ uint32_t radix_pass_pick(uint32_t *h, uint32_t &need, uint32_t &prefix, bool first,
                                                    int width)
{
    const int lane = threadIdx.x & 63;
    wave_fence();
    uint32_t hv[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        hv[q] = h[255 - 4 * lane - q];
        sum += hv[q];
    }
    const uint32_t incl = wave_incl_scan(sum);
    const int ls = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;
    uint32_t digit = 0, above = 0, cntd = 0;
    {  // every lane computes; lane ls's values are the ones used
        uint32_t acc = incl - sum;
        bool found = false;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool hit = !found && acc + hv[q] >= need;
            digit = hit ? 255u - 4u * (uint32_t)lane - (uint32_t)q : digit;
            above = hit ? acc : above;
            cntd = hit ? hv[q] : cntd;
            found = found || hit;
            acc += hv[q];
        }
    }
    digit = lane_value(digit, ls);
    above = lane_value(above, ls);
    cntd = lane_value(cntd, ls);
    need -= above;
    prefix = first ? digit : (prefix << width) | digit;
    wave_fence();
    return cntd;
}

template <int P>  // pair slots per lane: n <= 64 P
__device__ __forceinline__ void merge_staged_p(uint2 *st, uint32_t *h, uint32_t n, int32_t nc, int32_t kk,
                                               int32_t *__restrict__ out, float *__restrict__ osc)
{
    const int lane = threadIdx.x & 63;
    uint32_t key[P], nblk[P];  // key and ~block; an empty slot is (0, 0)
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const uint32_t idx = (uint32_t)(i * kWave + lane);
        const uint2 e = idx < n ? st[idx] : make_uint2(0u, 0xffffffffu);
        key[i] = e.x;
        nblk[i] = ~e.y;
    }
    // ---- kk-th largest key.  Bits that every pair shares are skipped (the
    // first pass starts below them, so its digits spread over the bins); a
    // pass counts the next digit of every key whose resolved top bits match,
    // and a non-matching key (or an empty slot) counts in the lane's spare
    // slot.  (key >> sh) > tp is kept, == tp is the current bin. ----
    uint32_t need = (uint32_t)kk, tp = 0, cnt = 0;
    int sh = 32;
    if ((uint32_t)kk < n) {
        const uint32_t k0 = lane_value(key[0], 0);  // the first staged pair
        uint32_t x = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) x |= key[i] != 0u ? key[i] ^ k0 : 0u;
        x = wave_or(x);
        sh = x ? 32 - __clz(x) : 0;  // pair keys share bit 31, so sh <= 31
        tp = k0 >> sh;
        cnt = n;
        while (sh > 0 && cnt != need) {
            const int nsh = max(sh - 8, 0), width = sh - nsh;
            const uint32_t himask = 0xffffffffu << sh, hv = tp << sh;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[4 * lane + q] = 0u;
            wave_fence();
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const bool m = (key[i] & himask) == hv;
                atomicAdd(&h[m ? (key[i] >> nsh) & ((1u << width) - 1u) : 256u + (uint32_t)lane], 1u);
            }
            cnt = radix_pass_pick(h, need, tp, false, width);
            sh = nsh;
        }
    }
    // ---- ties at T cut: keep the `need` lowest blocks among key == T, the
    // largest values of ~block ----
    const bool cut = sh == 0 && cnt != need;
    uint32_t bp = 0;
    int bsh = 32;
    if (cut) {
        for (; bsh > 0;) {
            const int nsh = bsh - 8;
            const uint32_t himask = bsh == 32 ? 0u : 0xffffffffu << bsh;
            const uint32_t hv = bsh == 32 ? 0u : bp << bsh;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[4 * lane + q] = 0u;
            wave_fence();
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const bool m = (key[i] == tp) & ((nblk[i] & himask) == hv);
                atomicAdd(&h[m ? (nblk[i] >> nsh) & 0xffu : 256u + (uint32_t)lane], 1u);
            }
            cnt = radix_pass_pick(h, need, bp, bsh == 32, 8);
            bsh = nsh;
            if (cnt == need) break;
        }
    }
    // kept <=> (key << 32 | ~block) >= C: every composite above the resolved
    // bin, and all of the final bin (kept whole, or cut by the block passes)
    uint64_t C;
    if (sh == 32) C = 1ull;  // keep every pair (empty slots are 0)
    else if (!cut) C = (uint64_t)(tp << sh) << 32;
    else C = ((uint64_t)tp << 32) | (uint64_t)(bsh == 32 ? 0u : bp << bsh);
    // ---- emission through the bitmap, window by window ----
    uint32_t *bm = (uint32_t *)st;
    uint16_t *pre = (uint16_t *)(bm + kBmSlots);
    uint32_t base = 0;
    for (int32_t w0 = 0; w0 < nc; w0 += 32 * kWinWords) {
        const int nwords = min(kWinWords, (nc - w0 + 31) / 32);
        const uint32_t wbits = 32u * (uint32_t)nwords;
        // the lane's run of 32 words (the padding words are never read)
#pragma unroll
        for (int j = 0; j < kWinWords / kWave / 4; ++j)
            ((uint4 *)(bm + bm_slot((uint32_t)lane * (kWinWords / kWave))))[j] = make_uint4(0u, 0u, 0u, 0u);
        wave_fence();
#pragma unroll
        for (int i = 0; i < P; ++i) {  // a pair not kept ORs 0 into its lane's word
            const uint32_t b = ~nblk[i] - (uint32_t)w0;
            const bool k = ((((uint64_t)key[i] << 32) | nblk[i]) >= C) & (b < wbits);
            atomicOr(&bm[k ? bm_slot(b >> 5) : (uint32_t)lane], k ? 1u << (b & 31u) : 0u);
        }
        wave_fence();
        // the lane's words, read once (all reads in flight together), and the
        // exclusive prefix count of its run in word order
        constexpr int kPer = kWinWords / kWave;
        uint32_t words[kPer], c = 0;
#pragma unroll
        for (int j = 0; j < kPer / 4; ++j) {
            const uint4 x = ((const uint4 *)(bm + bm_slot((uint32_t)(lane * kPer))))[j];
            words[4 * j] = x.x;
            words[4 * j + 1] = x.y;
            words[4 * j + 2] = x.z;
            words[4 * j + 3] = x.w;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) c += (uint32_t)__popc(words[j]);
        const uint32_t incl = wave_incl_scan(c);
        // each kept pair finds its slot from its word's prefix count and the
        // bits below it (kept blocks cluster, so walking each lane's set bits
        // would serialise on the lanes that hold the clusters)
        uint32_t run = incl - c;
#pragma unroll
        for (int j = 0; j < kPer / 8; ++j) {  // 8 counts per 16-byte write
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = run;
                run += (uint32_t)__popc(words[8 * j + 2 * e]);
                h[e] = lo | (run << 16);
                run += (uint32_t)__popc(words[8 * j + 2 * e + 1]);
            }
            ((uint4 *)(pre + pre_slot((uint32_t)(lane * kPer))))[j] = make_uint4(h[0], h[1], h[2], h[3]);
        }
        wave_fence();
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t b = ~nblk[i] - (uint32_t)w0;
            const bool k = ((((uint64_t)key[i] << 32) | nblk[i]) >= C) & (b < wbits);
            const uint32_t wd = k ? b >> 5 : 0u;
            const uint32_t pos =
                base + (uint32_t)pre[pre_slot(wd)] + (uint32_t)__popc(bm[bm_slot(wd)] & ((1u << (b & 31u)) - 1u));
            if (k && pos < (uint32_t)kk) {
                out[pos] = (int32_t)(w0 + b);
                if (osc) osc[pos] = scaled(key_score(key[i]));
            }
        }
        base += lane_value(incl, kWave - 1);
        if (w0 + 32 * kWinWords < nc) wave_fence();  // the next window reuses the bitmap
    }
}

// The passes run over as few register slots per lane as the row's pairs
// need: 8, 16, 24 or 32 (at a threshold of the ~40th sampled score most rows
// of a long context fit 24; rows with few visible blocks fit fewer).
__device__ __forceinline__ void merge_staged(uint2 *st, uint32_t *h, uint32_t n, int32_t nc, int32_t kk,
                                             int32_t *__restrict__ out, float *__restrict__ osc)
{
    if (n <= 8u * kWave)
        merge_staged_p<8>(st, h, n, nc, kk, out, osc);
    else if (n <= 16u * kWave)
        merge_staged_p<16>(st, h, n, nc, kk, out, osc);
    else if (n <= 24u * kWave)
        merge_staged_p<24>(st, h, n, nc, kk, out, osc);
    else
        merge_staged_p<kRegPairs>(st, h, n, nc, kk, out, osc);
}

// Every pair of a row's lists, read lane-parallel: lane i walks list i of
// each group of 64 lists with 16-byte loads (two pairs each, eight in
// flight); fn(pair, valid) sees 16 pair slots per lane and step, in the same
// order on every lane, so it may use wave-wide ballots.
template <typename F>
__device__ __forceinline__ void for_each_listed(const uint2 *__restrict__ lists, const uint32_t *__restrict__ cnt,
                                                int nlists, int32_t subcap, bool inter, F &&fn)
{
    const int lane = threadIdx.x & 63;
    for (int i0 = 0; i0 < nlists; i0 += kWave) {
        const int li = i0 + lane;
        const uint32_t c = li < nlists ? cnt[li] : 0u;
        uint32_t cmax = c;
        for (int o = 1; o < 64; o <<= 1) cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, o));
        const uint2 *src = lists + list_slot(min(li, nlists - 1), 0u, subcap, inter);
        // a load past the list's last pair re-reads that one (every load stays in
        // the list, none needs a guard, so all of a round are issued together)
        if (inter) {  // pair j at [16 j]
            const uint32_t last = c > 0u ? c - 1u : 0u;
            for (uint32_t j = 0; j < cmax; j += 16) {
                uint2 e[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) e[q] = src[16 * min(j + (uint32_t)q, last)];
#pragma unroll
                for (int q = 0; q < 16; ++q) fn(e[q], j + q < c);
            }
        } else {  // pair j at [j]: 16-byte loads of two pairs
            const uint32_t qlast = c > 0u ? (c - 1u) >> 1 : 0u;
            for (uint32_t j = 0; j < cmax; j += 16) {
                uint4 e[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = ((const uint4 *)src)[min((j >> 1) + (uint32_t)q, qlast)];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    fn(make_uint2(e[q].x, e[q].y), j + 2 * q < c);
                    fn(make_uint2(e[q].z, e[q].w), j + 2 * q + 1 < c);
                }
            }
        }
    }
}

// Histogram of a pair key's bits [30:19]: the float exponent and the top 4
// mantissa bits of the score (every pair key carries bit 31), 1/16 octave per
// bin; the table fills the wave's stage exactly.
constexpr int kPreShift = 19;
constexpr uint32_t kPreBins = 4096;
static_assert(kPreBins * 4 == kStage * 8, "the prefilter histogram fills the stage");

}  // namespace

template <bool FP8>
__global__ __launch_bounds__(256, 2) void select_merge_kernel(FusedScoreArgs a, int32_t *__restrict__ sel_blocks,
                                                         int32_t *__restrict__ sel_count, float *__restrict__ sel_scores)
{
    __shared__ __align__(16) uint2 stage[kMergeWaves][kStage];
    __shared__ uint32_t hb[kMergeWaves][256 + kWave];  // 256 bins + a spare slot per lane
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * kMergeWaves + w;
    if (r >= a.rows) return;
    const uint64_t lt = (1ull << lane) - 1ull;  // lanes below this one
    const int32_t nc = (int32_t)min(visible_blocks(a.row_pos[r]), (int64_t)a.max_nb);
    const int32_t kk = max(0, min(a.top_k, nc));
    int32_t *out = sel_blocks + r * a.top_k;
    float *osc = sel_scores ? sel_scores + r * a.top_k : nullptr;
    if (lane == 0) {
        sel_count[r] = kk;
        a.mode[r] = kMergeNone;
    }
    for (int32_t i = kk + lane; i < a.top_k; i += kWave) {
        out[i] = -1;
        if (osc) osc[i] = 0.0f;
    }
    if (nc <= 0) return;  // no visible block (the GEMMs may not have run at all)
    uint2 *st = stage[w];
    uint32_t *h = hb[w];
    // ---- the row's pairs (list i of 16 * nsplit) ----
    const int nlists = a.nsplit * 16;
    uint32_t total = 0;
    bool overflow = false;
    for (int i0 = 0; i0 < nlists; i0 += kWave) {
        const uint32_t c = i0 + lane < nlists ? a.cnt[r * nlists + i0 + lane] : 0u;
        overflow |= __ballot(c > (uint32_t)a.subcap) != 0ull;
        uint32_t s = c;
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        total += s;
    }
    // exact only if at least kk pairs reached tau (and none was dropped); a
    // kept set too large to sort in LDS is ranked and emitted in block order
    // from recomputed scores
    int mode = (overflow || total < (uint32_t)kk || kk > kStage) ? 2 : (total <= (uint32_t)kStage ? 0 : 1);
    if (lane == 0) a.mode[r] = mode == 0 ? kMergeStaged : mode == 1 ? kMergeListWalk : kMergeRecompute;
    const uint2 *lists = a.buf + (int64_t)r * nlists * a.subcap;
    const bool inter = lists_interleaved(a.nsplit);
    uint32_t n = 0;
    if (mode == 0) {  // stage the pairs in LDS: 64 lists at a time, lane i copies list i
        for (int i0 = 0; i0 < nlists; i0 += kWave) {
            const int li = i0 + lane;
            const uint32_t c = li < nlists ? a.cnt[r * nlists + li] : 0u;
            uint32_t off = c, cmax = c;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(off, o);
                if (lane >= o) off += y;
                cmax = max(cmax, __shfl_xor(cmax, o));
            }
            const uint32_t chunk = __shfl(off, 63);
            off = n + off - c;
            const uint2 *src = lists + list_slot(min(li, nlists - 1), 0u, a.subcap, inter);
            if (inter) {
                // pair j at [16 j]: 16 pairs in flight per lane; the lanes of a split read
                // the same slot of their 16 lists, one 128-byte line; a load past the
                // list's last pair re-reads that one
                const uint32_t last = c > 0u ? c - 1u : 0u;
                for (uint32_t j = 0; j < cmax; j += 16) {
                    uint2 e[16];
#pragma unroll
                    for (int q = 0; q < 16; ++q) e[q] = src[16 * min(j + (uint32_t)q, last)];
#pragma unroll
                    for (int q = 0; q < 16; ++q)
                        if (j + q < c) st[off + j + q] = e[q];
                }
            } else {
                // pair j at [j]: 16-byte loads, two pairs each, 8 in flight per lane
                // (a list's capacity is a multiple of 8 pairs, so a load never leaves it)
                for (uint32_t j = 0; j < cmax; j += 16) {
                    uint4 e[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        e[q] = j + 2 * q < c ? ((const uint4 *)src)[(j >> 1) + q] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        if (j + 2 * q < c) st[off + j + 2 * q] = make_uint2(e[q].x, e[q].y);
                        if (j + 2 * q + 1 < c) st[off + j + 2 * q + 1] = make_uint2(e[q].z, e[q].w);
                    }
                }
            }
            n += chunk;
        }
    } else if (mode == 1) {
        n = total;
        // More pairs than the stage holds.  The histogram locates the bin of
        // the kk-th largest key; only the pairs in or above that bin are
        // staged.  They hold every pair the full ranking keeps (all keys above
        // the kk-th and all keys equal to it), so merging them is exact.  A
        // bin too crowded to stage falls through to the list-walking path.
        uint32_t *hist = (uint32_t *)st;
        for (uint32_t i = (uint32_t)lane; i < kPreBins; i += kWave) hist[i] = 0u;
        wave_fence();
        const uint32_t *lcnt = a.cnt + r * nlists;
        for_each_listed(lists, lcnt, nlists, a.subcap, inter, [&](uint2 e, bool v) {
            if (v) atomicAdd(&hist[(e.x >> kPreShift) & (kPreBins - 1u)], 1u);
        });
        wave_fence();
        // lane l sums bins [4032 - 64l, 4095 - 64l]: lanes in order walk the
        // bins from the top
        uint32_t sum = 0;
        {
            const uint4 *hv = (const uint4 *)(hist + kPreBins - 64u * (uint32_t)(lane + 1));
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const uint4 x = hv[q];
                sum += (x.x + x.y) + (x.z + x.w);
            }
        }
        const uint32_t incl = wave_incl_scan(sum);
        const int ls = __ffsll((unsigned long long)__ballot(incl >= (uint32_t)kk)) - 1;  // total >= kk
        const uint32_t above_ls = lane_value(incl - sum, ls);
        // within lane ls's 64 bins: lane j takes bin 4095 - 64 ls - j
        const uint32_t bj = kPreBins - 1u - 64u * (uint32_t)ls - (uint32_t)lane;
        const uint32_t incl2 = above_ls + wave_incl_scan(hist[bj]);
        const int lj = __ffsll((unsigned long long)__ballot(incl2 >= (uint32_t)kk)) - 1;
        const uint32_t bin = lane_value(bj, lj), staged = lane_value(incl2, lj);
        wave_fence();  // the histogram is read out before the stage reuses it
        if (staged <= (uint32_t)kStage) {
            const uint32_t kmin = 0x80000000u | (bin << kPreShift);
            uint32_t nst = 0;
            for_each_listed(lists, lcnt, nlists, a.subcap, inter, [&](uint2 e, bool v) {
                const bool take = v && e.x >= kmin;
                const uint64_t tb = __ballot(take);
                if (take) st[nst + (uint32_t)__popcll(tb & lt)] = e;
                nst += (uint32_t)__popcll(tb);
            });
            if (lane == 0) a.mode[r] = kMergePrefilter;
            mode = 0;  // ranked from the stage like a staged row
            n = nst;
        }
    } else {
        n = (uint32_t)nc;
    }
    wave_fence();
    if (mode == 0) {
        merge_staged(st, h, n, nc, kk, out, osc);
        return;
    }
    const int32_t seq = a.row_seq[r];
    const bf16_t *q4 = (const bf16_t *)a.qrot + r * kIdxHeads * kDim;
    // visit every candidate, 64 at a time: fn(pair, valid).  Staged and listed
    // pairs come in no particular order; recomputed ones in block order.
    auto visit = [&](auto &&fn) {
        if (mode == 0) {
            for (uint32_t i0 = 0; i0 < n; i0 += kWave) {
                const uint32_t i = i0 + lane;
                fn(i < n ? st[i] : make_uint2(0u, 0u), i < n);
            }
        } else if (mode == 1) {
            for (int li = 0; li < nlists; ++li) {
                const uint32_t c = a.cnt[r * nlists + li];
                for (uint32_t i0 = 0; i0 < c; i0 += kWave) {
                    const uint32_t i = i0 + lane;
                    fn(i < c ? lists[list_slot(li, i, a.subcap, inter)] : make_uint2(0u, 0u), i < c);
                }
            }
        } else {
            for (int32_t b0 = 0; b0 < nc; b0 += kWave) {
                const int32_t b = b0 + lane;
                const bool v = b < nc;
                fn(make_uint2(v ? pos_key(recompute_block<FP8>(a, q4, seq, b)) : 0u, (uint32_t)b), v);
            }
        }
    };
    // ---- radix select of the kk-th largest key T, 8 bits at a time: keys
    // whose top bits beat `prefix` are kept, and of those equal to it the
    // `need` lowest blocks ----
    uint32_t need = (uint32_t)kk, prefix = 0;
    int sh = 32;  // key >> sh is compared with prefix (32: every key is kept)
    auto select_t = [&]() {
        need = (uint32_t)kk;
        prefix = 0;
        sh = 32;
        if ((uint32_t)kk >= n) return;
        for (int pass = 0; pass < 4; ++pass) {
            const int nsh = sh - 8;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[4 * lane + q] = 0u;
            wave_fence();
            visit([&](uint2 e, bool v) {
                if (v && (sh == 32 || (e.x >> sh) == prefix)) atomicAdd(&h[(e.x >> nsh) & 0xffu], 1u);
            });
            wave_fence();
            uint32_t hv[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                hv[q] = h[255 - 4 * lane - q];
                sum += hv[q];
            }
            uint32_t incl = sum;
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const int ls = __ffsll((unsigned long long)__ballot(incl >= need)) - 1;
            uint32_t digit = 0, above = 0, cntd = 0;
            if (lane == ls) {
                uint32_t acc = incl - sum;
                for (int q = 0; q < 4; ++q) {
                    if (acc + hv[q] >= need) {
                        digit = 255u - 4u * (uint32_t)lane - (uint32_t)q;
                        above = acc;
                        cntd = hv[q];
                        break;
                    }
                    acc += hv[q];
                }
            }
            digit = __shfl(digit, ls);
            above = __shfl(above, ls);
            cntd = __shfl(cntd, ls);
            need -= above;
            prefix = (sh == 32 ? 0u : (prefix << 8)) | digit;
            sh = nsh;
            wave_fence();
            if (cntd == need) break;  // the whole bin is kept
        }
    };
    select_t();
    auto above_t = [&](uint32_t key) { return sh == 32 || (key >> sh) > prefix; };
    auto at_t = [&](uint32_t key) { return sh != 32 && (key >> sh) == prefix; };
    // ---- gather the keys >= T as (block << 32 | key), sort them by block ----
    uint32_t g = 0;
    if (mode != 2) {
        visit([&](uint2 e, bool v) { g += (uint32_t)__popcll(__ballot(v && (above_t(e.x) || at_t(e.x)))); });
        if (g > (uint32_t)kStage) {  // too many exact ties to sort: rank recomputed scores instead
            mode = 2;
            if (lane == 0) a.mode[r] = kMergeRecompute;
            n = (uint32_t)nc;
            select_t();
        }
    }
    if (mode == 2) {  // recomputed pairs come in block order: emit directly
        uint32_t eq_before = 0, out_before = 0;
        visit([&](uint2 e, bool v) {
            const bool gt = v && above_t(e.x), eq = v && at_t(e.x);
            const uint64_t eb = __ballot(eq);
            const bool take = gt || (eq && eq_before + (uint32_t)__popcll(eb & lt) < need);
            const uint64_t tb = __ballot(take);
            const uint32_t pos = out_before + (uint32_t)__popcll(tb & lt);
            if (take && pos < (uint32_t)kk) {
                out[pos] = (int32_t)e.y;
                if (osc) osc[pos] = scaled(key_score(e.x));
            }
            eq_before += (uint32_t)__popcll(eb);
            out_before += (uint32_t)__popcll(tb);
        });
        return;
    }
    // in place for staged pairs: each write lands at or below its read
    uint32_t filled = 0;
    visit([&](uint2 e, bool v) {
        const bool take = v && (above_t(e.x) || at_t(e.x));
        const uint64_t tb = __ballot(take);
        const uint32_t pos = filled + (uint32_t)__popcll(tb & lt);
        wave_fence();
        if (take) *(uint64_t *)&st[pos] = ((uint64_t)e.y << 32) | e.x;
        wave_fence();
        filled += (uint32_t)__popcll(tb);
    });
    uint64_t *kept = (uint64_t *)st;
    uint32_t n2 = 1;
    while (n2 < g) n2 <<= 1;
    for (uint32_t i = g + lane; i < n2; i += kWave) kept[i] = ~0ull;
    wave_fence();
    for (uint32_t size = 2; size <= n2; size <<= 1) {  // bitonic sort by block id
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t i = lane; i < n2 / 2; i += kWave) {
                const uint32_t lo = 2 * i - (i & (stride - 1));
                const uint32_t hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint64_t x = kept[lo], y = kept[hi];
                if ((x > y) == up) {
                    kept[lo] = y;
                    kept[hi] = x;
                }
            }
            wave_fence();
        }
    }
    // emit in block order: keys above T, and the first `need` equal to T
    uint32_t eq_before = 0, out_before = 0;
    for (uint32_t i0 = 0; i0 < g; i0 += kWave) {
        const uint32_t i = i0 + lane;
        const bool v = i < g;
        const uint64_t e = v ? kept[i] : 0ull;
        const uint32_t key = (uint32_t)e;
        const bool gt = v && above_t(key), eq = v && at_t(key);
        const uint64_t eb = __ballot(eq);
        const bool take = gt || (eq && eq_before + (uint32_t)__popcll(eb & lt) < need);
        const uint64_t tb = __ballot(take);
        const uint32_t pos = out_before + (uint32_t)__popcll(tb & lt);
        if (take && pos < (uint32_t)kk) {
            out[pos] = (int32_t)(e >> 32);
            if (osc) osc[pos] = scaled(key_score(key));
        }
        eq_before += (uint32_t)__popcll(eb);
        out_before += (uint32_t)__popcll(tb);
    }
}

// Split of the main pass's block range: enough workgroups to fill the chip.
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

// A lane list holds its expected share of ~3k pairs with a wide margin, and
// every visible block of a row without a threshold (fewer than j samples,
// i.e. fewer than about 32*j visible blocks).
int32_t fused_score_subcap(int32_t top_k, int32_t nsplit)
{
    const int32_t j = sample_j(top_k);
    const int32_t no_tau = (j + 1) * kSampleStride / 16 + 8;
    const int32_t share = (int32_t)(((int64_t)6 * top_k + 16 * nsplit - 1) / (16 * nsplit));
    return (max(no_tau, share) + 7) / 8 * 8;
}

int32_t fused_score_nsample(int32_t max_nb) { return (max_nb + kSampleStride - 1) / kSampleStride; }

// Sample-range splits: enough sampling workgroups to fill the chip, at most 8
// (the threshold kernel holds 8 candidates per lane), at least 64 samples each.
int32_t fused_score_ssplit(int32_t rows, int32_t nsample)
{
    const int64_t tiles = ((int64_t)rows + kFRows - 1) / kFRows;
    int64_t s = (512 + tiles - 1) / tiles;
    s = min(s, (int64_t)8);
    s = min(s, ((int64_t)nsample + kFStep - 1) / kFStep);
    return (int32_t)max((int64_t)1, s);
}

void launch_score_fused(const FusedScoreArgs &a, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                        hipStream_t stream)
{
    const bool fp8 = a.codes != nullptr;
    if (a.max_nb > 0) {
        const unsigned tiles = (unsigned)((a.rows + kFRows - 1) / kFRows);
        if (fp8)
            QSA_LAUNCH("score_sample_fp8", score_sample_kernel<true>, dim3(tiles, (unsigned)a.ssplit), dim3(256), 0,
                       stream, a);
        else
            QSA_LAUNCH("score_sample", score_sample_kernel<false>, dim3(tiles, (unsigned)a.ssplit), dim3(256), 0,
                       stream, a);
        if (a.ssplit <= 4)
            QSA_LAUNCH("sample_threshold", sample_threshold_kernel<4>, dim3((unsigned)((a.rows + 3) / 4)), dim3(256),
                       0, stream, a);
        else
            QSA_LAUNCH("sample_threshold", sample_threshold_kernel<8>, dim3((unsigned)((a.rows + 3) / 4)), dim3(256),
                       0, stream, a);
        const bool inter = lists_interleaved(a.nsplit);
        if (fp8 && inter)
            QSA_LAUNCH("score_filter_fp8", (score_filter_kernel<true, true>), dim3(tiles, (unsigned)a.nsplit),
                       dim3(256), 0, stream, a);
        else if (fp8)
            QSA_LAUNCH("score_filter_fp8", (score_filter_kernel<true, false>), dim3(tiles, (unsigned)a.nsplit),
                       dim3(256), 0, stream, a);
        else if (inter)
            QSA_LAUNCH("score_filter", (score_filter_kernel<false, true>), dim3(tiles, (unsigned)a.nsplit),
                       dim3(256), 0, stream, a);
        else
            QSA_LAUNCH("score_filter", (score_filter_kernel<false, false>), dim3(tiles, (unsigned)a.nsplit),
                       dim3(256), 0, stream, a);
    }
    const dim3 mgrid((unsigned)((a.rows + kMergeWaves - 1) / kMergeWaves)), mblock(kMergeWaves * kWave);
    if (fp8)
        QSA_LAUNCH("select_merge", select_merge_kernel<true>, mgrid, mblock, 0, stream, a, sel_blocks, sel_count,
                   sel_scores);
    else
        QSA_LAUNCH("select_merge", select_merge_kernel<false>, mgrid, mblock, 0, stream, a, sel_blocks, sel_count,
                   sel_scores);
}

}  // namespace qsa
