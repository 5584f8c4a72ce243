// score.hip -- step a5: block scores raw(t,b), materialized as fp32.
//
// "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
// Attention", score equation: s_{t,b} = 1/sqrt(128) * sum over the 4 index
// heads of ReLU(<q_{t,h}, kbar_b>), over the blocks visible to t.  The kernels
// store the un-scaled sum raw(t,b); the selection ranks raw (the scale is a
// positive constant) and only reported scores are scaled.
//
// bf16 uses the gfx950 MFMA v_mfma_f32_16x16x32_bf16.  Lane l of a wave
// supplies A[m = l%16][8 k-slots] and B[8 k-slots][n = l%16] and receives
// C[4*(l/16) + j][l%16], j = 0..3.  A and B take the same 8 k-slots for one
// lane group l/16, so any one-to-one assignment of head dims to (group, slot)
// pairs gives the same dot product: in the bf16 decode scorer lane group g
// supplies the dims 8g + 32s .. +7 at MFMA step s (s = 0..3), so the four
// groups of a key column read one contiguous 64-byte run per step.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kChunk = 2048;  // blocks per workgroup in the row-split kernels
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float relu_sum4(f32x4_t a)
{
    return ((relu(a[0]) + relu(a[1])) + relu(a[2])) + relu(a[3]);
}

// Per-row histogram of the score keys' top 12 bits: counted in LDS, then
// added to the row's global histogram (only the non-empty bins).
// Paged pools: the table entries of a lane's 4 keys of a step (block
// min(base + 4m + nt, b_end - 1)), read one step ahead of the keys, so a key
// load never waits for its table entry.  Contiguous keys read no table.
struct PageAhead {
    int32_t pg[4];
};
__device__ __forceinline__ void page_ahead(const KeyPages &kp, int64_t seq, int64_t base, int m, int64_t b_end,
                                           PageAhead &p)
{
    if (!kp.table) return;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) p.pg[nt] = page_entry(kp, seq, min(base + 4 * m + nt, b_end - 1));
}

__device__ __forceinline__ void hist_clear(uint32_t *lhist)
{
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lhist[i] = 0u;
    __syncthreads();
}
__device__ __forceinline__ void hist_flush(const uint32_t *lhist, uint32_t *ghist)
{
    __syncthreads();
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) {
        const uint32_t c = lhist[i];
        if (c) atomicAdd(&ghist[i], c);
    }
}

// ---------------------------------------------------------------------------
// Few rows, many blocks (decode): grid (chunks of 2048 blocks, rows).  The 4
// index heads sit in MFMA rows 0..3 (rows 4..15 are zero), 16 blocks per MFMA
// column tile.  HBM-bound: each block's 256 bytes are read once per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_rows_bf16_kernel(
    const bf16_t *__restrict__ qrot, const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos,
    const bf16_t *__restrict__ pooled, int64_t pooled_stride, KeyPages kp, int32_t max_nb, float *__restrict__ scores,
    int64_t sc_stride, uint32_t *__restrict__ hist)
{
    __shared__ uint32_t lhist[kHistBins];
    const int r = blockIdx.y;
    const int64_t nc = min(visible_blocks(row_pos[r]), (int64_t)max_nb);
    const int64_t b_begin = (int64_t)blockIdx.x * kChunk;
    if (b_begin >= nc) return;
    const int64_t b_end = min(nc, b_begin + (int64_t)kChunk);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the step loop branches on scalars
    const int m = lane & 15, g = lane >> 4;
    const int64_t seq = row_seq[r];
    float *srow = scores + (int64_t)r * sc_stride;
    // Each wave handles 64 consecutive blocks per step: MFMA column m of tile
    // nt is block base + 4m + nt, so lane m of group 0 ends the step with the
    // scores of 4 consecutive blocks and stores them at once.  Two register
    // buffers take turns: the next step's keys are in flight during this
    // step's MFMAs.  Every load is issued unconditionally (addresses are
    // clamped to the last visible block), so the wait before each MFMA counts
    // only the loads it needs and never drains the prefetch.
    auto load = [&](int64_t base, const PageAhead &p, uint4 (&v)[4][4]) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int64_t b = min(base + 4 * m + nt, b_end - 1);  // clamp: stays inside the visible range
            const int64_t off = kp.table ? key_at(kp, 0, seq, b, p.pg[nt]) * kDim : seq * pooled_stride + b * kDim;
            // lane group g takes head dims 8g + 32s .. +7 at step s: the four
            // groups read one 64-byte run of the key per step; the keys are read
            // once per call, so the loads are non-temporal
            const uint4 *src = (const uint4 *)(pooled + off + 8 * g);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4_t x = __builtin_nontemporal_load((const u32x4_t *)(src + 4 * s));
                v[nt][s] = make_uint4(x.x, x.y, x.z, x.w);
            }
        }
    };
    uint4 v0[4][4], v1[4][4];
    PageAhead p0{}, p1{};  // table entries of the next v0 / v1 loads
    int64_t base = b_begin + wave * 64;
    page_ahead(kp, seq, base, m, b_end, p0);
    load(base, p0, v0);
    page_ahead(kp, seq, base + 256, m, b_end, p1);
    page_ahead(kp, seq, base + 512, m, b_end, p0);
    if (hist) hist_clear(lhist);
    bf16x8_t a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a[s] = m < kIdxHeads
                   ? as_bf16x8(*(const uint4 *)(qrot + ((int64_t)r * kIdxHeads + m) * kDim + 8 * g + 32 * s))
                   : zero_bf16x8();
    auto score = [&](int64_t base, const uint4 (&v)[4][4]) {
        float sc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], as_bf16x8(v[nt][s]), acc, 0, 0, 0);
            sc[nt] = relu_sum4(acc);
        }
        const int64_t b = base + 4 * m;
        if (g == 0 && b < b_end) {
            if (b + 3 < b_end) {
                *(float4 *)(srow + b) = make_float4(sc[0], sc[1], sc[2], sc[3]);
            } else {
                for (int j = 0; j < (int)(b_end - b); ++j) srow[b + j] = sc[j];
            }
            if (hist) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (b + j < b_end) atomicAdd(&lhist[score_key(sc[j]) >> kHistShift], 1u);
            }
        }
    };
    // Two steps per trip and one exit test keep the loop a single uniform
    // block; a second step past the end only re-reads the clamped last block
    // and stores nothing.
    for (; base < b_end; base += 512) {
        load(base + 256, p1, v1);
        page_ahead(kp, seq, base + 768, m, b_end, p1);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the MFMAs
        score(base, v0);
        load(base + 512, p0, v0);
        page_ahead(kp, seq, base + 1024, m, b_end, p0);
        __builtin_amdgcn_sched_barrier(0);
        score(base + 256, v1);
    }
    if (hist) hist_flush(lhist, hist + (int64_t)r * kRowScratch);
}

// ---------------------------------------------------------------------------
// The same on FP8 keys: a block is 128 E4M3 codes (128 bytes) and one FP32
// scale.  A lane converts its 32 codes of a tile to bf16 (exact) for the MFMA,
// and the ReLU-sum of a block is multiplied by the block's scale (a
// non-negative factor commutes with the ReLUs).  Half the bytes of the bf16
// keys, read once per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_rows_fp8_kernel(
    const bf16_t *__restrict__ qrot, const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos,
    const uint8_t *__restrict__ codes, const float *__restrict__ scales, int64_t pooled_stride, KeyPages kp,
    int32_t max_nb, float *__restrict__ scores, int64_t sc_stride, uint32_t *__restrict__ hist)
{
    __shared__ uint32_t lhist[kHistBins];
    const int r = blockIdx.y;
    const int64_t nc = min(visible_blocks(row_pos[r]), (int64_t)max_nb);
    const int64_t b_begin = (int64_t)blockIdx.x * kChunk;
    if (b_begin >= nc) return;
    const int64_t b_end = min(nc, b_begin + (int64_t)kChunk);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, g = lane >> 4;
    const int64_t seq = row_seq[r];
    float *srow = scores + (int64_t)r * sc_stride;
    // as the bf16 kernel: column m of tile nt is block base + 4m + nt; lane
    // group g holds the codes of dims 32g .. 32g + 31 (32 bytes), and every
    // lane also loads the scales of its 4 blocks (clamped, unconditional)
    struct Step {
        uint4 c[4][2];
        float sc[4];
    };
    auto load = [&](int64_t base, const PageAhead &p, Step &v) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int64_t key = key_at(kp, pooled_stride, seq, min(base + 4 * m + nt, b_end - 1), p.pg[nt]);
            const uint4 *src = (const uint4 *)(codes + key * kDim + 32 * g);
            v.c[nt][0] = src[0];
            v.c[nt][1] = src[1];
            v.sc[nt] = scales[key];
        }
    };
    Step v0, v1;
    PageAhead p0{}, p1{};  // table entries of the next v0 / v1 loads
    int64_t base = b_begin + wave * 64;
    page_ahead(kp, seq, base, m, b_end, p0);
    load(base, p0, v0);
    page_ahead(kp, seq, base + 256, m, b_end, p1);
    page_ahead(kp, seq, base + 512, m, b_end, p0);
    if (hist) hist_clear(lhist);
    bf16x8_t a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
        a[s] = m < kIdxHeads
                   ? as_bf16x8(*(const uint4 *)(qrot + ((int64_t)r * kIdxHeads + m) * kDim + 32 * g + 8 * s))
                   : zero_bf16x8();
    auto score = [&](int64_t base, const Step &v) {
        float sc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const bf16x8_t bk[4] = {fp8x8_to_bf16x8(v.c[nt][0].x, v.c[nt][0].y),
                                    fp8x8_to_bf16x8(v.c[nt][0].z, v.c[nt][0].w),
                                    fp8x8_to_bf16x8(v.c[nt][1].x, v.c[nt][1].y),
                                    fp8x8_to_bf16x8(v.c[nt][1].z, v.c[nt][1].w)};
            f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], bk[s], acc, 0, 0, 0);
            sc[nt] = relu_sum4(acc) * v.sc[nt];
        }
        const int64_t b = base + 4 * m;
        if (g == 0 && b < b_end) {
            if (b + 3 < b_end) {
                *(float4 *)(srow + b) = make_float4(sc[0], sc[1], sc[2], sc[3]);
            } else {
                for (int j = 0; j < (int)(b_end - b); ++j) srow[b + j] = sc[j];
            }
            if (hist) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (b + j < b_end) atomicAdd(&lhist[score_key(sc[j]) >> kHistShift], 1u);
            }
        }
    };
    for (; base < b_end; base += 512) {
        load(base + 256, p1, v1);
        page_ahead(kp, seq, base + 768, m, b_end, p1);
        __builtin_amdgcn_sched_barrier(0);
        score(base, v0);
        load(base + 512, p0, v0);
        page_ahead(kp, seq, base + 1024, m, b_end, p0);
        __builtin_amdgcn_sched_barrier(0);
        score(base + 256, v1);
    }
    if (hist) hist_flush(lhist, hist + (int64_t)r * kRowScratch);
}

// ---------------------------------------------------------------------------
// fp32, any number of rows: grid (chunks of 256 blocks, rows), one thread per
// block, q~ of the row in LDS (read by broadcast).  A thread's 512-byte key
// is read with all of its 16-byte loads in flight: two batches of 16.
// ---------------------------------------------------------------------------
constexpr int kChunkF32 = 256;
__global__ __launch_bounds__(kChunkF32) void score_rows_f32_kernel(
    const float *__restrict__ qrot, const int32_t *__restrict__ row_seq, const int32_t *__restrict__ row_pos,
    const float *__restrict__ pooled, int64_t pooled_stride, KeyPages kp, int32_t max_nb, float *__restrict__ scores,
    int64_t sc_stride, uint32_t *__restrict__ hist)
{
    __shared__ float4 qs[kIdxHeads * kDim / 4];
    __shared__ uint32_t lhist[kHistBins];
    const int r = blockIdx.y;
    const int64_t nc = min(visible_blocks(row_pos[r]), (int64_t)max_nb);
    const int64_t b_begin = (int64_t)blockIdx.x * kChunkF32;
    if (b_begin >= nc) return;
    const int64_t b = b_begin + threadIdx.x;
    const bool valid = b < nc;
    const int64_t seq = row_seq[r];
    // the key is requested before the query and histogram are set up
    const float4 *kr = (const float4 *)(pooled + key_offset(kp, pooled_stride, seq, valid ? b : nc - 1));
    constexpr int kHalf4 = kDim / 8;  // float4s per batch
    float4 kv[kHalf4];
#pragma unroll
    for (int i = 0; i < kHalf4; ++i) kv[i] = kr[i];
    if (hist) hist_clear(lhist);
    for (int i = threadIdx.x; i < kIdxHeads * kDim / 4; i += blockDim.x)
        qs[i] = ((const float4 *)(qrot + (int64_t)r * kIdxHeads * kDim))[i];
    __syncthreads();
    float d[kIdxHeads] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (half == 1) {
#pragma unroll
            for (int i = 0; i < kHalf4; ++i) kv[i] = kr[kHalf4 + i];
        }
#pragma unroll
        for (int i = 0; i < kHalf4; ++i) {
#pragma unroll
            for (int h = 0; h < kIdxHeads; ++h) {
                const float4 qv = qs[h * (kDim / 4) + half * kHalf4 + i];
                d[h] = fmaf(qv.x, kv[i].x, d[h]);
                d[h] = fmaf(qv.y, kv[i].y, d[h]);
                d[h] = fmaf(qv.z, kv[i].z, d[h]);
                d[h] = fmaf(qv.w, kv[i].w, d[h]);
            }
        }
    }
    if (valid) {
        const float sc = ((fmaxf(d[0], 0.0f) + fmaxf(d[1], 0.0f)) + fmaxf(d[2], 0.0f)) + fmaxf(d[3], 0.0f);
        scores[(int64_t)r * sc_stride + b] = sc;
        if (hist) atomicAdd(&lhist[score_key(sc) >> kHistShift], 1u);
    }
    if (hist) hist_flush(lhist, hist + (int64_t)r * kRowScratch);
}

int64_t score_chunks(int32_t max_nb) { return ((int64_t)max_nb + kChunk - 1) / kChunk; }

void launch_score_rows(const void *qrot, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                       const void *pooled, int64_t pooled_stride, const KeyPages &kp, int32_t max_nb, float *scores,
                       int64_t sc_stride, uint32_t *hist, bool bf16, hipStream_t stream)
{
    if (bf16) {
        const dim3 grid((unsigned)score_chunks(max_nb), (unsigned)rows), block(256);
        QSA_LAUNCH("score_rows_bf16", score_rows_bf16_kernel, grid, block, 0, stream, (const bf16_t *)qrot, row_seq,
                   row_pos, (const bf16_t *)pooled, pooled_stride, kp, max_nb, scores, sc_stride, hist);
    } else {
        const dim3 grid((unsigned)(((int64_t)max_nb + kChunkF32 - 1) / kChunkF32), (unsigned)rows), block(kChunkF32);
        QSA_LAUNCH("score_rows_f32", score_rows_f32_kernel, grid, block, 0, stream, (const float *)qrot, row_seq,
                   row_pos, (const float *)pooled, pooled_stride, kp, max_nb, scores, sc_stride, hist);
    }
}

void launch_score_rows_fp8(const void *qrot, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                           const uint8_t *codes, const float *scales, int64_t pooled_stride, const KeyPages &kp,
                           int32_t max_nb, float *scores, int64_t sc_stride, uint32_t *hist, hipStream_t stream)
{
    const dim3 grid((unsigned)score_chunks(max_nb), (unsigned)rows), block(256);
    QSA_LAUNCH("score_rows_fp8", score_rows_fp8_kernel, grid, block, 0, stream, (const bf16_t *)qrot, row_seq,
               row_pos, codes, scales, pooled_stride, kp, max_nb, scores, sc_stride, hist);
}

}  // namespace qsa
