// pool.hip -- steps a1-a4: block mean pooling with post-pool RoPE, and the
// rotation of the index queries.
//
// "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
// Attention": four raw index keys are averaged in FP32 and rotated with the
// first token's position; the compressed key is stored in BF16.  Architecture
// guide, "How a token moves through the model", item 2: the rotation comes
// after pooling, so keys of different positions are not averaged with
// different phases.  The index queries are rotated at their own positions
// (reading: the pages use RoPE in the indexer but do not spell out the query
// side; without it a score would not depend on the query's position).
#include <cmath>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

// RoPE frequencies theta^(-j/64) of the 64 rotary pairs.
RopeFreq rope_freq_plain(double theta)
{
    RopeFreq r;
    for (int j = 0; j < kHalf; ++j) r.f[j] = std::pow(theta, -(double)j / (double)kHalf);
    return r;
}

// YaRN for long contexts (the pages: the 262,144-token native context extends
// to one million tokens with YaRN; the method is Peng, Quesnelle, Fan and
// Shippole, "YaRN: Efficient Context Window Extension of Large Language
// Models", 2023, its interpolation by parts).  Pair j turns
// r = L * theta_j / (2 pi) times over the original context of L tokens; a
// pair with r > beta keeps theta_j, a pair with r < alpha gets theta_j / s,
// and between them the weight gamma = (r - alpha) / (beta - alpha) blends the
// two: (1 - gamma) * theta_j / s + gamma * theta_j.  The method's attention
// temperature scales scores by a positive constant, which the indexer's
// ranking cannot see; it is not applied here.
RopeFreq rope_freq_yarn(double theta, double s, double L, double alpha, double beta)
{
    RopeFreq r = rope_freq_plain(theta);
    if (s == 1.0) return r;
    const double two_pi = 6.283185307179586476925;
    for (int j = 0; j < kHalf; ++j) {
        const double th = r.f[j];
        const double turns = L * th / two_pi;
        const double gamma = turns < alpha ? 0.0 : turns > beta ? 1.0 : (turns - alpha) / (beta - alpha);
        r.f[j] = (1.0 - gamma) * th / s + gamma * th;
    }
    return r;
}

// One wave per pooled block: lane j owns the rotary pair (j, j + 64).  The
// wave reads the block's 4 tokens x 128 dims (contiguous in memory) with 8
// coalesced loads.  The key goes to block b of its sequence, contiguous or
// through the page table of a paged compressed-key pool.
template <typename T>
__global__ __launch_bounds__(256) void pool_rope_kernel(const T *__restrict__ raw, int64_t raw_stride,
                                                        T *__restrict__ pooled, int64_t pooled_stride, KeyPages kp,
                                                        int64_t total, int32_t nblk, int32_t block_begin,
                                                        RopeFreq rf, uint32_t flags,
                                                        const float *__restrict__ norm_w)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (w >= total) return;
    const int64_t s = w / nblk;
    const int64_t b = block_begin + w % nblk;
    const double freq = rf.f[lane];  // loaded ahead of the keys: the angle is formed while they are in flight
    const T *src = raw + s * raw_stride + b * (kBlock * kDim);
    float vx[kBlock], vy[kBlock];
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
        vx[i] = load_f32(src + i * kDim + lane);
        vy[i] = load_f32(src + i * kDim + kHalf + lane);
    }
    double c, sn;
    rope_angle(kBlock * b, freq, c, sn);
    float x = 0.0f, y = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {  // FP32 sum in token order, then times 1/4
        x += vx[i];
        y += vy[i];
    }
    x *= 0.25f;
    y *= 0.25f;
    double dx = x, dy = y;
    if (flags & kFlagRmsNorm) {
        const double ss = wave_sum_f64(dx * dx + dy * dy);
        const double inv = 1.0 / sqrt(ss / (double)kDim + 1e-6);
        dx *= inv;
        dy *= inv;
        if (norm_w) {  // learned per-dim weight of the norm
            dx *= (double)norm_w[lane];
            dy *= (double)norm_w[kHalf + lane];
        }
    }
    if (!(flags & kFlagNoRope)) rope_apply(dx, dy, c, sn);
    T *dst = pooled + key_offset(kp, pooled_stride, s, b);
    store_f64(dst + lane, dx);
    store_f64(dst + kHalf + lane, dy);
}

// The same block pooling with the compressed key stored in FP8 E4M3 and one
// FP32 scale ("Qwen3.8-Flash-Next, Layer by Layer", section "Serving it": the
// indexer's keys are kept in FP8).  The rotated key is rounded to FP32; its
// largest magnitude amax maps to 448, the largest E4M3 value: inv = 448/amax,
// scale = amax/448 (IEEE FP32 quotients), code = E4M3(k * inv) rounded to
// nearest even by v_cvt_pk_fp8_f32.  |k * inv| <= 448 (1 + 2^-23), so no code
// overflows.  A zero key gets scale 0 and zero codes.
template <typename T>
__global__ __launch_bounds__(256) void pool_rope_fp8_kernel(const T *__restrict__ raw, int64_t raw_stride,
                                                            uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                            int64_t pooled_stride, KeyPages kp, int64_t total,
                                                            int32_t nblk, int32_t block_begin, RopeFreq rf,
                                                            uint32_t flags)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (w >= total) return;
    const int64_t s = w / nblk;
    const int64_t b = block_begin + w % nblk;
    const double freq = rf.f[lane];  // loaded ahead of the keys: the angle is formed while they are in flight
    const T *src = raw + s * raw_stride + b * (kBlock * kDim);
    float vx[kBlock], vy[kBlock];
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {
        vx[i] = load_f32(src + i * kDim + lane);
        vy[i] = load_f32(src + i * kDim + kHalf + lane);
    }
    double c, sn;
    rope_angle(kBlock * b, freq, c, sn);
    float x = 0.0f, y = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlock; ++i) {  // FP32 sum in token order, then times 1/4
        x += vx[i];
        y += vy[i];
    }
    x *= 0.25f;
    y *= 0.25f;
    double dx = x, dy = y;
    if (flags & kFlagRmsNorm) {
        const double ss = wave_sum_f64(dx * dx + dy * dy);
        const double inv = 1.0 / sqrt(ss / (double)kDim + 1e-6);
        dx *= inv;
        dy *= inv;
    }
    if (!(flags & kFlagNoRope)) rope_apply(dx, dy, c, sn);
    const float fx = (float)dx, fy = (float)dy;
    const float amax = wave_max(fmaxf(fabsf(fx), fabsf(fy)));
    const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
    const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fx * inv, fy * inv, 0, false);
    const int64_t slot = key_index(kp, pooled_stride, s, b);
    codes[slot * kDim + lane] = (uint8_t)(pk & 0xffu);
    codes[slot * kDim + kHalf + lane] = (uint8_t)((pk >> 8) & 0xffu);
    if (lane == 0) scales[slot] = amax / 448.0f;
}

// One wave per row: q~ = round_dtype(RoPE(q, row_pos)) for the row's 4 index
// heads.  Lane j forms the angle of rotary pair (j, j + 64) once and rotates
// that pair of every head.  The wave also clears `zero_per_row` words of the
// row's select scratch, so the selection needs no separate fill.
template <typename T>
__global__ __launch_bounds__(256) void rope_query_kernel(const T *__restrict__ q, const int32_t *__restrict__ row_pos,
                                                         int32_t rows, T *__restrict__ qrot, RopeFreq rf,
                                                         uint32_t flags, uint32_t *__restrict__ zero,
                                                         int64_t zero_per_row)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (r >= rows) return;
    if (zero) {
        uint32_t *z = zero + r * zero_per_row;
        if ((zero_per_row & 3) == 0 && ((uintptr_t)z & 15u) == 0) {  // 16-byte stores
            for (int64_t i = lane; i < zero_per_row / 4; i += kWave) ((uint4 *)z)[i] = make_uint4(0u, 0u, 0u, 0u);
        } else {
            for (int64_t i = lane; i < zero_per_row; i += kWave) z[i] = 0u;
        }
    }
    // the position and the frequency are loaded first, so the angle's sine
    // and cosine are formed while the query's 8 loads are in flight
    const int64_t pos = row_pos[r];
    const double freq = rf.f[lane];
    const T *src = q + r * kIdxHeads * kDim;
    float fx[kIdxHeads], fy[kIdxHeads];
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) {
        fx[h] = load_f32(src + h * kDim + lane);
        fy[h] = load_f32(src + h * kDim + kHalf + lane);
    }
    double dx[kIdxHeads], dy[kIdxHeads];
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) {
        dx[h] = fx[h];
        dy[h] = fy[h];
    }
    double c, s;
    rope_angle(pos, freq, c, s);  // formed on every path, so its loads stay ahead of the query's
    if (!(flags & kFlagNoRope)) {
#pragma unroll
        for (int h = 0; h < kIdxHeads; ++h) rope_apply(dx[h], dy[h], c, s);
    }
    T *dst = qrot + r * kIdxHeads * kDim;
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) {
        store_f64(dst + h * kDim + lane, dx[h]);
        store_f64(dst + h * kDim + kHalf + lane, dy[h]);
    }
}

// Incremental pooling for decode: one wave per request.  The new raw key goes
// to ring slot t mod 4; when it completes block b = t / 4, the four ring keys
// (slots 0..3 are tokens 4b..4b+3; slot 3 is the new key, taken from
// registers) are pooled in FP32 token order, rotated at 4b and stored at
// compressed slot full_slot / 4.  "Qwen3.8-Flash-Next: Day-0 Support in
// SGLang", section "Qwen Sparse Attention": the raw keys of the unfinished
// block live in a four-slot per-request ring, and page-aligned full_slot / 4
// addressing places the compressed key.
template <typename T>
__global__ __launch_bounds__(256) void pool_append_kernel(const T *__restrict__ new_keys,
                                                          const int32_t *__restrict__ positions,
                                                          const int64_t *__restrict__ full_slots, T *__restrict__ ring,
                                                          T *__restrict__ compressed, int32_t batch, RopeFreq rf,
                                                          uint32_t flags)
{
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (r >= batch) return;
    const int64_t t = positions[r];
    const int slot = (int)(t & (kBlock - 1));
    const T *src = new_keys + r * kDim;
    const T kx = src[lane], ky = src[kHalf + lane];
    T *rr = ring + r * kBlock * kDim;
    rr[slot * kDim + lane] = kx;
    rr[slot * kDim + kHalf + lane] = ky;
    if (slot != kBlock - 1) return;
    float x = 0.0f, y = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlock - 1; ++i) {  // FP32 sum in token order, then times 1/4
        x += load_f32(rr + i * kDim + lane);
        y += load_f32(rr + i * kDim + kHalf + lane);
    }
    x += load_f32(&kx);
    y += load_f32(&ky);
    x *= 0.25f;
    y *= 0.25f;
    double dx = x, dy = y;
    if (flags & kFlagRmsNorm) {
        const double ss = wave_sum_f64(dx * dx + dy * dy);
        const double inv = 1.0 / sqrt(ss / (double)kDim + 1e-6);
        dx *= inv;
        dy *= inv;
    }
    if (!(flags & kFlagNoRope)) rope_pair(dx, dy, t - slot, rf.f[lane]);
    T *dst = compressed + (full_slots[r] / kBlock) * kDim;
    store_f64(dst + lane, dx);
    store_f64(dst + kHalf + lane, dy);
}

void launch_pool_append(const void *new_keys, const int32_t *positions, const int64_t *full_slots, void *ring,
                        void *compressed, int32_t batch, const RopeFreq &rf, uint32_t flags, bool bf16,
                        hipStream_t stream)
{
    const dim3 grid((unsigned)((batch + 3) / 4)), block(256);
    if (bf16)
        QSA_LAUNCH("pool_append", (pool_append_kernel<bf16_t>), grid, block, 0, stream, (const bf16_t *)new_keys,
                   positions, full_slots, (bf16_t *)ring, (bf16_t *)compressed, batch, rf, flags);
    else
        QSA_LAUNCH("pool_append", (pool_append_kernel<float>), grid, block, 0, stream, (const float *)new_keys,
                   positions, full_slots, (float *)ring, (float *)compressed, batch, rf, flags);
}

void launch_pool(const void *raw, int64_t raw_stride, void *pooled, int64_t pooled_stride, const KeyPages &kp,
                 int32_t batch, int32_t block_begin, int32_t block_end, const RopeFreq &rf, uint32_t flags,
                 bool bf16, hipStream_t stream, const float *norm_weight)
{
    const int32_t nblk = block_end - block_begin;
    const int64_t total = (int64_t)batch * nblk;
    const dim3 grid((unsigned)((total + 3) / 4)), block(256);
    if (bf16)
        QSA_LAUNCH("pool_rope", (pool_rope_kernel<bf16_t>), grid, block, 0, stream, (const bf16_t *)raw,
                   raw_stride, (bf16_t *)pooled, pooled_stride, kp, total, nblk, block_begin, rf, flags,
                   norm_weight);
    else
        QSA_LAUNCH("pool_rope", (pool_rope_kernel<float>), grid, block, 0, stream, (const float *)raw, raw_stride,
                   (float *)pooled, pooled_stride, kp, total, nblk, block_begin, rf, flags, norm_weight);
}

void launch_pool_fp8(const void *raw, int64_t raw_stride, uint8_t *codes, float *scales, int64_t pooled_stride,
                     const KeyPages &kp, int32_t batch, int32_t block_begin, int32_t block_end, const RopeFreq &rf,
                     uint32_t flags, bool bf16_raw, hipStream_t stream)
{
    const int32_t nblk = block_end - block_begin;
    const int64_t total = (int64_t)batch * nblk;
    const dim3 grid((unsigned)((total + 3) / 4)), block(256);
    if (bf16_raw)
        QSA_LAUNCH("pool_rope_fp8", (pool_rope_fp8_kernel<bf16_t>), grid, block, 0, stream, (const bf16_t *)raw,
                   raw_stride, codes, scales, pooled_stride, kp, total, nblk, block_begin, rf, flags);
    else
        QSA_LAUNCH("pool_rope_fp8", (pool_rope_fp8_kernel<float>), grid, block, 0, stream, (const float *)raw,
                   raw_stride, codes, scales, pooled_stride, kp, total, nblk, block_begin, rf, flags);
}

void launch_rope_query(const void *q, const int32_t *row_pos, int32_t rows, void *qrot, const RopeFreq &rf,
                       uint32_t flags, bool bf16, uint32_t *zero, int64_t zero_per_row, hipStream_t stream)
{
    const dim3 grid((unsigned)(((int64_t)rows + 3) / 4)), block(256);
    if (bf16)
        QSA_LAUNCH("rope_query", (rope_query_kernel<bf16_t>), grid, block, 0, stream, (const bf16_t *)q, row_pos,
                   rows, (bf16_t *)qrot, rf, flags, zero, zero_per_row);
    else
        QSA_LAUNCH("rope_query", (rope_query_kernel<float>), grid, block, 0, stream, (const float *)q, row_pos,
                   rows, (float *)qrot, rf, flags, zero, zero_per_row);
}

}  // namespace qsa
