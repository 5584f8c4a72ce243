// qsa_device.h -- device helpers shared by the libqsa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa_internal.h"

namespace qsa {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));   // MFMA operand (8 x bf16)
typedef float f32x4_t __attribute__((ext_vector_type(4)));      // 16x16 MFMA accumulator

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ bf16x8_t zero_bf16x8() { return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, b16x2_t));
}

// Eight FP8 E4M3 codes (bytes of w0 then w1, lowest first) -> eight bf16, as
// one MFMA operand.  The conversion is exact: every E4M3 value (at most 4
// significant bits, 2^-9 .. 448) is a bf16 value.
__device__ __forceinline__ uint4 fp8x8_to_bf16_words(uint32_t w0, uint32_t w1)
{
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
    return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(b[0], b[1]), pack_bf16x2(c[0], c[1]),
                      pack_bf16x2(d[0], d[1]));
}
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    return as_bf16x8(fp8x8_to_bf16_words(w0, w1));
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16, round to nearest, ties to even.
__device__ __forceinline__ bf16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// double -> bf16 with a single rounding (nearest-even): narrow to float with
// round-to-odd (truncate toward zero, then set the last bit if anything was
// dropped); float keeps 16 more bits than bf16, so the final nearest-even
// step then rounds exactly as a direct double -> bf16 rounding would.
__device__ __forceinline__ bf16_t f64_to_bf16(double x)
{
    float r = (float)x;
    if (!isfinite(r) || (double)r == x) return f32_to_bf16(r);
    if (fabs((double)r) > fabs(x)) r = __uint_as_float(__float_as_uint(r) - 1u);  // toward zero
    return f32_to_bf16(__uint_as_float(__float_as_uint(r) | 1u));
}

template <typename T> __device__ __forceinline__ float load_f32(const T *p);
template <> __device__ __forceinline__ float load_f32<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t *p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ void store_f64(T *p, double v);
template <> __device__ __forceinline__ void store_f64<float>(float *p, double v) { *p = (float)v; }
template <> __device__ __forceinline__ void store_f64<bf16_t>(bf16_t *p, double v) { *p = f64_to_bf16(v); }

template <typename T> __device__ __forceinline__ void store_f32(T *p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float *p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<bf16_t>(bf16_t *p, float v) { *p = f32_to_bf16(v); }

// Eight consecutive elements as floats (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load8(const bf16_t *p, float *o)
{
    const uint4 v = *(const uint4 *)p;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(w[i] << 16);
        o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float *o)
{
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Order-preserving unsigned key of a float score (bigger score -> bigger
// key); -0 and +0 map to one key.
__device__ __forceinline__ uint32_t score_key(float s)
{
    uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

// Key number of block b of sequence seq: seq*keys_per_seq + b, or through
// the page table of the compressed-key pool.
__device__ __forceinline__ int64_t key_index(const KeyPages &kp, int64_t keys_per_seq, int64_t seq, int64_t b)
{
    if (!kp.table) return seq * keys_per_seq + b;
    return (int64_t)kp.table[seq * kp.stride + b / kp.bpp] * kp.bpp + b % kp.bpp;
}
// The table entry of block b's page (paged pools; 0 when contiguous), and
// the key number of block b given that entry, as key_index.  Reading the
// entry a step ahead of the key lets a key load skip the wait for the table.
__device__ __forceinline__ int32_t page_entry(const KeyPages &kp, int64_t seq, int64_t b)
{
    return kp.table ? kp.table[seq * kp.stride + (uint32_t)b / (uint32_t)kp.bpp] : 0;
}
__device__ __forceinline__ int64_t key_at(const KeyPages &kp, int64_t keys_per_seq, int64_t seq, int64_t b,
                                          int32_t pg)
{
    if (!kp.table) return seq * keys_per_seq + b;
    return (int64_t)pg * kp.bpp + (int64_t)((uint32_t)b % (uint32_t)kp.bpp);
}
// Element offset of that key's 128 values in a bf16 / fp32 key array whose
// sequences are `seq_stride` elements apart when contiguous.
__device__ __forceinline__ int64_t key_offset(const KeyPages &kp, int64_t seq_stride, int64_t seq, int64_t b)
{
    if (!kp.table) return seq * seq_stride + b * kDim;
    return key_index(kp, 0, seq, b) * kDim;
}

// Complete micro-blocks visible to a query at position t: 4b + 3 <= t.
__device__ __forceinline__ int64_t visible_blocks(int64_t t) { return (t + 1) / kBlock; }

// Rotate the pair (x, y) = (v[j], v[j+64]) at integer position `pos` with
// frequency inv_freq = theta^(-j/64); the angle and the rotation are formed
// in double precision.
__device__ __forceinline__ void rope_angle(int64_t pos, double inv_freq, double &c, double &s)
{
#pragma clang fp contract(off)
    const double ang = (double)pos * inv_freq;
    sincos(ang, &s, &c);
}
__device__ __forceinline__ void rope_apply(double &x, double &y, double c, double s)
{
#pragma clang fp contract(off)
    const double nx = x * c - y * s;
    const double ny = x * s + y * c;
    x = nx;
    y = ny;
}
__device__ __forceinline__ void rope_pair(double &x, double &y, int64_t pos, double inv_freq)
{
    double c, s;
    rope_angle(pos, inv_freq, c, s);
    rope_apply(x, y, c, s);
}

// max(x, 0) of a finite float as one integer max on its bits: a negative
// float (or -0) has the sign bit set and so compares below 0 as an int; the
// float form would first quiet a possible signalling NaN.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Inclusive scan of `op` over the 64 lanes of a wave through DPP lane moves
// (no LDS round trip): shifts by 1, 2, 4 and 8 inside each 16-lane row, then
// the last lane of a row is broadcast into the rows after it.
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan_op(uint32_t v, Op op)
{
    const int lane = threadIdx.x & 63, rl = lane & 15;
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v = rl >= 1 ? op(v, t) : v;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v = rl >= 2 ? op(v, t) : v;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v = rl >= 4 ? op(v, t) : v;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v = rl >= 8 ? op(v, t) : v;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x142, 0xf, 0xf, false);  // row_bcast:15
    v = (lane & 31) >= 16 ? op(v, t) : v;
    t = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x143, 0xf, 0xf, false);  // row_bcast:31
    v = lane >= 32 ? op(v, t) : v;
    return v;
}

// Inclusive prefix sum over the wave's lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v)
{
    return wave_incl_scan_op(v, [](uint32_t x, uint32_t y) { return x + y; });
}

// Value of a wave-uniform lane's register.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int lane) { return (uint32_t)__builtin_amdgcn_readlane((int)v, lane); }

// Bitwise OR of a value over the wave's lanes.
__device__ __forceinline__ uint32_t wave_or(uint32_t v)
{
    return lane_value(wave_incl_scan_op(v, [](uint32_t x, uint32_t y) { return x | y; }), 63);
}

// Max and sum of a float over the wave's lanes (every lane gets the result):
// the DPP scan on the value's bits, then lane 63's total.
__device__ __forceinline__ float wave_max(float v)
{
    const uint32_t s = wave_incl_scan_op(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    });
    return __uint_as_float(lane_value(s, 63));
}
__device__ __forceinline__ float wave_sum(float v)
{
    const uint32_t s = wave_incl_scan_op(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    });
    return __uint_as_float(lane_value(s, 63));
}
__device__ __forceinline__ double wave_sum_f64(double v)
{
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace qsa
