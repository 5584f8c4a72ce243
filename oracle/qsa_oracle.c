/*
 * qsa_oracle.c -- plain CPU oracle for the Qwen Sparse Attention (QSA) hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this code.  The product
 * library never links it, and it shares no source, header, constant or helper
 * with the GPU path.
 *
 * Sources (the web pages, by title and section):
 *   [SGL]  "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section
 *          "Qwen Sparse Attention: Retrieve Coarsely, Attend Precisely"
 *          (pooling, the score equation s_{t,b}, top-512, tail, attention on
 *          the original K/V) and section "IndexShare MTP" (one selection
 *          shared by the draft rows plus the positions drafted since).
 *   [ARCH] "Qwen3.8-Flash-Next architecture" guide, "How a token moves through
 *          the model", item 2 (RoPE after pooling, 512 blocks = 2,048 tokens
 *          plus the incomplete tail block).
 *   [LBL]  "Qwen3.8-Flash-Next, Layer by Layer", section "Token mixing"
 *          (4 query heads, 1 key head, 128 dims, mean of 4 keys, best 512)
 *          and section "Serving it" (indexer keys and the KV cache in FP8).
 *
 * Every floating-point step runs in double precision, except where the pages
 * fix the precision: the block mean is taken in FP32 ([SGL]) and the
 * compressed key is stored in BF16 ([SGL]).  Readings taken where the pages
 * are silent are stated at each function.
 *
 * The code is deliberately plain: one row at a time, a full sort for the
 * selection, a textbook max-subtracted softmax.  An OpenMP loop over
 * independent rows (or blocks) is the only concession to speed.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_DIM 128        /* indexer head dimension ([SGL], [LBL]) */
#define OR_HALF 64        /* rotate-half pairs (j, j + 64) */
#define OR_BLOCK 4        /* tokens per micro-block, "c4" ([SGL]) */
#define OR_IDX_HEADS 4    /* indexer query heads ([SGL], [LBL]) */

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_FLAG_NO_ROPE = 1u, OR_FLAG_POOL_RMSNORM = 2u };

enum {
    OR_OK = 0,
    OR_ERR_ARG = 1,
    OR_ERR_ALLOC = 2
};

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 bits -> value: a bf16 number is the top half of an IEEE binary32. */
double qsa_oracle_bf16_to_double(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * value -> bf16 bits, rounding to the nearest representable bf16 number with
 * ties to even, straight from the double (one rounding).  bf16 keeps 8
 * significant bits and binary32's exponent range; below 2^-126 the spacing is
 * the subnormal step 2^-133.
 */
uint16_t qsa_oracle_bf16_from_double(double x)
{
    if (isnan(x))
        return 0x7fc0;
    if (isinf(x))
        return x > 0 ? 0x7f80 : 0xff80;
    if (x == 0.0)
        return signbit(x) ? 0x8000 : 0x0000;
    double ax = fabs(x);
    int e;
    frexp(ax, &e); /* ax = m * 2^e, m in [0.5, 1) -> top bit has weight 2^(e-1) */
    int ulp_exp = (e - 1) - 7;
    if (ulp_exp < -133)
        ulp_exp = -133;
    double ulp = ldexp(1.0, ulp_exp);
    double r = rint(ax / ulp) * ulp; /* rint: round half to even (default mode) */
    const double bf16_max = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
    uint32_t bits;
    if (r > bf16_max) {
        bits = 0x7f800000u;
    } else {
        float f = (float)r; /* exact: r has at most 8 significant bits */
        memcpy(&bits, &f, sizeof bits);
    }
    uint16_t h = (uint16_t)(bits >> 16);
    return x < 0 ? (uint16_t)(h | 0x8000u) : h;
}

/*
 * FP8 E4M3 (the OCP 8-bit format: 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; exponent
 * 15 with mantissa 7 is NaN; no infinities; largest finite value 448).
 * Reading: "Qwen3.8-Flash-Next, Layer by Layer", section "Serving it", stores
 * the indexer's keys in FP8 without naming the variant; E4M3 is the FP8 KV
 * format of the engines it names.
 */
double qsa_oracle_fp8_to_double(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/*
 * x -> E4M3 code: the nearest representable value, ties to the even code
 * (mantissa lsb 0).  Magnitudes beyond 464 (halfway from 448 to the next
 * binade step) have no finite neighbour and give NaN (0x7f / 0xff); the key
 * scaling below never produces them.  The value is located on the grid of
 * its binade: spacing 2^-9 below 2^-6, else 2^(e-3) for 2^e <= |x| < 2^(e+1).
 */
uint8_t qsa_oracle_fp8_from_double(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (isnan(a) || a > 464.0)
        return sign | 0x7f;
    double q;  /* grid spacing at a */
    if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9);
    } else {
        int e;
        frexp(a, &e);          /* a = f * 2^e, 0.5 <= f < 1: binade [2^(e-1), 2^e) */
        q = ldexp(1.0, e - 1 - 3);
    }
    double r = nearbyint(a / q) * q;  /* a / q is exact; nearbyint rounds ties to even */
    if (r == 0.0)
        return sign;
    if (r < ldexp(1.0, -6))            /* subnormal: mantissa = r / 2^-9 */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    int e;
    double f = frexp(r, &e);           /* r = f * 2^e, f in [0.5, 1) */
    int ef = e - 1 + 7;                /* biased exponent of r = (2f) * 2^(e-1) */
    int mant = (int)((2.0 * f - 1.0) * 8.0);
    return sign | (uint8_t)(ef << 3) | (uint8_t)mant;
}

/* The same rounding over an array (n values). */
void qsa_oracle_fp8_encode(const double *x, uint8_t *codes, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        codes[i] = qsa_oracle_fp8_from_double(x[i]);
}

static double load_elem(const void *base, int64_t idx, int dtype)
{
    if (dtype == OR_BF16)
        return qsa_oracle_bf16_to_double(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/* Round to the storage dtype and store. fp32: C's conversion, nearest-even. */
static void store_elem(void *base, int64_t idx, int dtype, double v)
{
    if (dtype == OR_BF16)
        ((uint16_t *)base)[idx] = qsa_oracle_bf16_from_double(v);
    else
        ((float *)base)[idx] = (float)v;
}

/* Value after rounding to the dtype, kept as a double. */
static double round_to_dtype(double v, int dtype)
{
    if (dtype == OR_BF16)
        return qsa_oracle_bf16_to_double(qsa_oracle_bf16_from_double(v));
    return (double)(float)v;
}

/* ------------------------------------------------------------------------ */
/* RoPE                                                                      */
/* ------------------------------------------------------------------------ */

/*
 * Rotary embedding of one 128-d vector at integer position `pos`.
 * Reading (the pages give no layout): the full 128 dims rotate, as
 * "rotate-half" pairs (j, j + 64), j = 0..63, with angle pos * theta^(-j/64)
 * (= theta^(-2j/128)).  Text MRoPE has equal position components, so it is
 * plain 1-D RoPE at the token index ([SGL] "first token's MRoPE position").
 * The angle is formed and rotated in double precision.
 */
void qsa_oracle_rope(double *v, int64_t pos, double theta)
{
    for (int j = 0; j < OR_HALF; ++j) {
        double inv_freq = pow(theta, -(double)j / (double)OR_HALF);
        double ang = (double)pos * inv_freq;
        double c = cos(ang), s = sin(ang);
        double x = v[j], y = v[j + OR_HALF];
        v[j] = x * c - y * s;
        v[j + OR_HALF] = x * s + y * c;
    }
}

/*
 * The same rotation with the 64 pair frequencies given (inv_freq[j] for the
 * pair (j, j + 64)): the angle of pair j at `pos` is pos * inv_freq[j].
 */
void qsa_oracle_rope_freq(double *v, int64_t pos, const double *inv_freq)
{
    for (int j = 0; j < OR_HALF; ++j) {
        double ang = (double)pos * inv_freq[j];
        double c = cos(ang), s = sin(ang);
        double x = v[j], y = v[j + OR_HALF];
        v[j] = x * c - y * s;
        v[j + OR_HALF] = x * s + y * c;
    }
}

/* Plain RoPE's frequencies theta^(-j/64), as qsa_oracle_rope forms them. */
void qsa_oracle_rope_plain_freq(double theta, double *inv_freq)
{
    for (int j = 0; j < OR_HALF; ++j)
        inv_freq[j] = pow(theta, -(double)j / (double)OR_HALF);
}

/*
 * YaRN-scaled frequencies for long contexts.  The pages say only that the
 * 262,144-token native context extends to one million tokens with YaRN
 * (flozi.net guide, "What the published evidence does and does not show";
 * aicontrolled journal, "Remembering does not require looking at everything
 * at once"); they give no parameters.  Reading: the published YaRN method
 * (Peng, Quesnelle, Fan and Shippole, "YaRN: Efficient Context Window
 * Extension of Large Language Models", 2023), its frequency interpolation
 * "by parts", in its notation:
 *   theta_d = base^(-2d/|D|) is pair d's frequency and lambda_d = 2 pi / theta_d
 *     its wavelength (|D| = 128 rotary dims, so theta_d = base^(-d/64));
 *   r(d) = L / lambda_d is how many turns pair d makes over the original
 *     context L;
 *   the ramp gamma(r) is 0 for r < alpha, 1 for r > beta and
 *     (r - alpha) / (beta - alpha) between;
 *   h(theta_d) = (1 - gamma(r(d))) * theta_d / s + gamma(r(d)) * theta_d,
 *     with s the context scale factor.
 * Pairs that turn many times over L keep their frequency, pairs that turn
 * less than once are interpolated by 1/s, and the ramp blends in between.
 * For the indexer, s = 1,048,576 / 262,144 = 4, L = 262,144 and the paper's
 * alpha = 1, beta = 32.  YaRN's attention temperature scales logits by a
 * positive constant; the indexer's ranking of ReLU sums cannot see it, so it
 * is not applied here (for the final attention it is part of the softmax
 * scale the caller passes).  s == 1 gives plain RoPE's frequencies up to
 * rounding.
 */
int qsa_oracle_yarn_freq(double base, double s, double L, double alpha, double beta, double *inv_freq)
{
    if (!(base > 1.0) || !(s >= 1.0) || !(L > 0.0) || !(beta > alpha) || !inv_freq)
        return OR_ERR_ARG;
    const double two_pi = 2.0 * acos(-1.0);
    for (int d = 0; d < OR_HALF; ++d) {
        const double theta_d = pow(base, -2.0 * d / (double)OR_DIM);
        const double lambda_d = two_pi / theta_d;
        const double r = L / lambda_d;
        double gamma;
        if (r < alpha)
            gamma = 0.0;
        else if (r > beta)
            gamma = 1.0;
        else
            gamma = (r - alpha) / (beta - alpha);
        inv_freq[d] = (1.0 - gamma) * theta_d / s + gamma * theta_d;
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* a1-a3: block pooling, then RoPE at the block's first position             */
/* ------------------------------------------------------------------------ */

/*
 * [SGL]: every four raw index keys are averaged in FP32 and rotated with the
 * first token's position to form one compressed key (stored in BF16).
 * [ARCH] item 2: the rotation comes after the pooling, so keys of different
 * positions are not averaged with different phases.
 *
 * Block b of sequence s covers tokens 4b..4b+3 and is rotated at position 4b.
 * The mean is the FP32 sum x0+x1+x2+x3 (in that order) times 0.25.
 * OR_FLAG_POOL_RMSNORM applies x / sqrt(mean(x^2) + 1e-6) with unit weight
 * before the rotation (the pages say "normalized" without a definition; this
 * is an optional reading, off by default).  OR_FLAG_NO_ROPE skips the
 * rotation.
 *
 * raw:    [batch][raw_seq_stride] elements, token i of sequence s at
 *         raw + s*raw_seq_stride + i*128.
 * pooled: [batch][pooled_seq_stride], block b at pooled + s*stride + b*128.
 */
static int pool_core(const void *raw, int64_t raw_seq_stride, void *pooled, int64_t pooled_seq_stride,
                     int32_t batch, int32_t block_begin, int32_t block_end, const double *inv_freq,
                     const float *norm_weight, uint32_t flags, int32_t dtype)
{
    if (!raw || !pooled || batch < 0 || block_begin < 0 || block_end < block_begin)
        return OR_ERR_ARG;
    int64_t nblk = (int64_t)block_end - block_begin;
    int64_t total = (int64_t)batch * nblk;
#pragma omp parallel for schedule(static)
    for (int64_t w = 0; w < total; ++w) {
        int64_t s = w / nblk;
        int64_t b = block_begin + w % nblk;
        double m[OR_DIM];
        for (int d = 0; d < OR_DIM; ++d) {
            float acc = 0.0f;
            for (int i = 0; i < OR_BLOCK; ++i) {
                int64_t tok = OR_BLOCK * b + i;
                acc += (float)load_elem(raw, s * raw_seq_stride + tok * OR_DIM + d, dtype);
            }
            m[d] = (double)(acc * 0.25f);
        }
        if (flags & OR_FLAG_POOL_RMSNORM) {
            double ss = 0.0;
            for (int d = 0; d < OR_DIM; ++d)
                ss += m[d] * m[d];
            double inv = 1.0 / sqrt(ss / OR_DIM + 1e-6);
            for (int d = 0; d < OR_DIM; ++d)
                m[d] *= inv;
            if (norm_weight)
                for (int d = 0; d < OR_DIM; ++d)
                    m[d] *= (double)norm_weight[d];
        }
        if (!(flags & OR_FLAG_NO_ROPE))
            qsa_oracle_rope_freq(m, OR_BLOCK * b, inv_freq);
        for (int d = 0; d < OR_DIM; ++d)
            store_elem(pooled, s * pooled_seq_stride + b * OR_DIM + d, dtype, m[d]);
    }
    return OR_OK;
}

int qsa_oracle_pool(const void *raw, int64_t raw_seq_stride, void *pooled,
                    int64_t pooled_seq_stride, int32_t batch, int32_t block_begin,
                    int32_t block_end, double theta, uint32_t flags, int32_t dtype)
{
    double inv_freq[OR_HALF];
    qsa_oracle_rope_plain_freq(theta, inv_freq);
    return pool_core(raw, raw_seq_stride, pooled, pooled_seq_stride, batch, block_begin, block_end, inv_freq,
                     NULL, flags, dtype);
}

/*
 * qsa_oracle_pool with the rotation's pair frequencies given (plain RoPE's, or
 * YaRN's from qsa_oracle_yarn_freq) and a learned per-dimension weight for the
 * normalization.  [SGL] says the averaged keys are "normalized" before the
 * rotation and gives neither the norm nor a weight; reading, for a learned
 * weight w: with OR_FLAG_POOL_RMSNORM, m <- (m / sqrt(mean(m^2) + 1e-6)) * w
 * element by element (RMS norm with a weight, as in the rest of the model);
 * norm_weight NULL is unit weight.  A weight without the flag is an error.
 */
int qsa_oracle_pool_ex(const void *raw, int64_t raw_seq_stride, void *pooled, int64_t pooled_seq_stride,
                       int32_t batch, int32_t block_begin, int32_t block_end, const double *inv_freq,
                       const float *norm_weight, uint32_t flags, int32_t dtype)
{
    if (!inv_freq || (norm_weight && !(flags & OR_FLAG_POOL_RMSNORM)))
        return OR_ERR_ARG;
    return pool_core(raw, raw_seq_stride, pooled, pooled_seq_stride, batch, block_begin, block_end, inv_freq,
                     norm_weight, flags, dtype);
}

/*
 * Incremental pooling for decode ([SGL]: the raw index keys of a request's
 * unfinished block live in a four-slot per-request ring; one compressed key
 * per four tokens is kept, addressed by page-aligned full_slot / 4).
 *
 * For each request r with its new token at position t = positions[r] and
 * physical KV slot full_slots[r]:
 *   ring[r][t mod 4] = new_keys[r];
 *   if t mod 4 == 3 (the block b = t / 4 is now complete), the four ring
 *   slots -- tokens 4b .. 4b+3, in that order -- are pooled exactly as
 *   qsa_oracle_pool pools a block (FP32 sum in token order times 1/4,
 *   optional RMS norm, rotation at 4b, rounding to dtype) and stored at
 *   compressed[full_slots[r] / 4].
 * Contract (pages aligned to 4 tokens): full_slots[r] mod 4 == t mod 4, so
 * the block's four tokens share one compressed slot.
 * new_keys [batch][128], ring [batch][4][128], compressed [slots / 4][128].
 */
int qsa_oracle_pool_append(const void *new_keys, const int32_t *positions, const int64_t *full_slots, void *ring,
                           void *compressed, int32_t batch, double theta, uint32_t flags, int32_t dtype)
{
    if (!new_keys || !positions || !full_slots || !ring || !compressed || batch < 0)
        return OR_ERR_ARG;
    for (int32_t r = 0; r < batch; ++r) {
        const int64_t t = positions[r];
        if (t < 0)
            return OR_ERR_ARG;
        const int64_t slot = t % OR_BLOCK;
        for (int d = 0; d < OR_DIM; ++d)
            store_elem(ring, ((int64_t)r * OR_BLOCK + slot) * OR_DIM + d, dtype,
                       load_elem(new_keys, (int64_t)r * OR_DIM + d, dtype));
        if (slot != OR_BLOCK - 1)
            continue;
        double m[OR_DIM];
        for (int d = 0; d < OR_DIM; ++d) {
            float acc = 0.0f;
            for (int i = 0; i < OR_BLOCK; ++i)
                acc += (float)load_elem(ring, ((int64_t)r * OR_BLOCK + i) * OR_DIM + d, dtype);
            m[d] = (double)(acc * 0.25f);
        }
        if (flags & OR_FLAG_POOL_RMSNORM) {
            double ss = 0.0;
            for (int d = 0; d < OR_DIM; ++d)
                ss += m[d] * m[d];
            double inv = 1.0 / sqrt(ss / OR_DIM + 1e-6);
            for (int d = 0; d < OR_DIM; ++d)
                m[d] *= inv;
        }
        if (!(flags & OR_FLAG_NO_ROPE))
            qsa_oracle_rope(m, OR_BLOCK * (t / OR_BLOCK), theta);
        const int64_t cslot = full_slots[r] / OR_BLOCK;
        for (int d = 0; d < OR_DIM; ++d)
            store_elem(compressed, cslot * OR_DIM + d, dtype, m[d]);
    }
    return OR_OK;
}

/*
 * a1-a3 with the compressed key stored in FP8 ("Qwen3.8-Flash-Next, Layer by
 * Layer", section "Serving it": the indexer's keys kept in FP8).  The block
 * is pooled and rotated exactly as qsa_oracle_pool does, the rotated key is
 * rounded to FP32, and one FP32 scale per key carries its range.  Reading
 * (the pages give no scaling): the largest magnitude amax maps to 448, the
 * largest E4M3 value:
 *     inv = 448 / amax, scale = amax / 448    (FP32 quotients)
 *     code_d = E4M3(k_d * inv)                (FP32 product, then nearest-even)
 * and a zero key gets scale 0 and zero codes.  Key element d stands for
 * code_d * scale.
 * raw:    [batch][raw_seq_stride] elements of raw_dtype (as qsa_oracle_pool).
 * codes:  [batch][pooled_seq_stride * 128] bytes, block b at codes + (s*stride + b)*128.
 * scales: [batch][pooled_seq_stride] FP32, block b at scales + s*stride + b.
 */
int qsa_oracle_pool_fp8(const void *raw, int64_t raw_seq_stride, uint8_t *codes, float *scales,
                        int64_t pooled_seq_stride, int32_t batch, int32_t block_begin, int32_t block_end,
                        double theta, uint32_t flags, int32_t raw_dtype)
{
    if (!raw || !codes || !scales || batch < 0 || block_begin < 0 || block_end < block_begin)
        return OR_ERR_ARG;
    int64_t nblk = (int64_t)block_end - block_begin;
    int64_t total = (int64_t)batch * nblk;
#pragma omp parallel for schedule(static)
    for (int64_t w = 0; w < total; ++w) {
        int64_t s = w / nblk;
        int64_t b = block_begin + w % nblk;
        double m[OR_DIM];
        for (int d = 0; d < OR_DIM; ++d) {
            float acc = 0.0f;
            for (int i = 0; i < OR_BLOCK; ++i)
                acc += (float)load_elem(raw, s * raw_seq_stride + (OR_BLOCK * b + i) * OR_DIM + d, raw_dtype);
            m[d] = (double)(acc * 0.25f);
        }
        if (flags & OR_FLAG_POOL_RMSNORM) {
            double ss = 0.0;
            for (int d = 0; d < OR_DIM; ++d)
                ss += m[d] * m[d];
            double inv = 1.0 / sqrt(ss / OR_DIM + 1e-6);
            for (int d = 0; d < OR_DIM; ++d)
                m[d] *= inv;
        }
        if (!(flags & OR_FLAG_NO_ROPE))
            qsa_oracle_rope(m, OR_BLOCK * b, theta);
        float k[OR_DIM];
        float amax = 0.0f;
        for (int d = 0; d < OR_DIM; ++d) {
            k[d] = (float)m[d];
            amax = fabsf(k[d]) > amax ? fabsf(k[d]) : amax;
        }
        const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
        const int64_t slot = s * pooled_seq_stride + b;
        scales[slot] = amax / 448.0f;
        for (int d = 0; d < OR_DIM; ++d) {
            const float v = k[d] * inv;
            codes[slot * OR_DIM + d] = qsa_oracle_fp8_from_double((double)v);
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* a4-a6: query rotation, block scores, top-k selection                      */
/* ------------------------------------------------------------------------ */

/* Complete blocks visible to a query at position t: blocks with 4b+3 <= t. */
static int64_t visible_blocks(int64_t t)
{
    return (t + 1) / OR_BLOCK;
}

typedef struct {
    double raw;
    int32_t block;
} scored_block;

/* Order of [SGL]'s "best" blocks: higher score first; equal scores -> lower
 * block index first (reading: the pages do not say how ties break). */
static int by_score_desc_then_block(const void *pa, const void *pb)
{
    const scored_block *a = (const scored_block *)pa, *b = (const scored_block *)pb;
    if (a->raw > b->raw)
        return -1;
    if (a->raw < b->raw)
        return 1;
    return (a->block > b->block) - (a->block < b->block);
}

static int by_int_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Where the compressed keys come from: `pooled` elements of `dtype`, or FP8
 * codes with one scale per key (see qsa_oracle_pool_fp8). */
typedef struct {
    const void *pooled;
    int dtype;
    const uint8_t *codes;
    const float *scales;
} key_source;

/*
 * [SGL] score equation for one block (key slot `slot` = s*stride + b):
 * sum_h ReLU(<q~_h, kbar_b>), in double precision.  For an FP8 key,
 * kbar_b = code_b * scale_b, and the non-negative scale is taken out of the
 * ReLU: scale_b * sum_h ReLU(<q~_h, code_b>).
 */
static double block_raw(const double q[OR_IDX_HEADS][OR_DIM], const key_source *ks, int64_t slot)
{
    double sum = 0.0;
    for (int h = 0; h < OR_IDX_HEADS; ++h) {
        double dot = 0.0;
        for (int d = 0; d < OR_DIM; ++d) {
            const double k = ks->codes ? qsa_oracle_fp8_to_double(ks->codes[slot * OR_DIM + d])
                                       : load_elem(ks->pooled, slot * OR_DIM + d, ks->dtype);
            dot += q[h][d] * k;
        }
        sum += dot > 0.0 ? dot : 0.0; /* ReLU */
    }
    return ks->codes ? (double)ks->scales[slot] * sum : sum;
}

/*
 * Scores and selection for `rows` query rows.
 *
 * [SGL] score equation:
 *     s_{t,b} = (1/sqrt(128)) * sum_{h=1..4} ReLU(<q^I_{t,h}, kbar^I_b>)
 * over the visible compressed blocks.  The best 512 blocks are kept ([SGL],
 * [LBL]); with fewer visible blocks, all of them ("up to 512").
 *
 * Readings: the index query of row r is rotated at its own position
 * t = row_pos[r] and rounded to the dtype (it is a matrix operand); the
 * selection ranks the un-scaled sum (1/sqrt(128) is a positive constant);
 * ties go to the lower block index; the kept blocks are listed in ascending
 * order and padded with -1.
 *
 * q_index: [rows][4][128] of q_dtype, un-rotated.  `stride` counts keys per
 * sequence.  sel_blocks: [rows][top_k]; sel_count: [rows]; sel_scores
 * ([rows][top_k], may be NULL) gets s_{t,b} of each kept block.  raw_out (may
 * be NULL) gets the un-scaled sum of every visible block:
 * raw_out[r*raw_stride + b].
 */
static int score_topk_core(const void *q_index, int q_dtype, const int32_t *row_seq, const int32_t *row_pos,
                           int32_t rows, const key_source *ks, int64_t stride, int32_t top_k,
                           const double *inv_freq, uint32_t flags, int32_t *sel_blocks, int32_t *sel_count,
                           float *sel_scores, double *raw_out, int64_t raw_stride)
{
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; ++r) {
        int64_t t = row_pos[r];
        int64_t s = row_seq[r];
        int64_t nc = visible_blocks(t);
        double q[OR_IDX_HEADS][OR_DIM];
        for (int h = 0; h < OR_IDX_HEADS; ++h) {
            for (int d = 0; d < OR_DIM; ++d)
                q[h][d] = load_elem(q_index, ((int64_t)r * OR_IDX_HEADS + h) * OR_DIM + d, q_dtype);
            if (!(flags & OR_FLAG_NO_ROPE))
                qsa_oracle_rope_freq(q[h], t, inv_freq);
            for (int d = 0; d < OR_DIM; ++d)
                q[h][d] = round_to_dtype(q[h][d], q_dtype);
        }
        scored_block *all = (scored_block *)malloc(sizeof(scored_block) * (size_t)(nc > 0 ? nc : 1));
        if (!all) {
            failed = 1;
            continue;
        }
        for (int64_t b = 0; b < nc; ++b) {
            const double sum = block_raw(q, ks, s * stride + b);
            all[b].raw = sum;
            all[b].block = (int32_t)b;
            if (raw_out)
                raw_out[(int64_t)r * raw_stride + b] = sum;
        }
        int64_t keep = nc;
        if (nc > top_k) {
            qsort(all, (size_t)nc, sizeof(scored_block), by_score_desc_then_block);
            keep = top_k;
        }
        int32_t *out = sel_blocks + (int64_t)r * top_k;
        for (int64_t i = 0; i < keep; ++i)
            out[i] = all[i].block;
        qsort(out, (size_t)keep, sizeof(int32_t), by_int_asc);
        for (int64_t i = keep; i < top_k; ++i)
            out[i] = -1;
        sel_count[r] = (int32_t)keep;
        if (sel_scores) {
            /* scores of the kept blocks, listed in the same (ascending) order */
            float *so = sel_scores + (int64_t)r * top_k;
            for (int64_t i = 0; i < keep; ++i)
                so[i] = (float)(block_raw(q, ks, s * stride + out[i]) / sqrt((double)OR_DIM));
            for (int64_t i = keep; i < top_k; ++i)
                so[i] = 0.0f;
        }
        free(all);
    }
    return failed ? OR_ERR_ALLOC : OR_OK;
}

/* pooled: see qsa_oracle_pool; pooled_seq_stride counts elements. */
int qsa_oracle_score_topk(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                          int32_t rows, const void *pooled, int64_t pooled_seq_stride,
                          int32_t top_k, double theta, uint32_t flags, int32_t dtype,
                          int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                          double *raw_out, int64_t raw_stride)
{
    if (rows < 0 || top_k < 1 || !q_index || !row_seq || !row_pos || !pooled || !sel_blocks ||
        !sel_count || pooled_seq_stride % OR_DIM)
        return OR_ERR_ARG;
    const key_source ks = {pooled, dtype, NULL, NULL};
    double inv_freq[OR_HALF];
    qsa_oracle_rope_plain_freq(theta, inv_freq);
    return score_topk_core(q_index, dtype, row_seq, row_pos, rows, &ks, pooled_seq_stride / OR_DIM, top_k,
                           inv_freq, flags, sel_blocks, sel_count, sel_scores, raw_out, raw_stride);
}

/* qsa_oracle_score_topk with the index queries rotated by the given pair
 * frequencies (plain RoPE's, or YaRN's from qsa_oracle_yarn_freq): the keys
 * must have been pooled with the same ones. */
int qsa_oracle_score_topk_ex(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                             int32_t rows, const void *pooled, int64_t pooled_seq_stride,
                             int32_t top_k, const double *inv_freq, uint32_t flags, int32_t dtype,
                             int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                             double *raw_out, int64_t raw_stride)
{
    if (rows < 0 || top_k < 1 || !q_index || !row_seq || !row_pos || !pooled || !sel_blocks ||
        !sel_count || !inv_freq || pooled_seq_stride % OR_DIM)
        return OR_ERR_ARG;
    const key_source ks = {pooled, dtype, NULL, NULL};
    return score_topk_core(q_index, dtype, row_seq, row_pos, rows, &ks, pooled_seq_stride / OR_DIM, top_k,
                           inv_freq, flags, sel_blocks, sel_count, sel_scores, raw_out, raw_stride);
}

/* The same with FP8 keys (see qsa_oracle_pool_fp8); pooled_seq_stride counts
 * keys.  The index query stays in q_dtype (the pages put only the stored keys
 * in FP8). */
int qsa_oracle_score_topk_fp8(const void *q_index, int32_t q_dtype, const int32_t *row_seq,
                              const int32_t *row_pos, int32_t rows, const uint8_t *codes, const float *scales,
                              int64_t pooled_seq_stride, int32_t top_k, double theta, uint32_t flags,
                              int32_t *sel_blocks, int32_t *sel_count, float *sel_scores, double *raw_out,
                              int64_t raw_stride)
{
    if (rows < 0 || top_k < 1 || !q_index || !row_seq || !row_pos || !codes || !scales || !sel_blocks ||
        !sel_count)
        return OR_ERR_ARG;
    const key_source ks = {NULL, 0, codes, scales};
    double inv_freq[OR_HALF];
    qsa_oracle_rope_plain_freq(theta, inv_freq);
    return score_topk_core(q_index, q_dtype, row_seq, row_pos, rows, &ks, pooled_seq_stride, top_k, inv_freq,
                           flags, sel_blocks, sel_count, sel_scores, raw_out, raw_stride);
}

/* ------------------------------------------------------------------------ */
/* a7-a9: expansion to token positions, tail, sparse GQA attention           */
/* ------------------------------------------------------------------------ */

/*
 * [SGL]: the kept blocks expand to 4 token positions each ("2048 logical token
 * positions") and the zero-to-three tokens of the current incomplete block are
 * appended, so at most 2051 positions.  For a plain row, the tail is
 * [4*nc(t), t].  [SGL] "IndexShare MTP": draft rows reuse one selection and add
 * the positions drafted since; then the tail starts at the caller's
 * tail_start.  Returns the number of positions written to `pos`.
 */
static int64_t expand_positions(const int32_t *sel, int32_t count, int64_t tail_start, int64_t t,
                                int64_t *pos)
{
    int64_t n = 0;
    for (int32_t i = 0; i < count; ++i)
        for (int j = 0; j < OR_BLOCK; ++j)
            pos[n++] = (int64_t)sel[i] * OR_BLOCK + j;
    for (int64_t p = tail_start; p <= t; ++p)
        pos[n++] = p;
    return n;
}

/*
 * A K or V cache: elements of the query's dtype, or FP8 codes.  Reading for
 * the FP8 KV cache of [LBL] "Serving it" (the page names neither the variant
 * nor the scaling): OCP E4M3 codes with one FP32 scale per cache tensor (one
 * for K, one for V); an element's value is scale * E4M3(code), in double.
 */
enum { OR_KV_FP8 = 2 };
typedef struct {
    const void *ptr;
    int dtype;       /* OR_F32, OR_BF16 or OR_KV_FP8 */
    double scale;    /* OR_KV_FP8 only */
} kv_src;

static double load_kv(const kv_src *c, int64_t idx)
{
    if (c->dtype == OR_KV_FP8)
        return c->scale * qsa_oracle_fp8_to_double(((const uint8_t *)c->ptr)[idx]);
    return load_elem(c->ptr, idx, c->dtype);
}

/*
 * Softmax attention of one query head over the listed positions, on the
 * original K/V ([SGL]: "the compressed keys are only an index").  GQA reading:
 * query head h uses KV head floor(h / (Hq/Hkv)).  Max-subtracted softmax in
 * double; lse = max + log(sum exp).
 */
static void attend_one_head(const void *qrow, int64_t qoff, const kv_src *k_cache,
                            const kv_src *v_cache, int64_t kv_base, int32_t Hkv, int32_t g, int32_t D,
                            const int64_t *pos, int64_t n, double scale, int32_t dtype, void *out,
                            int64_t ooff, float *lse_out, double *logit)
{
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
        int64_t koff = kv_base + (pos[i] * Hkv + g) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += load_elem(qrow, qoff + d, dtype) * load_kv(k_cache, koff + d);
        logit[i] = scale * dot;
        if (logit[i] > mx)
            mx = logit[i];
    }
    double denom = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        logit[i] = exp(logit[i] - mx);
        denom += logit[i];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            int64_t voff = kv_base + (pos[i] * Hkv + g) * D;
            acc += logit[i] * load_kv(v_cache, voff + d);
        }
        store_elem(out, ooff + d, dtype, acc / denom);
    }
    if (lse_out)
        *lse_out = (float)(mx + log(denom));
}

/*
 * a7+a8, prefill: row r (sequence row_seq[r], position t = row_pos[r]) attends
 * its own selection sel_blocks[r][0..sel_count[r]) expanded to tokens, plus the
 * tail [4*nc(t), t].
 * q: [rows][Hq][D]; k_cache, v_cache: [B][kv_seq_stride], token p of sequence
 * s, KV head g at s*kv_seq_stride + (p*Hkv + g)*D; out: [rows][Hq][D];
 * lse: [rows][Hq] or NULL.
 */
static int attn_prefill(const void *q, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                        const kv_src *k_cache, const kv_src *v_cache, int64_t kv_seq_stride,
                        const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k, int32_t Hq,
                        int32_t Hkv, int32_t D, double softmax_scale, int32_t dtype, void *out, float *lse)
{
    if (rows < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || top_k < 1 || !q || !row_seq ||
        !row_pos || !k_cache->ptr || !v_cache->ptr || !sel_blocks || !sel_count || !out)
        return OR_ERR_ARG;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; ++r) {
        int64_t t = row_pos[r];
        int64_t cap = (int64_t)OR_BLOCK * top_k + OR_BLOCK;
        int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
        double *logit = (double *)malloc(sizeof(double) * (size_t)cap);
        if (!pos || !logit) {
            free(pos);
            free(logit);
            failed = 1;
            continue;
        }
        int64_t n = expand_positions(sel_blocks + (int64_t)r * top_k, sel_count[r],
                                     OR_BLOCK * visible_blocks(t), t, pos);
        int64_t kv_base = (int64_t)row_seq[r] * kv_seq_stride;
        for (int32_t h = 0; h < Hq; ++h) {
            int32_t g = h / (Hq / Hkv);
            int64_t qo = ((int64_t)r * Hq + h) * D;
            attend_one_head(q, qo, k_cache, v_cache, kv_base, Hkv, g, D, pos, n, softmax_scale,
                            dtype, out, qo, lse ? &lse[(int64_t)r * Hq + h] : NULL, logit);
        }
        free(pos);
        free(logit);
    }
    return failed ? OR_ERR_ALLOC : OR_OK;
}

int qsa_oracle_sparse_attn_prefill(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                   int32_t rows, const void *k_cache, const void *v_cache,
                                   int64_t kv_seq_stride, const int32_t *sel_blocks,
                                   const int32_t *sel_count, int32_t top_k, int32_t Hq, int32_t Hkv,
                                   int32_t D, double softmax_scale, int32_t dtype, void *out,
                                   float *lse)
{
    kv_src k = {k_cache, dtype, 1.0}, v = {v_cache, dtype, 1.0};
    return attn_prefill(q, row_seq, row_pos, rows, &k, &v, kv_seq_stride, sel_blocks, sel_count, top_k, Hq,
                        Hkv, D, softmax_scale, dtype, out, lse);
}

/*
 * The same with an FP8 K/V cache: E4M3 codes, k_scale and v_scale (see
 * kv_src); q, out in q_dtype.
 */
int qsa_oracle_sparse_attn_prefill_fp8kv(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                         int32_t rows, const uint8_t *k_codes, const uint8_t *v_codes,
                                         int64_t kv_seq_stride, double k_scale, double v_scale,
                                         const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k,
                                         int32_t Hq, int32_t Hkv, int32_t D, double softmax_scale,
                                         int32_t q_dtype, void *out, float *lse)
{
    kv_src k = {k_codes, OR_KV_FP8, k_scale}, v = {v_codes, OR_KV_FP8, v_scale};
    return attn_prefill(q, row_seq, row_pos, rows, &k, &v, kv_seq_stride, sel_blocks, sel_count, top_k, Hq,
                        Hkv, D, softmax_scale, q_dtype, out, lse);
}

/*
 * a7+a9, decode: q_per_seq rows per sequence share that sequence's selection
 * sel_blocks[s] ([SGL] "IndexShare MTP").  Row j of sequence s sits at
 * row_pos[s][j] and attends the selection plus the positions
 * [tail_start[s], row_pos[s][j]].  tail_start == NULL means 4*nc(row_pos) for
 * each row (a plain decode row).
 * q, out: [batch][q_per_seq][Hq][D]; lse: [batch][q_per_seq][Hq] or NULL.
 */
static int attn_decode(const void *q, const int32_t *row_pos, int32_t batch, int32_t q_per_seq,
                       const int32_t *tail_start, const kv_src *k_cache, const kv_src *v_cache,
                       int64_t kv_seq_stride, const int32_t *sel_blocks, const int32_t *sel_count,
                       int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D, double softmax_scale, int32_t dtype,
                       void *out, float *lse)
{
    if (batch < 0 || q_per_seq < 1 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || top_k < 1 ||
        !q || !row_pos || !k_cache->ptr || !v_cache->ptr || !sel_blocks || !sel_count || !out)
        return OR_ERR_ARG;
    int64_t rows = (int64_t)batch * q_per_seq;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t s = r / q_per_seq;
        int64_t t = row_pos[r];
        int64_t ts = tail_start ? (int64_t)tail_start[s] : OR_BLOCK * visible_blocks(t);
        int64_t tail_n = t >= ts ? t - ts + 1 : 0;
        int64_t cap = (int64_t)OR_BLOCK * top_k + tail_n + 1;
        int64_t *pos = (int64_t *)malloc(sizeof(int64_t) * (size_t)cap);
        double *logit = (double *)malloc(sizeof(double) * (size_t)cap);
        if (!pos || !logit) {
            free(pos);
            free(logit);
            failed = 1;
            continue;
        }
        int64_t n = expand_positions(sel_blocks + s * top_k, sel_count[s], ts, t, pos);
        int64_t kv_base = s * kv_seq_stride;
        for (int32_t h = 0; h < Hq; ++h) {
            int32_t g = h / (Hq / Hkv);
            int64_t qo = (r * Hq + h) * D;
            attend_one_head(q, qo, k_cache, v_cache, kv_base, Hkv, g, D, pos, n, softmax_scale,
                            dtype, out, qo, lse ? &lse[r * Hq + h] : NULL, logit);
        }
        free(pos);
        free(logit);
    }
    return failed ? OR_ERR_ALLOC : OR_OK;
}

int qsa_oracle_sparse_attn_decode(const void *q, const int32_t *row_pos, int32_t batch,
                                  int32_t q_per_seq, const int32_t *tail_start,
                                  const void *k_cache, const void *v_cache, int64_t kv_seq_stride,
                                  const int32_t *sel_blocks, const int32_t *sel_count,
                                  int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D,
                                  double softmax_scale, int32_t dtype, void *out, float *lse)
{
    kv_src k = {k_cache, dtype, 1.0}, v = {v_cache, dtype, 1.0};
    return attn_decode(q, row_pos, batch, q_per_seq, tail_start, &k, &v, kv_seq_stride, sel_blocks, sel_count,
                       top_k, Hq, Hkv, D, softmax_scale, dtype, out, lse);
}

/* The same with an FP8 K/V cache (see kv_src). */
int qsa_oracle_sparse_attn_decode_fp8kv(const void *q, const int32_t *row_pos, int32_t batch,
                                        int32_t q_per_seq, const int32_t *tail_start, const uint8_t *k_codes,
                                        const uint8_t *v_codes, int64_t kv_seq_stride, double k_scale,
                                        double v_scale, const int32_t *sel_blocks, const int32_t *sel_count,
                                        int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D,
                                        double softmax_scale, int32_t q_dtype, void *out, float *lse)
{
    kv_src k = {k_codes, OR_KV_FP8, k_scale}, v = {v_codes, OR_KV_FP8, v_scale};
    return attn_decode(q, row_pos, batch, q_per_seq, tail_start, &k, &v, kv_seq_stride, sel_blocks, sel_count,
                       top_k, Hq, Hkv, D, softmax_scale, q_dtype, out, lse);
}

/* Threads the OpenMP loops above will use (reported by the CPU baseline). */
int qsa_oracle_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
