// attn.hip -- steps a7-a9: expansion of the kept blocks to token positions,
// the incomplete tail block, and softmax attention on the original K/V.
//
// "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
// Attention": each kept block stands for its 4 token positions (512 blocks =
// 2048 positions), the zero-to-three tokens of the query's incomplete block
// are appended (at most 2051 positions), and attention reads the original,
// uncompressed K/V at those positions -- the compressed keys only index.
// Section "IndexShare MTP": draft rows reuse one selection and add the
// positions drafted since it was taken (`tail_start`).
// Readings: query head h uses KV head floor(h / (Hq/Hkv)); logits are
// softmax_scale * <q, k>.
//
// A workgroup owns one "query group": the query heads that share one KV head
// g, for every query row that shares one selection (prefill: one row; decode:
// the Qn rows of a sequence).  It walks the group's positions in chunks of 64:
// gather K and V rows of the chunk into LDS (fp32), logits for every (query,
// position), an online-softmax update, then P.V.  Prefill walks all chunks
// and writes the output; decode gives each chunk of the selection its own
// workgroup (split) and a combine kernel merges the partial softmaxes.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

constexpr int kAC = kAttnChunk;   // positions per chunk
// LDS row stride of K: 16-byte rows, and 4 banks of skew per row, so the 16
// lanes of a quarter-wave reading 16 bytes each of 16 rows hit all 64 banks once
constexpr int kKPad = kDim + 4;

template <typename T, int MAXQ>
struct alignas(16) AttnSmem {
    float q[MAXQ][kDim];
    float k[kAC][kKPad];
    float v[kAC][kDim];
    float w[MAXQ][kAC];
    float m[MAXQ], l[MAXQ], alpha[MAXQ];
    int32_t lo[MAXQ], hi[MAXQ];  // per-query admissible tail range [lo, hi]
    int64_t pos[kAC];
};

// One chunk: positions pos[0..n) (n <= 64) from the selection (every query
// admits them) or from the tail (query qi admits lo[qi] <= p <= hi[qi]).
template <typename T, int MAXQ>
__device__ __forceinline__ void attn_chunk(AttnSmem<T, MAXQ> &sm, const T *__restrict__ kbase,
                                           const T *__restrict__ vbase, int64_t row_stride, int n, bool tail,
                                           int nq, float scale, float (&o)[MAXQ / 2])
{
    const int t = threadIdx.x;
    // gather K/V rows: thread t -> row t/4, dims [32*(t%4), +32); every load of
    // the thread is issued before its LDS stores, which are 16 bytes each
    {
        const int p = t >> 2, d0 = (t & 3) * 32;
        if (p < n) {
            const T *ks = kbase + sm.pos[p] * row_stride + d0;
            const T *vs = vbase + sm.pos[p] * row_stride + d0;
            float kf[32], vf[32];
#pragma unroll
            for (int i = 0; i < 32; i += 8) {
                load8(ks + i, kf + i);
                load8(vs + i, vf + i);
            }
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                *(float4 *)&sm.k[p][d0 + i] = make_float4(kf[i], kf[i + 1], kf[i + 2], kf[i + 3]);
                *(float4 *)&sm.v[p][d0 + i] = make_float4(vf[i], vf[i + 1], vf[i + 2], vf[i + 3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; i += 4) {
                *(float4 *)&sm.k[p][d0 + i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                *(float4 *)&sm.v[p][d0 + i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
    }
    __syncthreads();
    // logits: lane -> position p, wave w -> queries w, w+4, ...; four dims per
    // LDS read, summed in dim order
    {
        const int p = t & 63, w = t >> 6;
        float acc[MAXQ / 4];
#pragma unroll
        for (int i = 0; i < MAXQ / 4; ++i) acc[i] = 0.0f;
#pragma unroll 4
        for (int d = 0; d < kDim; d += 4) {
            const float4 kv = *(const float4 *)&sm.k[p][d];
#pragma unroll
            for (int i = 0; i < MAXQ / 4; ++i) {
                const float4 qv = *(const float4 *)&sm.q[w + 4 * i][d];
                acc[i] = fmaf(kv.x, qv.x, acc[i]);
                acc[i] = fmaf(kv.y, qv.y, acc[i]);
                acc[i] = fmaf(kv.z, qv.z, acc[i]);
                acc[i] = fmaf(kv.w, qv.w, acc[i]);
            }
        }
        const int64_t pp = sm.pos[p < n ? p : 0];
#pragma unroll
        for (int i = 0; i < MAXQ / 4; ++i) {
            const int qi = w + 4 * i;
            if (qi >= nq) break;  // wave-uniform
            bool ok = p < n;
            if (tail) ok = ok && pp >= sm.lo[qi] && pp <= sm.hi[qi];
            const float s = ok ? acc[i] * scale : -INFINITY;
            const float cmax = wave_max(s);
            const float m_old = sm.m[qi];
            const float m_new = fmaxf(m_old, cmax);
            float e = 0.0f, alpha = 1.0f;
            if (m_new != -INFINITY) {
                e = ok ? __expf(s - m_new) : 0.0f;
                alpha = m_old == -INFINITY ? 0.0f : __expf(m_old - m_new);
            }
            const float esum = wave_sum(e);
            sm.w[qi][p] = e;
            // query qi belongs to this wave alone, and a wave's LDS accesses
            // complete in program order: every lane has read m/l above
            if (p == 0) {
                sm.l[qi] = sm.l[qi] * alpha + esum;
                sm.m[qi] = m_new;
                sm.alpha[qi] = alpha;
            }
        }
    }
    __syncthreads();
    // P.V: thread -> dim d, half h2 -> queries h2, h2+2, ...; the weights of
    // four positions per LDS read (past position n both the weights and V are
    // 0, so the last group of four adds exact zeros)
    {
        const int d = t & 127, h2 = t >> 7;
#pragma unroll
        for (int i = 0; i < MAXQ / 2; ++i) {
            const int qi = h2 + 2 * i;
            if (qi < nq) o[i] *= sm.alpha[qi];
        }
#pragma unroll 2
        for (int p = 0; p < n; p += 4) {
            const float v0 = sm.v[p][d], v1 = sm.v[p + 1][d], v2 = sm.v[p + 2][d], v3 = sm.v[p + 3][d];
#pragma unroll
            for (int i = 0; i < MAXQ / 2; ++i) {
                const float4 wv = *(const float4 *)&sm.w[h2 + 2 * i][p];
                o[i] = fmaf(wv.x, v0, o[i]);
                o[i] = fmaf(wv.y, v1, o[i]);
                o[i] = fmaf(wv.z, v2, o[i]);
                o[i] = fmaf(wv.w, v3, o[i]);
            }
        }
    }
    __syncthreads();
}

// Grid: x = split (decode) or 0 (prefill), y = query group (sel index * Hkv + g).
template <typename T, int MAXQ, bool SPLIT>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a)
{
    __shared__ AttnSmem<T, MAXQ> sm;
    const int t = threadIdx.x;
    const int64_t grp = blockIdx.y;
    const int64_t sidx = grp / a.Hkv;           // selection index (prefill row / decode sequence)
    const int g = (int)(grp % a.Hkv);           // KV head
    const int hg = a.Hq / a.Hkv;                // query heads per KV head
    const int nq = a.q_per_sel * hg;
    const int64_t seq = SPLIT ? sidx : (int64_t)a.row_seq[sidx];
    const int32_t count = min(a.sel_count[sidx], a.top_k);
    const int32_t *sel = a.sel_blocks + sidx * a.top_k;
    const int split = blockIdx.x;
    // queries of the group, their admissible tail range, softmax state
    int32_t tail_lo = INT32_MAX, tail_hi = -1;
    for (int qi = 0; qi < nq; ++qi) {
        const int j = qi / hg;
        const int32_t tj = a.row_pos[sidx * a.q_per_sel + j];
        const int32_t ts = a.tail_start ? a.tail_start[sidx] : (int32_t)(kBlock * visible_blocks(tj));
        tail_lo = min(tail_lo, ts);
        tail_hi = max(tail_hi, tj);
        if (t == 0) {
            sm.lo[qi] = ts;
            sm.hi[qi] = tj;
            sm.m[qi] = -INFINITY;
            sm.l[qi] = 0.0f;
        }
    }
    for (int i = t; i < nq * kDim; i += blockDim.x) {
        const int qi = i / kDim, d = i % kDim;
        const int j = qi / hg, h = g * hg + qi % hg;
        const T *qp = (const T *)a.q + ((sidx * a.q_per_sel + j) * (int64_t)a.Hq + h) * kDim;
        sm.q[qi][d] = load_f32(qp + d);
    }
    for (int i = nq * kDim + t; i < MAXQ * kDim; i += blockDim.x) sm.q[i / kDim][i % kDim] = 0.0f;
    __syncthreads();
    float o[MAXQ / 2];
#pragma unroll
    for (int i = 0; i < MAXQ / 2; ++i) o[i] = 0.0f;
    const T *kbase = (const T *)a.k_cache + seq * a.kv_seq_stride + (int64_t)g * kDim;
    const T *vbase = (const T *)a.v_cache + seq * a.kv_seq_stride + (int64_t)g * kDim;
    const int64_t row_stride = (int64_t)a.Hkv * kDim;
    const int32_t n_sel_chunks = (kBlock * count + kAC - 1) / kAC;
    // the kept blocks, 16 per chunk
    const int32_t c_lo = SPLIT ? split : 0;
    const int32_t c_hi = SPLIT ? (split < a.nsplit - 1 ? min(split + 1, n_sel_chunks) : 0) : n_sel_chunks;
    for (int32_t c = c_lo; c < c_hi; ++c) {
        const int n = min(kAC, kBlock * count - c * kAC);
        if (t < kAC) sm.pos[t] = t < n ? (int64_t)sel[c * (kAC / kBlock) + t / kBlock] * kBlock + (t % kBlock) : 0;
        __syncthreads();
        attn_chunk<T, MAXQ>(sm, kbase, vbase, row_stride, n, false, nq, a.scale, o);
    }
    // the tail: positions [min lo, max hi], masked per query
    if (!SPLIT || split == a.nsplit - 1) {
        for (int64_t p0 = tail_lo; p0 <= tail_hi; p0 += kAC) {
            const int n = (int)min((int64_t)kAC, (int64_t)tail_hi - p0 + 1);
            if (t < kAC) sm.pos[t] = t < n ? p0 + t : 0;
            __syncthreads();
            attn_chunk<T, MAXQ>(sm, kbase, vbase, row_stride, n, true, nq, a.scale, o);
        }
    }
    // results
    const int d = t & 127, h2 = t >> 7;
#pragma unroll
    for (int i = 0; i < MAXQ / 2; ++i) {
        const int qi = h2 + 2 * i;
        if (qi >= nq) break;
        const int j = qi / hg, h = g * hg + qi % hg;
        const int64_t qrow = (sidx * a.q_per_sel + j) * (int64_t)a.Hq + h;  // [row][head]
        const float m = sm.m[qi], l = sm.l[qi];
        if (SPLIT) {
            float *pp = a.partial + (qrow * a.nsplit + split) * (kDim + 2);
            pp[d] = o[i];
            if (d == 0) {
                pp[kDim] = m;
                pp[kDim + 1] = l;
            }
        } else {
            store_f32((T *)a.out + qrow * kDim + d, l > 0.0f ? o[i] / l : 0.0f);
            if (a.lse && d == 0) a.lse[qrow] = l > 0.0f ? m + __logf(l) : -INFINITY;
        }
    }
}

// Merge the decode splits of one (row, head): grid = rows*Hq, DIM threads.
// Wave 0 reduces the splits' (m, l) with one split per lane; then every thread
// owns one output dim and sums the splits' weighted partial outputs, several
// loads in flight at once.
constexpr int kMaxDecodeSplits = (kBlock * QSA_MAX_TOP_K + kAC - 1) / kAC + 1;

template <typename T, int DIM>
__global__ __launch_bounds__(DIM) void attn_combine_kernel(const float *__restrict__ partial, int32_t nsplit,
                                                           void *out, float *lse)
{
    __shared__ float wsplit[kMaxDecodeSplits];
    __shared__ float s_m, s_l;
    const int64_t qrow = blockIdx.x;
    const int d = threadIdx.x;
    const float *pp = partial + qrow * nsplit * (DIM + 2);
    // the first kPre splits' values, read up front (clamped, so every read is
    // in the row and none needs a guard) while wave 0 forms the weights: the
    // reads do not depend on them
    constexpr int kPre = 48;
    float pv[kPre];
#pragma unroll
    for (int j = 0; j < kPre; ++j) pv[j] = pp[min(j, nsplit - 1) * (DIM + 2) + d];
    if (d < kWave) {
        // each lane's first split's (m, l) is read once and kept for both passes
        const float m0 = d < nsplit ? pp[d * (DIM + 2) + DIM] : -INFINITY;
        const float l0 = d < nsplit ? pp[d * (DIM + 2) + DIM + 1] : 0.0f;
        float m = m0;
        for (int s = d + kWave; s < nsplit; s += kWave) m = fmaxf(m, pp[s * (DIM + 2) + DIM]);
        m = wave_max(m);
        float l = 0.0f;
        if (d < nsplit) {
            const float e = m0 == -INFINITY ? 0.0f : __expf(m0 - m);
            wsplit[d] = e;
            l = l0 * e;
        }
        for (int s = d + kWave; s < nsplit; s += kWave) {
            const float ms = pp[s * (DIM + 2) + DIM];
            const float e = ms == -INFINITY ? 0.0f : __expf(ms - m);
            wsplit[s] = e;
            l += pp[s * (DIM + 2) + DIM + 1] * e;
        }
        l = wave_sum(l);
        if (d == 0) {
            s_m = m;
            s_l = l;
        }
    }
    __syncthreads();
    const float M = s_m, L = s_l;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (L > 0.0f) {
#pragma unroll
        for (int j = 0; j < kPre; ++j) acc[j & 3] += (j < nsplit ? wsplit[j] : 0.0f) * pv[j];
        int s = kPre;
        for (; s + 4 <= nsplit; s += 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += wsplit[s + j] * pp[(s + j) * (DIM + 2) + d];
        }
        for (; s < nsplit; ++s) acc[0] += wsplit[s] * pp[s * (DIM + 2) + d];
    }
    const float o = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    store_f32((T *)out + qrow * DIM + d, L > 0.0f ? o / L : 0.0f);
    if (lse && d == 0) lse[qrow] = L > 0.0f ? M + __logf(L) : -INFINITY;
}

int32_t attn_decode_splits(int32_t top_k) { return (kBlock * top_k + kAC - 1) / kAC + 1; }

void launch_attn_prefill(const AttnArgs &a, bool bf16, hipStream_t stream)
{
    const dim3 grid(1, (unsigned)((int64_t)a.n_sel * a.Hkv)), block(256);
    const int nq = a.q_per_sel * (a.Hq / a.Hkv);
    if (nq <= 8) {
        if (bf16) QSA_LAUNCH("attn_prefill", (attn_kernel<bf16_t, 8, false>), grid, block, 0, stream, a);
        else QSA_LAUNCH("attn_prefill", (attn_kernel<float, 8, false>), grid, block, 0, stream, a);
    } else if (nq <= 16) {
        if (bf16) QSA_LAUNCH("attn_prefill", (attn_kernel<bf16_t, 16, false>), grid, block, 0, stream, a);
        else QSA_LAUNCH("attn_prefill", (attn_kernel<float, 16, false>), grid, block, 0, stream, a);
    } else {
        if (bf16) QSA_LAUNCH("attn_prefill", (attn_kernel<bf16_t, kAttnMaxQ, false>), grid, block, 0, stream, a);
        else QSA_LAUNCH("attn_prefill", (attn_kernel<float, kAttnMaxQ, false>), grid, block, 0, stream, a);
    }
}

void launch_attn_decode(const AttnArgs &a, bool bf16, hipStream_t stream)
{
    const dim3 grid((unsigned)a.nsplit, (unsigned)((int64_t)a.n_sel * a.Hkv)), block(256);
    const int nq = a.q_per_sel * (a.Hq / a.Hkv);
    if (nq <= 8) {
        if (bf16) QSA_LAUNCH("attn_decode", (attn_kernel<bf16_t, 8, true>), grid, block, 0, stream, a);
        else QSA_LAUNCH("attn_decode", (attn_kernel<float, 8, true>), grid, block, 0, stream, a);
    } else if (nq <= 16) {
        if (bf16) QSA_LAUNCH("attn_decode", (attn_kernel<bf16_t, 16, true>), grid, block, 0, stream, a);
        else QSA_LAUNCH("attn_decode", (attn_kernel<float, 16, true>), grid, block, 0, stream, a);
    } else {
        if (bf16) QSA_LAUNCH("attn_decode", (attn_kernel<bf16_t, kAttnMaxQ, true>), grid, block, 0, stream, a);
        else QSA_LAUNCH("attn_decode", (attn_kernel<float, kAttnMaxQ, true>), grid, block, 0, stream, a);
    }
    launch_attn_combine(a, bf16, stream);
}

void launch_attn_combine(const AttnArgs &a, bool bf16, hipStream_t stream)
{
    const int64_t qrows = (int64_t)a.n_sel * a.q_per_sel * a.Hq;
    const dim3 grid((unsigned)qrows);
    if (a.D == 256)  // the bf16 MFMA path's head dim
        QSA_LAUNCH("attn_combine", (attn_combine_kernel<bf16_t, 256>), grid, dim3(256), 0, stream, a.partial,
                   a.nsplit, a.out, a.lse);
    else if (bf16)
        QSA_LAUNCH("attn_combine", (attn_combine_kernel<bf16_t, kDim>), grid, dim3(kDim), 0, stream, a.partial,
                   a.nsplit, a.out, a.lse);
    else
        QSA_LAUNCH("attn_combine", (attn_combine_kernel<float, kDim>), grid, dim3(kDim), 0, stream, a.partial,
                   a.nsplit, a.out, a.lse);
}

}  // namespace qsa
