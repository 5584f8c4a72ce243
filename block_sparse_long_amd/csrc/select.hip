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
#include "qsa_wg.h"

namespace qsa {

constexpr int kSelThreads = 512;
constexpr int kSplitThreads = 256;
constexpr int kCollectChunk = 4096;  // blocks per collect workgroup
constexpr int kCandStage = 3072;     // candidates the final pass keeps in LDS
constexpr int kEmitWords = 8192;     // bitmap window of the final pass: 262,144 blocks
// Word w of the final pass's bitmap sits at w + w/32, so the 64 lanes of a
// wave walking their own runs of 32 words hit distinct LDS banks.
constexpr int kEmitSlots = kEmitWords + kEmitWords / 32;
__device__ __forceinline__ int emit_slot(int w) { return w + (w >> 5); }
// u16 count of word w: 2 slots of padding per 32 words, so the threads writing
// their runs of 32 hit distinct banks
__device__ __forceinline__ int emit_pre_slot(int w) { return w + 2 * (w >> 5); }

// Reported score s = raw / sqrt(128) (the score equation's scale), divided in
// double and rounded once to float.
__device__ __forceinline__ float scaled_score(float raw) { return (float)((double)raw / sqrt((double)kDim)); }

__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(const float *__restrict__ scores, int64_t sc_stride,
                                                                  const int32_t *__restrict__ row_pos, int32_t max_nb,
                                                                  int32_t top_k,
                                                                  int32_t *__restrict__ sel_blocks,
                                                                  int32_t *__restrict__ sel_count,
                                                                  float *__restrict__ sel_scores)
{
    __shared__ uint32_t hist[4096];
    __shared__ uint32_t wtot[kSelThreads / kWave];
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
        find_bin<kSelThreads>(hist, nbins, need, wtot, &s_bin, &s_above);
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
        const uint32_t eq_rank = eq_before + wg_rank<kSelThreads>(eq, wtot, eq_total);
        const bool take = gt || (eq && eq_rank < need);
        const uint32_t pos = out_before + wg_rank<kSelThreads>(take, wtot, take_total);
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

// ---------------------------------------------------------------------------
// Few rows, many blocks: the selection split over many workgroups.
//   - the scorer has filled the row's 12-bit key histogram;
//   - collect (grid: chunks of 4096 blocks x rows): every workgroup finds the
//     bin b* holding the k-th best key, gathers the blocks of its chunk above
//     b* ("sure") and inside b* (candidates) in LDS, then reserves room in
//     the row's two global lists with one atomic each and copies them out;
//   - final (one workgroup per row, a second launch): picks the missing
//     `need` entries among the candidates with a radix select on the unique
//     composite (low 20 key bits, ~block) -- a higher score first, then the
//     lower block -- and writes the kept set sorted by block id.
// ---------------------------------------------------------------------------
// Append the wave's `pred` items to an LDS list (slot `base + i`, or
// `base - i` when `down`): one LDS atomic per wave.
__device__ __forceinline__ void wave_append_lds(bool pred, uint2 item, uint32_t *counter, uint2 *list, uint32_t base,
                                                bool down)
{
    const uint64_t mask = __ballot(pred);
    if (!mask) return;
    const int lane = threadIdx.x & 63;
    const uint32_t n = (uint32_t)__popcll(mask);
    const int leader = __ffsll((unsigned long long)mask) - 1;
    uint32_t off = 0;
    if (lane == leader) off = atomicAdd(counter, n);
    off = __shfl(off, leader) + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
    if (pred) list[down ? base - off : base + off] = item;
}

__device__ __forceinline__ uint64_t composite20(uint2 e)
{
    return ((uint64_t)(e.x & 0x000fffffu) << 32) | (uint64_t)(~e.y);
}

// find_bin over a row's 4096-bin histogram in global memory: thread t owns
// bins [4080 - 16t, 4096 - 16t), read with four 16-byte loads issued together
// and kept in registers for the search inside the owning thread.
__device__ __forceinline__ void find_bin_global(const uint32_t *__restrict__ hist, uint32_t need, uint32_t *wtot,
                                                uint32_t *out_bin, uint32_t *out_above)
{
    static_assert(kHistBins == 16 * kSplitThreads, "16 bins per thread");
    const int lo = kHistBins - 16 * ((int)threadIdx.x + 1);
    uint4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = ((const uint4 *)(hist + lo))[j];
    const uint32_t c[16] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w,
                            q[2].x, q[2].y, q[2].z, q[2].w, q[3].x, q[3].y, q[3].z, q[3].w};
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[i];
    const uint32_t incl = wg_inclusive_scan<kSplitThreads>(sum, wtot);
    const uint32_t before = incl - sum;
    if (before < need && incl >= need) {
        uint32_t acc = before;
        for (int i = 15; i >= 0; --i) {
            if (acc + c[i] >= need) {
                *out_bin = (uint32_t)(lo + i);
                *out_above = acc;
                break;
            }
            acc += c[i];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kSplitThreads) void select_collect_kernel(
    const float *__restrict__ scores, int64_t sc_stride, const int32_t *__restrict__ row_pos, int32_t max_nb,
    int32_t top_k, SplitSelect ss, int32_t *__restrict__ sel_blocks, int32_t *__restrict__ sel_count,
    float *__restrict__ sel_scores)
{
    __shared__ uint32_t wtot[kSplitThreads / kWave];
    __shared__ uint32_t s_bin, s_above;
    // the chunk's sure entries grow from the front, its candidates from the
    // back: together at most one per block of the chunk
    __shared__ uint2 st[kCollectChunk];
    __shared__ uint32_t s_n[2], s_base[2];
    const int t = threadIdx.x;
    const int64_t r = blockIdx.y;
    const int32_t nc = (int32_t)min(visible_blocks(row_pos[r]), (int64_t)max_nb);
    const int32_t kk = min(top_k, nc);
    const float *srow = scores + r * sc_stride;
    int32_t *out = sel_blocks + r * top_k;
    float *osc = sel_scores ? sel_scores + r * top_k : nullptr;
    uint32_t *hist = ss.scratch + r * kRowScratch;
    uint32_t *cnt = hist + kHistBins;
    uint2 *sure = ss.sure + r * top_k;
    uint2 *cand = ss.cand + r * ss.cand_stride;
    const int64_t b_begin = (int64_t)blockIdx.x * kCollectChunk;
    if (nc <= top_k) {  // every visible block is kept: one workgroup writes the row
        if (blockIdx.x != 0) return;
        if (t == 0) sel_count[r] = kk;
        for (int32_t i = t; i < top_k; i += kSplitThreads) {
            out[i] = i < nc ? i : -1;
            if (osc) osc[i] = i < nc ? scaled_score(srow[i]) : 0.0f;
        }
        return;
    }
    if (b_begin >= nc) return;
    if (t < 2) s_n[t] = 0u;
    // ---- collect ----
    // the whole chunk in flight at once, issued before the histogram search:
    // thread t holds blocks b_begin + 1024*j + 4*t + i (rows are padded to 64
    // floats, so a 4-block group that starts inside the row ends inside it)
    const int64_t b_end = min((int64_t)nc, b_begin + kCollectChunk);
    // a group past the chunk's end reads the last group inside it instead
    // (every load stays in the row, none needs a guard, so all are issued
    // together); its entries are masked below
    const int64_t b_last4 = (b_end - 1) & ~(int64_t)3;
    float4 v[kCollectChunk / (4 * kSplitThreads)];
#pragma unroll
    for (int j = 0; j < kCollectChunk / (4 * kSplitThreads); ++j) {
        const int64_t b4 = b_begin + (int64_t)j * 4 * kSplitThreads + 4 * t;
        v[j] = *(const float4 *)(srow + min(b4, b_last4));
    }
    find_bin_global(hist, (uint32_t)kk, wtot, &s_bin, &s_above);
    const uint32_t beta = s_bin;
#pragma unroll
    for (int j = 0; j < kCollectChunk / (4 * kSplitThreads); ++j) {
        const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t b = b_begin + (int64_t)j * 4 * kSplitThreads + 4 * t + i;
            const bool valid = b < b_end;
            const uint32_t key = valid ? score_key(e[i]) : 0u;
            const uint32_t bin = key >> kHistShift;
            const uint2 item = make_uint2(key, (uint32_t)b);
            wave_append_lds(valid && bin > beta, item, &s_n[0], st, 0u, false);
            wave_append_lds(valid && bin == beta, item, &s_n[1], st, kCollectChunk - 1u, true);
        }
    }
    __syncthreads();
    const uint32_t n_sure = s_n[0], n_cand = s_n[1];
    if (t == 0) s_base[0] = n_sure ? atomicAdd(&cnt[0], n_sure) : 0u;
    if (t == kWave) s_base[1] = n_cand ? atomicAdd(&cnt[1], n_cand) : 0u;
    __syncthreads();
    for (uint32_t i = t; i < n_sure; i += kSplitThreads) sure[s_base[0] + i] = st[i];
    for (uint32_t i = t; i < n_cand; i += kSplitThreads) cand[s_base[1] + i] = st[kCollectChunk - 1u - i];
}

// One workgroup per row: picks the missing `need` entries among the row's
// candidates and writes the kept set sorted by block id.
__global__ __launch_bounds__(kSplitThreads) void select_final_kernel(
    const float *__restrict__ scores, int64_t sc_stride, const int32_t *__restrict__ row_pos, int32_t max_nb,
    int32_t top_k, SplitSelect ss, int32_t *__restrict__ sel_blocks, int32_t *__restrict__ sel_count,
    float *__restrict__ sel_scores)
{
    __shared__ uint64_t buf[QSA_MAX_TOP_K];
    __shared__ uint2 cst[kCandStage];
    __shared__ uint32_t bm[kEmitSlots];
    __shared__ uint32_t dhist[256];
    __shared__ uint32_t wtot[kSplitThreads / kWave];
    __shared__ uint32_t s_digit, s_dabove, s_dcnt, s_fill, s_total;
    const int t = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int32_t nc = (int32_t)min(visible_blocks(row_pos[r]), (int64_t)max_nb);
    const int32_t kk = min(top_k, nc);
    if (nc <= top_k) return;  // written by the collect kernel
    int32_t *out = sel_blocks + r * top_k;
    float *osc = sel_scores ? sel_scores + r * top_k : nullptr;
    const uint32_t *cnt = ss.scratch + r * kRowScratch + kHistBins;
    const uint2 *sure = ss.sure + r * top_k;
    const uint2 *cand = ss.cand + r * ss.cand_stride;
    const uint32_t n_sure = cnt[0];
    const uint32_t n_cand = cnt[1];
    uint32_t need = (uint32_t)kk - n_sure;  // 1 <= need <= n_cand
    // the kept-for-sure entries (fewer than kk) are loaded now, alongside the
    // candidates, and held in registers until the kept set is gathered
    constexpr int kSurePer = QSA_MAX_TOP_K / kSplitThreads;
    uint2 sure_r[kSurePer];
#pragma unroll
    for (int j = 0; j < kSurePer; ++j) {
        const uint32_t i = (uint32_t)(t + j * kSplitThreads);
        sure_r[j] = i < n_sure ? sure[i] : make_uint2(0u, 0u);
    }
    // candidates staged in LDS once when they fit (read by every radix pass)
    const bool staged = n_cand <= (uint32_t)kCandStage;
    if (staged)
        for (uint32_t i = t; i < n_cand; i += kSplitThreads) cst[i] = cand[i];
    __syncthreads();
    const uint2 *cl = staged ? cst : cand;
    uint64_t prefix = 0, pmask = 0;
    if (need < n_cand) {
        for (int sh = 44;; sh -= 8) {  // 8-bit digits of the 52-bit composite, from the top
            const int s2 = sh < 0 ? 0 : sh;
            const uint32_t dmask = sh < 0 ? (1u << (8 + sh)) - 1u : 0xffu;
            dhist[t] = 0u;
            __syncthreads();
            for (uint32_t i = t; i < n_cand; i += kSplitThreads) {
                const uint64_t c = composite20(cl[i]);
                if ((c & pmask) == prefix) atomicAdd(&dhist[(uint32_t)(c >> s2) & dmask], 1u);
            }
            __syncthreads();
            const uint32_t hv = dhist[255 - t];
            const uint32_t incl = wg_inclusive_scan<kSplitThreads>(hv, wtot);
            if (hv && incl - hv < need && incl >= need) {
                s_digit = 255u - (uint32_t)t;
                s_dabove = incl - hv;
                s_dcnt = hv;
            }
            __syncthreads();
            prefix |= (uint64_t)s_digit << s2;
            pmask |= (uint64_t)dmask << s2;
            need -= s_dabove;
            const bool done = s_dcnt == need || s2 == 0;
            __syncthreads();
            if (done) break;
        }
    }
    // ---- kept set: the sure entries and the picked candidates ----
    if (t == 0) s_fill = 0;
    __syncthreads();
    // one LDS atomic per wave and pass (the ballot gives each lane its slot)
    auto keep = [&](bool pred, uint2 e) {
        const uint64_t mask = __ballot(pred);
        if (!mask) return;
        const int lane = t & (kWave - 1);
        const int leader = __ffsll((unsigned long long)mask) - 1;
        uint32_t off = 0;
        if (lane == leader) off = atomicAdd(&s_fill, (uint32_t)__popcll(mask));
        off = __shfl(off, leader) + (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
        if (pred) buf[off] = ((uint64_t)e.y << 32) | e.x;
    };
#pragma unroll
    for (int j = 0; j < kSurePer; ++j) {
        const uint32_t i = (uint32_t)(t + j * kSplitThreads);
        keep(i < n_sure, sure_r[j]);
    }
    for (uint32_t i0 = 0; i0 < n_cand; i0 += kSplitThreads) {
        const uint32_t i = i0 + t;
        const uint2 e = i < n_cand ? cl[i] : make_uint2(0u, 0u);
        keep(i < n_cand && (composite20(e) & pmask) >= prefix, e);
    }
    __syncthreads();
    const uint32_t n = min(s_fill, (uint32_t)kk);
    if (t == 0) sel_count[r] = (int32_t)n;
    // ---- emit in block order: mark the kept blocks in an LDS bitmap (one
    // window of the visible range at a time); each thread reads its run of
    // words once, the runs' prefix counts give every word its exclusive
    // count, and each kept entry then finds its slot from its word's count
    // and the bits below it.  (Kept blocks cluster, so walking each thread's
    // set bits would serialise on the threads that hold the clusters.)  The
    // candidate stage is free by now and holds the word counts. ----
    static_assert(kEmitWords + 2 * (kEmitWords / 32) <= 4 * kCandStage, "word counts fit the candidate stage");
    static_assert(kEmitWords % (32 * kSplitThreads) == 0, "whole 32-word runs per thread");
    uint16_t *pre = (uint16_t *)cst;
    uint32_t out_base = 0;
    for (int64_t w0 = 0; w0 < nc; w0 += 32 * kEmitWords) {
        const int nwords = (int)min((int64_t)kEmitWords, (nc - w0 + 31) / 32);
        // the whole bitmap is cleared, so words past the window read as 0
        static_assert(kEmitSlots % kSplitThreads == 0, "the bitmap clears in whole rounds");
#pragma unroll
        for (int q = 0; q < kEmitSlots / kSplitThreads; ++q) bm[q * kSplitThreads + t] = 0u;
        __syncthreads();
        for (uint32_t i = t; i < n; i += kSplitThreads) {
            const int64_t b = (int64_t)(buf[i] >> 32) - w0;
            if (b >= 0 && b < 32 * (int64_t)nwords) atomicOr(&bm[emit_slot((int)(b >> 5))], 1u << (b & 31));
        }
        __syncthreads();
        // the thread's run of kPer words, read once into registers (all
        // reads in flight together; no guards, so the reads are not split
        // into separate branches)
        constexpr int kPer = kEmitWords / kSplitThreads;
        const int i0 = t * kPer;
        uint32_t words[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) words[j] = bm[emit_slot(i0 + j)];
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) c += (uint32_t)__popc(words[j]);
        const uint32_t incl = wg_inclusive_scan<kSplitThreads>(c, wtot);
        if (t == kSplitThreads - 1) s_total = incl;
        uint32_t run = incl - c;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            pre[emit_pre_slot(i0 + j)] = (uint16_t)run;
            run += (uint32_t)__popc(words[j]);
        }
        __syncthreads();
        for (uint32_t i = t; i < n; i += kSplitThreads) {
            const uint64_t e = buf[i];
            const int64_t blk = (int64_t)(e >> 32), b = blk - w0;
            if (b < 0 || b >= 32 * (int64_t)nwords) continue;
            const int wd = (int)(b >> 5);
            const uint32_t pos = out_base + (uint32_t)pre[emit_pre_slot(wd)] +
                                 (uint32_t)__popc(bm[emit_slot(wd)] & ((1u << (b & 31)) - 1u));
            if (pos < (uint32_t)kk) {
                out[pos] = (int32_t)blk;
                if (osc) osc[pos] = scaled_score(key_score((uint32_t)e));  // the entry's key is its score's
            }
        }
        __syncthreads();
        out_base += s_total;
    }
    for (int32_t i = (int32_t)n + t; i < top_k; i += kSplitThreads) {
        out[i] = -1;
        if (osc) osc[i] = 0.0f;
    }
}

void launch_select_split(const float *scores, int64_t sc_stride, const int32_t *row_pos, int32_t rows, int32_t max_nb,
                         int32_t top_k, const SplitSelect &ss, int32_t *sel_blocks, int32_t *sel_count,
                         float *sel_scores, hipStream_t stream)
{
    const int64_t chunks = max((int64_t)1, ((int64_t)max_nb + kCollectChunk - 1) / kCollectChunk);
    QSA_LAUNCH("select_collect", select_collect_kernel, dim3((unsigned)chunks, (unsigned)rows), dim3(kSplitThreads),
               0, stream, scores, sc_stride, row_pos, max_nb, top_k, ss, sel_blocks, sel_count, sel_scores);
    QSA_LAUNCH("select_final", select_final_kernel, dim3((unsigned)rows), dim3(kSplitThreads), 0, stream, scores,
               sc_stride, row_pos, max_nb, top_k, ss, sel_blocks, sel_count, sel_scores);
}

}  // namespace qsa
