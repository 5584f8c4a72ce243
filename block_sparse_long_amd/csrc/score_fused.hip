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
// blocks), everything above or below lumped into the end bins.  tau is the
// lowest key of bin b*, the highest bin at which k written pairs are reached;
// every written pair lies in a bin <= b*, so after each 64-block step b*
// only moves up while the bins above it still hold k pairs (a few LDS reads
// per row).  A step's pairs get their slots with one LDS atomic per row,
// ordered by block, so each split's list is ascending.
//
// Workgroup: 4 waves x 16 query rows (MFMA row m of tile mt = query row
// 4*mt + m/4, index head m%4, so a lane's 4 accumulators are the 4 heads of
// one (row, block) pair), one split of the block range.  The 64-block key
// tile is staged through LDS (double buffered) and shared by the 4 waves.
// The merge kernel takes, per row, the pairs of every split at or above the
// best split's tau -- in block order, since the splits are ordered and each
// list is ascending -- finds the exact k-th key with a radix select (12, 12,
// 8 bits), and emits, in block order, every pair above it and the first
// `need` pairs equal to it (lower blocks win ties).  A row whose pair buffer
// overflowed (e.g. massive exact ties) is redone from recomputed scores.
#include "qsa_device.h"
#include "qsa_internal.h"
#include "qsa_wg.h"

namespace qsa {

namespace {

constexpr int kFRows = 64;            // rows per workgroup
constexpr int kFStep = 64;            // blocks per step
constexpr int kFKRow = kDim + 8;      // LDS key row stride (bf16): conflict-free b128 reads
constexpr int kTauBins = 256;
constexpr int kTauShift = 18;         // 2^18 key units = 1/32 octave
constexpr int kMergeWaves = 4;        // merge: rows per workgroup, one wave each
constexpr int kStage = 2048;          // merge: pairs a wave stages in LDS

__device__ __forceinline__ float relu_sum4f(f32x4_t a)
{
    return ((fmaxf(a[0], 0.0f) + fmaxf(a[1], 0.0f)) + fmaxf(a[2], 0.0f)) + fmaxf(a[3], 0.0f);
}

// Top of a row's bin window: its anchor key + 4 octaves (2^25 key units).
__device__ __forceinline__ uint32_t window_top(uint32_t anchor)
{
    const uint64_t t = (uint64_t)anchor + (1ull << 25);
    return t > 0xffffffffull ? 0xffffffffu : (uint32_t)t;
}

// Bin of a key: 0 at and above the window top, 255 for everything 8 octaves down.
__device__ __forceinline__ int tau_bin(uint32_t key, uint32_t top)
{
    if (key >= top) return 0;
    const uint32_t b = (top - key) >> kTauShift;
    return b >= (uint32_t)(kTauBins - 1) ? kTauBins - 1 : (int)b;
}

// Threshold key -> float for `score >= tau` (key 0: no threshold yet).
__device__ __forceinline__ float tau_float(uint32_t key) { return key == 0u ? -INFINITY : key_score(key); }

// Lowest key of bin b (the last bin reaches down to every key).
__device__ __forceinline__ uint32_t tau_bin_floor(int b, uint32_t top)
{
    if (b >= kTauBins - 1) return 0u;
    const int64_t k = (int64_t)top - ((int64_t)(b + 1) << kTauShift) + 1;
    return k <= 0 ? 0u : (uint32_t)k;
}

__device__ __forceinline__ uint32_t hist_get(const uint32_t *h, int b) { return (h[b >> 1] >> (16 * (b & 1))) & 0xffffu; }

__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

}  // namespace

__global__ __launch_bounds__(256, 2) void score_filter_kernel(FusedScoreArgs a)
{
    const bf16_t *__restrict__ qrot = (const bf16_t *)a.qrot;
    const bf16_t *__restrict__ pooled = (const bf16_t *)a.pooled;
    __shared__ bf16_t keys[2][kFStep][kFKRow];
    __shared__ uint32_t hist[kFRows][kTauBins / 2];  // two 16-bit bins per word
    __shared__ uint32_t cnt[kFRows], tau[kFRows], wtop[kFRows], removed[kFRows];
    __shared__ int32_t bstar[kFRows];
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
        wtop[t] = window_top(0x80000000u);
        removed[t] = 0u;
        bstar[t] = kTauBins - 1;
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
    uint2 *my_buf[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int rw = 16 * wave + 4 * mt + g;
        my_nc[mt] = rw < nrows ? min(visible_blocks(a.row_pos[row0 + rw]), (int64_t)a.max_nb) : 0;
        my_seq[mt] = rw < nrows ? a.row_seq[row0 + rw] : -1;
        my_buf[mt] = a.buf + ((row0 + min(rw, nrows - 1)) * a.nsplit + split) * (int64_t)a.cap;
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
            // ---- scores of the step: 4 block tiles x (4 independent row-tile chains) ----
            float sc[4][4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                bf16x8_t bk[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) bk[s] = as_bf16x8(*(const uint4 *)&keys[cur][nt * 16 + m][32 * g + 8 * s]);
                f32x4_t acc[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][s], bk[s], acc[mt], 0, 0, 0);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) sc[mt][nt] = relu_sum4f(acc[mt]);
            }
            if (more) store_tile(cur ^ 1);
            // valid iff 16*nt < lr[mt] (block base + 16*nt + m below the row's bound)
            int32_t lr[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) lr[mt] = (int32_t)max(min(lim[mt] - base - m, (int64_t)kFStep), (int64_t)-1);
            // ---- anchors: each row's best score in its first step ----
            if (first_step) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    float mx = 0.0f;
#pragma unroll
                    for (int nt = 0; nt < 4; ++nt)
                        if (16 * nt < lr[mt]) mx = fmaxf(mx, sc[mt][nt]);
                    for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
                    if (m == 0 && lim[mt] > 0) wtop[16 * wave + 4 * mt + g] = window_top(score_key(mx));
                }
                wave_fence();
                first_step = false;
            }
            // ---- filter: pairs at or above the row's tau are written out ----
            bool appended = false;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                bool pass[4];
                bool any = false;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    pass[nt] = sc[mt][nt] >= tauf[mt] && 16 * nt < lr[mt];
                    any |= pass[nt];
                }
                if (!__ballot(any)) continue;  // wave-uniform
                appended = true;
                // slots of row 16*wave + 4*mt + g, ordered by block (nt, then m)
                const int rw = 16 * wave + 4 * mt + g;
                uint32_t mine[4], total = 0;
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const uint32_t grp = (uint32_t)(__ballot(pass[nt]) >> (16 * g)) & 0xffffu;
                    mine[nt] = total + (uint32_t)__popc(grp & ((1u << m) - 1u));
                    total += (uint32_t)__popc(grp);
                }
                uint32_t slot0 = 0;
                if (m == 0 && total) slot0 = atomicAdd(&cnt[rw], total);
                slot0 = __shfl(slot0, 16 * g);
                const uint32_t top = wtop[rw];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    const uint32_t slot = slot0 + mine[nt];
                    if (pass[nt] && slot < (uint32_t)a.cap) {
                        const uint32_t key = score_key(sc[mt][nt]);
                        my_buf[mt][slot] = make_uint2(key, (uint32_t)(base + nt * 16 + m));
                        const int bin = tau_bin(key, top);
                        atomicAdd(&hist[rw][bin >> 1], (bin & 1) ? 0x10000u : 1u);
                    }
                }
            }
            if (appended) {
                wave_fence();
                // ---- raise tau: lane i < 16 moves row 16*wave + i's b* up ----
                bool changed = false;
                if (lane < 16) {
                    const int rw = 16 * wave + lane;
                    const uint32_t c_all = cnt[rw];
                    if (c_all <= (uint32_t)a.cap) {
                        uint32_t c = c_all - removed[rw];
                        int bs = bstar[rw];
                        const uint32_t *h = hist[rw];
                        while (bs > 0) {
                            const uint32_t hb = hist_get(h, bs);
                            if (c - hb < (uint32_t)a.top_k) break;
                            c -= hb;
                            --bs;
                        }
                        if (bs != bstar[rw]) {
                            removed[rw] = c_all - c;
                            bstar[rw] = bs;
                            tau[rw] = tau_bin_floor(bs, wtop[rw]);
                            changed = true;
                        }
                    }
                }
                if (__ballot(changed)) {
                    wave_fence();
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

__device__ __forceinline__ float scaled(float raw) { return (float)((double)raw / sqrt((double)kDim)); }

}  // namespace

// One wave per row, four rows per workgroup; no workgroup barriers.  The
// row's pairs >= the best split's tau are visited in block order -- from LDS
// when they fit, else straight from the pair buffers -- or, for a row whose
// buffer overflowed, as recomputed scores of every visible block.
__global__ __launch_bounds__(256) void select_merge_kernel(FusedScoreArgs a, int32_t *__restrict__ sel_blocks,
                                                         int32_t *__restrict__ sel_count, float *__restrict__ sel_scores)
{
    __shared__ uint2 stage[kMergeWaves][kStage];
    __shared__ uint32_t hb[kMergeWaves][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t r = (int64_t)blockIdx.x * kMergeWaves + w;
    if (r >= a.rows) return;
    const uint64_t lt = (1ull << lane) - 1ull;  // lanes below this one
    const int32_t nc = (int32_t)min(visible_blocks(a.row_pos[r]), (int64_t)a.max_nb);
    const int32_t kk = max(0, min(a.top_k, nc));
    int32_t *out = sel_blocks + r * a.top_k;
    float *osc = sel_scores ? sel_scores + r * a.top_k : nullptr;
    if (lane == 0) sel_count[r] = kk;
    for (int32_t i = kk + lane; i < a.top_k; i += kWave) {
        out[i] = -1;
        if (osc) osc[i] = 0.0f;
    }
    if (nc <= 0) return;  // no visible block (the scorer may not have run at all)
    bool overflow = false;
    uint32_t tau_max = 0;
    for (int s = 0; s < a.nsplit; ++s) {
        overflow |= a.cnt[r * a.nsplit + s] > (uint32_t)a.cap;
        tau_max = max(tau_max, a.tau[r * a.nsplit + s]);
    }
    uint2 *st = stage[w];
    uint32_t *h = hb[w];
    // ---- the pairs to rank: mode 0 staged in LDS, 1 in the buffers, 2 recomputed ----
    uint32_t n = 0;
    int mode = 2;
    if (!overflow) {
        for (int s = 0; s < a.nsplit; ++s) {
            const uint32_t c = a.cnt[r * a.nsplit + s];
            const uint2 *src = a.buf + (r * a.nsplit + s) * (int64_t)a.cap;
            for (uint32_t i0 = 0; i0 < c; i0 += kWave) {
                const uint32_t i = i0 + lane;
                const uint2 e = i < c ? src[i] : make_uint2(0u, 0u);
                const bool keep = i < c && e.x >= tau_max;
                const uint64_t bal = __ballot(keep);
                const uint32_t pos = n + (uint32_t)__popcll(bal & lt);
                if (keep && pos < (uint32_t)kStage) st[pos] = e;
                n += (uint32_t)__popcll(bal);
            }
        }
        mode = n <= (uint32_t)kStage ? 0 : 1;
    }
    const int32_t seq = a.row_seq[r];
    const bf16_t *q4 = (const bf16_t *)a.qrot + r * kIdxHeads * kDim;
    const bf16_t *kb = (const bf16_t *)a.pooled + (int64_t)seq * a.pooled_stride;
    if (mode == 2) n = (uint32_t)nc;
    wave_fence();
    // visit every pair in block order, 64 at a time: fn(pair, valid)
    auto visit = [&](auto &&fn) {
        if (mode == 0) {
            for (uint32_t i0 = 0; i0 < n; i0 += kWave) {
                const uint32_t i = i0 + lane;
                fn(i < n ? st[i] : make_uint2(0u, 0u), i < n);
            }
        } else if (mode == 1) {
            for (int s = 0; s < a.nsplit; ++s) {
                const uint32_t c = a.cnt[r * a.nsplit + s];
                const uint2 *src = a.buf + (r * a.nsplit + s) * (int64_t)a.cap;
                for (uint32_t i0 = 0; i0 < c; i0 += kWave) {
                    const uint32_t i = i0 + lane;
                    const uint2 e = i < c ? src[i] : make_uint2(0u, 0u);
                    fn(e, i < c && e.x >= tau_max);
                }
            }
        } else {
            for (int32_t b0 = 0; b0 < nc; b0 += kWave) {
                const int32_t b = b0 + lane;
                const bool v = b < nc;
                const uint32_t key = v ? score_key(recompute_score(q4, kb + (int64_t)b * kDim)) : 0u;
                fn(make_uint2(key, (uint32_t)b), v);
            }
        }
    };
    // ---- radix select of the kk-th key, 8 bits at a time ----
    uint32_t need = (uint32_t)kk, prefix = 0;
    int sh = 32;  // key >> sh == prefix marks the current bin (32: none yet)
    if ((uint32_t)kk < n) {
        for (int pass = 0; pass < 4; ++pass) {
            const int nsh = sh - 8;
#pragma unroll
            for (int j = 0; j < 4; ++j) h[4 * lane + j] = 0u;
            wave_fence();
            visit([&](uint2 e, bool v) {
                if (v && (sh == 32 || (e.x >> sh) == prefix)) atomicAdd(&h[(e.x >> nsh) & 0xffu], 1u);
            });
            wave_fence();
            uint32_t hv[4], sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hv[j] = h[255 - 4 * lane - j];
                sum += hv[j];
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
                for (int j = 0; j < 4; ++j) {
                    if (acc + hv[j] >= need) {
                        digit = 255u - 4u * (uint32_t)lane - (uint32_t)j;
                        above = acc;
                        cntd = hv[j];
                        break;
                    }
                    acc += hv[j];
                }
            }
            digit = __shfl(digit, ls);
            above = __shfl(above, ls);
            cntd = __shfl(cntd, ls);
            need -= above;
            prefix = (sh == 32 ? 0u : (prefix << 8)) | digit;
            sh = nsh;
            if (cntd == need) break;
        }
    }
    // ---- emit in block order: keys above the bin, and the first `need` in it ----
    uint32_t eq_before = 0, out_before = 0;
    visit([&](uint2 e, bool v) {
        const bool all = sh == 32;
        const uint32_t top = all ? 0u : (e.x >> sh);
        const bool gt = v && (all || top > prefix);
        const bool eq = v && !all && top == prefix;
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
    QSA_LAUNCH("select_merge", select_merge_kernel, dim3((unsigned)((a.rows + kMergeWaves - 1) / kMergeWaves)),
               dim3(kMergeWaves * kWave), 0, stream, a, sel_blocks, sel_count, sel_scores);
}

}  // namespace qsa
