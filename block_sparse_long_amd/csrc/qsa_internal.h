// qsa_internal.h -- what the C-ABI layer (api.cpp) and the kernel files share:
// the launch wrapper and the host-side launchers of every kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

constexpr int kDim = 128;       // indexer key / query dim, attention head dim
constexpr int kDimWide = 256;   // the wider attention head dim (bf16 MFMA path)
constexpr int kHalf = 64;       // rotate-half pairs (j, j + 64)
constexpr int kIdxHeads = 4;    // indexer query heads
constexpr int kBlock = 4;       // tokens per micro-block
constexpr int kWave = 64;       // CDNA wavefront
constexpr uint32_t kFlagNoRope = 1u;
constexpr uint32_t kFlagRmsNorm = 2u;

// ---- launch bookkeeping (api.cpp) -----------------------------------------
bool profiling_enabled();
void prof_begin(const char *name, hipStream_t stream);
void prof_end(hipStream_t stream);
void note_launch(hipError_t err);

// ---- paged compressed keys (pool.hip, score.hip, score_fused.hip) -----------
// Paged compressed keys (table null: contiguous per sequence).  The KV pool
// keeps one compressed key per 4 token slots, at full_slot / 4; with pages of
// page_tokens slots (a multiple of 4), block b of sequence s is key
// table[s*stride + b/bpp]*bpp + b%bpp, bpp = page_tokens / 4.
struct KeyPages {
    const int32_t *table;
    int64_t stride;
    int32_t bpp;
};

// ---- pool.hip ---------------------------------------------------------------
// Frequencies of the 64 rotary pairs (inv_freq of pair (j, j + 64)), formed on
// the host in double precision and passed to the kernels by value.
struct RopeFreq {
    double f[kHalf];
};
RopeFreq rope_freq_plain(double theta);  // theta^(-j/64)
// YaRN's interpolated frequencies (scale s >= 1 over an original context of
// L tokens, ramp alpha..beta in turns over L); s == 1 gives rope_freq_plain.
RopeFreq rope_freq_yarn(double theta, double s, double L, double alpha, double beta);
void launch_pool(const void *raw, int64_t raw_stride, void *pooled, int64_t pooled_stride, const KeyPages &kp,
                 int32_t batch, int32_t block_begin, int32_t block_end, const RopeFreq &rf, uint32_t flags,
                 bool bf16, hipStream_t stream, const float *norm_weight = nullptr);
void launch_pool_fp8(const void *raw, int64_t raw_stride, uint8_t *codes, float *scales, int64_t pooled_stride,
                     const KeyPages &kp, int32_t batch, int32_t block_begin, int32_t block_end, const RopeFreq &rf,
                     uint32_t flags, bool bf16_raw, hipStream_t stream);
void launch_pool_append(const void *new_keys, const int32_t *positions, const int64_t *full_slots, void *ring,
                        void *compressed, int32_t batch, const RopeFreq &rf, uint32_t flags, bool bf16,
                        hipStream_t stream);
void launch_rope_query(const void *q, const int32_t *row_pos, int32_t rows, void *qrot, const RopeFreq &rf,
                       uint32_t flags, bool bf16, uint32_t *zero, int64_t zero_per_row, hipStream_t stream);

// ---- score.hip --------------------------------------------------------------
// Select histogram: 4096 bins of the top 12 bits of a score's order key.
constexpr int kHistBins = 4096;
constexpr int kHistShift = 20;
void launch_score_rows(const void *qrot, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                       const void *pooled, int64_t pooled_stride, const KeyPages &kp, int32_t max_nb, float *scores,
                       int64_t sc_stride, uint32_t *hist, bool bf16, hipStream_t stream);
void launch_score_rows_fp8(const void *qrot, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                           const uint8_t *codes, const float *scales, int64_t pooled_stride, const KeyPages &kp,
                           int32_t max_nb, float *scores, int64_t sc_stride, uint32_t *hist, hipStream_t stream);

// ---- score_fused.hip (many rows, bf16) ----------------------------------------
struct FusedScoreArgs {
    const uint16_t *qrot;     // [rows][4][128] rotated index queries (bf16)
    const int32_t *row_seq;
    const int32_t *row_pos;
    int32_t rows;
    const uint16_t *pooled;   // [B][pooled_stride] (bf16), or NULL with FP8 keys
    const uint8_t *codes;     // FP8 keys: [B][pooled_stride][128] E4M3 codes, else NULL
    const float *scales;      // FP8 keys: [B][pooled_stride] one scale per key
    int64_t pooled_stride;    // elements per sequence (bf16) or keys per sequence (FP8); unused when paged
    KeyPages kp;
    int32_t max_nb;
    int32_t top_k;
    int32_t nsplit;           // block-range splits of the main pass
    int32_t split_len;        // blocks per split (multiple of 64)
    int32_t subcap;           // capacity of one lane's pair list (16 lists per row and split)
    uint2 *buf;               // [rows][nsplit] blocks of 16 lists x subcap (key, block) pairs; the 16
                              // lists of a block interleaved slot by slot when nsplit >= 2
    uint32_t *cnt;            // [rows][nsplit][16] pairs per list (may exceed subcap: overflow)
    int32_t nsample;          // sampled blocks per row (one per 32)
    int32_t ssplit;           // sample-range splits
    uint32_t *cand;           // [rows][ssplit][16][4] best sampled keys of each lane (0: none)
    uint32_t *tau;            // [rows] threshold key (0: no threshold)
    int32_t *mode;            // [rows] how the merge ranked the row (kMergeMode*)
};
// Merge modes of a row, recorded for diagnostics.
enum : int32_t {
    kMergeNone = 0,         // no visible block
    kMergeStaged = 1,       // every pair staged in LDS and ranked there
    kMergePrefilter = 2,    // more pairs than the stage: a histogram picks those that can be kept
    kMergeListWalk = 3,     // the k-th key's bin too crowded to stage: radix passes over the lists
    kMergeRecompute = 4     // count short or a list overflowed (or too many exact ties): scores recomputed
};
int32_t fused_score_splits(int32_t rows, int32_t max_nb);
int32_t fused_score_split_len(int32_t max_nb, int32_t nsplit);
int32_t fused_score_subcap(int32_t top_k, int32_t nsplit);
int32_t fused_score_nsample(int32_t max_nb);
int32_t fused_score_ssplit(int32_t rows, int32_t nsample);
void launch_score_fused(const FusedScoreArgs &a, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                        hipStream_t stream);

// ---- select.hip -------------------------------------------------------------
void launch_select_rows(const float *scores, int64_t sc_stride, const int32_t *row_pos, int32_t rows,
                        int32_t max_nb, int32_t top_k, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                        hipStream_t stream);
// Few rows: per-row scratch of the split selection (zeroed by rope_query):
// row r owns kRowScratch words at scratch + r * kRowScratch, the histogram
// first, then the counters (kept-for-sure count, candidate count, finished
// chunks, unused).
constexpr int kSelCounters = 4;
constexpr int kRowScratch = kHistBins + kSelCounters;
struct SplitSelect {
    uint32_t *scratch;    // [rows][kRowScratch]
    uint2 *sure;          // [rows][top_k] (key, block)
    uint2 *cand;          // [rows][cand_stride] (key, block)
    int64_t cand_stride;  // >= max_nb
};
void launch_select_split(const float *scores, int64_t sc_stride, const int32_t *row_pos, int32_t rows, int32_t max_nb,
                         int32_t top_k, const SplitSelect &ss, int32_t *sel_blocks, int32_t *sel_count,
                         float *sel_scores, hipStream_t stream);

// ---- attn.hip ---------------------------------------------------------------
// Position chunk of the attention kernels and the largest query group one
// workgroup holds (query rows sharing a selection x query heads per KV head).
constexpr int kAttnChunk = 64;
constexpr int kAttnMaxQ = 64;

struct AttnArgs {
    const void *q;            // prefill [rows][Hq][D]; decode [B][Qn][Hq][D]
    const int32_t *row_seq;   // prefill: sequence of each row; decode: unused
    const int32_t *row_pos;   // prefill [rows]; decode [B][Qn]
    const int32_t *tail_start;  // decode [B] or null
    const void *k_cache;
    const void *v_cache;
    int64_t kv_seq_stride;
    const int32_t *sel_blocks;  // [groups-of-rows][top_k]
    const int32_t *sel_count;
    int32_t top_k;
    int32_t n_sel;            // prefill: rows; decode: batch
    int32_t q_per_sel;        // prefill 1; decode Qn
    int32_t Hq, Hkv;
    int32_t D;                // head dim: 128 (every path) or 256 (bf16 MFMA path)
    float scale;
    void *out;
    float *lse;
    float *partial;           // decode split partials, or null (prefill: no split)
    int32_t nsplit;
    // paged K/V (null: contiguous per sequence): token p of sequence s sits
    // at slot page_table[s*pt_stride + p/page_tokens]*page_tokens + p%page_tokens
    // of k_cache / v_cache, which are then [slots][Hkv][D]
    const int32_t *page_table;
    int64_t pt_stride;
    int32_t page_tokens;      // a multiple of 4: a block never straddles pages
    // FP8 K/V (MFMA path): k_cache / v_cache hold E4M3 codes whose values are
    // k_scale * E4M3(code) and v_scale * E4M3(code)
    int32_t kv_fp8;
    float k_scale, v_scale;
};
int32_t attn_decode_splits(int32_t top_k);
void launch_attn_prefill(const AttnArgs &a, bool bf16, hipStream_t stream);
void launch_attn_decode(const AttnArgs &a, bool bf16, hipStream_t stream);
void launch_attn_combine(const AttnArgs &a, bool bf16, hipStream_t stream);

// ---- attn_mfma.hip (bf16 q, bf16 or FP8 K/V, D 128 or 256, Hq/Hkv up to 64) ---
bool attn_mfma_supported(int32_t Hq, int32_t Hkv, int32_t q_per_sel, int32_t D, bool bf16);
void launch_attn_prefill_mfma(const AttnArgs &a, hipStream_t stream);
void launch_attn_decode_mfma(const AttnArgs &a, hipStream_t stream);

}  // namespace qsa

// Launch `kernel` on `stream`; record a failed launch for the calling entry
// point; bracket the launch with timing events while profiling is on.
#define QSA_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                  \
    do {                                                                           \
        const bool qsa_prof_ = qsa::profiling_enabled();                           \
        if (qsa_prof_) qsa::prof_begin(name, stream);                              \
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);        \
        qsa::note_launch(hipGetLastError());                                       \
        if (qsa_prof_) qsa::prof_end(stream);                                      \
    } while (0)
