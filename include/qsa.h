/*
 * qsa.h -- C-ABI of libqsa, the MI355X (gfx950) hot path of Qwen Sparse
 * Attention (QSA).
 *
 * Sources (web pages, by title and section):
 *   [SGL]  "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
 *          Attention: Retrieve Coarsely, Attend Precisely" (indexer pooling
 *          c4, post-pool rotation, score equation s_{t,b}, best 512 blocks,
 *          2048 token positions plus the zero-to-three tail tokens, attention
 *          on the original K/V) and section "IndexShare MTP" (draft rows
 *          reuse one selection plus the positions drafted since).
 *   [ARCH] "Qwen3.8-Flash-Next architecture" guide, "How a token moves through
 *          the model", item 2 (RoPE after key pooling; 512 blocks = 2,048
 *          tokens plus the incomplete tail block).
 *   [LBL]  "Qwen3.8-Flash-Next, Layer by Layer", section "Token mixing" (4 query
 *          heads and 1 key head of 128 dims, mean of every 4 keys, best 512;
 *          the full-attention layers' 24 query heads over 2 KV heads of 256
 *          dims) and section "Serving it" (indexer keys and the KV cache in
 *          FP8).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a device pointer (hipMalloc'd or equivalent).
 *     The caller owns every buffer; the library allocates no device memory,
 *     keeps no pointer after returning, and holds no state besides the
 *     optional timing records below.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream; the library never synchronizes.  Inputs
 *     must stay alive until the stream has passed the call.
 *   - Strides and sizes count elements, not bytes.  Tensors are read with
 *     16-byte vector loads: their base pointers must be 16-byte aligned and
 *     their strides multiples of 8 elements.
 *   - Arguments are validated on the host before any HIP call.  A rejected
 *     call returns its status and launches nothing.  Calls with nothing to do
 *     (zero rows, an empty block range) return QSA_OK and launch nothing.
 *   - Data-dependent contracts (positions inside the caches, pooled blocks
 *     present for every visible block, kept block ids below the row's visible
 *     count) are the caller's; they are not checked.
 *   - Index-key dim 128, 4 indexer heads, 4 tokens per block ([SGL], [LBL]);
 *     the attention head dim is 128, or 256 on the bf16 path ([LBL]).
 *   - FP8 arrays (E4M3 codes) are bytes: their strides count bytes, and code
 *     rows must be 16-byte aligned like the other tensors.
 *   - A block b is visible to a query at position t when it is complete:
 *     4b + 3 <= t, i.e. b < nc(t) = floor((t+1)/4) ([SGL]: the visible
 *     compressed blocks plus the zero-to-three tail tokens).
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QSA_OK = 0,
    QSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, stride or flag */
    QSA_ERR_UNSUPPORTED = 2, /* dtype or head shape the library does not implement */
    QSA_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace_size() */
    QSA_ERR_DEVICE = 4       /* a HIP call or kernel launch failed */
} qsa_status_t;

typedef enum {
    QSA_F32 = 0,  /* IEEE binary32 everywhere */
    QSA_BF16 = 1  /* bfloat16 storage; FP32 accumulation inside the kernels */
} qsa_dtype_t;

enum {
    QSA_FLAG_NO_ROPE = 1u << 0,       /* skip both rotations (keys and index queries) */
    QSA_FLAG_POOL_RMSNORM = 1u << 1,  /* pooled key -> x / sqrt(mean(x^2) + 1e-6) before RoPE */
    /* qsa_score_topk only: pick the scoring kernel instead of the library's
     * choice (per-row streaming for few rows, the MFMA GEMM for many rows).
     * The result does not depend on it; tests and tuning use it. */
    QSA_FLAG_SCORE_ROWS = 1u << 8,
    QSA_FLAG_SCORE_GEMM = 1u << 9
};

#define QSA_INDEX_DIM 128
#define QSA_INDEX_HEADS 4
#define QSA_BLOCK_TOKENS 4
#define QSA_MAX_TOP_K 4096
#define QSA_MAX_QUERY_GROUP 64 /* query rows sharing a selection x (Hq / Hkv) */

/*
 * Steps a1-a3 ([SGL] pooling; [ARCH] item 2 rotation order): for every
 * sequence s < batch and block b in [block_begin, block_end), average the
 * four raw index keys of tokens 4b..4b+3 in FP32 (sum in token order, times
 * 1/4), optionally RMS-normalize (QSA_FLAG_POOL_RMSNORM), rotate with RoPE at
 * position 4b (pairs (j, j+64), angle 4b * rope_theta^(-j/64), formed in
 * double precision), and store the result rounded to `dtype` (nearest-even).
 *
 *   raw_keys  [batch][raw_seq_stride]: token i of sequence s at
 *             raw_keys + s*raw_seq_stride + i*128.  Read only.
 *   pooled    [batch][pooled_seq_stride]: block b at pooled + s*stride + b*128.
 *             Blocks outside [block_begin, block_end) are not touched.
 *   Requirements: raw_seq_stride >= 4*block_end*128 and pooled_seq_stride >=
 *   block_end*128 when batch > 1, both multiples of 8; rope_theta > 1 unless
 *   QSA_FLAG_NO_ROPE.
 */
qsa_status_t qsa_pool_index_keys(const void *raw_keys, int64_t raw_seq_stride, void *pooled,
                                 int64_t pooled_seq_stride, int32_t batch, int32_t block_begin,
                                 int32_t block_end, double rope_theta, uint32_t flags,
                                 qsa_dtype_t dtype, void *stream);

/*
 * Rotation of the _ex entry points: RoPE with base `theta` (> 1) on the pairs
 * (j, j+64), optionally with YaRN's frequency scaling for contexts beyond the
 * native one (flozi.net guide, "What the published evidence does and does
 * not show", and the aicontrolled journal: the 262,144-token native context
 * extends to one million tokens with YaRN; the pages give no parameters).
 * YaRN is the published method of Peng, Quesnelle, Fan and Shippole (2023),
 * its interpolation by parts: pair j, of frequency th_j = theta^(-j/64),
 * turns r_j = L * th_j / (2 pi) times over the original context of
 * L = yarn_original_context tokens; with g_j = 0 for r_j < alpha, 1 for
 * r_j > beta and (r_j - alpha) / (beta - alpha) between, the pair rotates at
 * (1 - g_j) * th_j / s + g_j * th_j, s = yarn_factor.  yarn_factor == 1 is
 * plain RoPE (the other YaRN fields are then ignored).  For 1M tokens from
 * the native 262,144: s = 4, L = 262144, alpha = 1, beta = 32 (the paper's
 * ramp).  YaRN's attention temperature multiplies scores by a positive
 * constant, which cannot change the indexer's ranking; it is not applied
 * (for the final attention it belongs in the caller's softmax_scale).
 */
typedef struct {
    double theta;
    double yarn_factor;
    double yarn_original_context;
    double yarn_alpha;
    double yarn_beta;
} qsa_rope_t;

/*
 * qsa_pool_index_keys with the rotation given as a qsa_rope_t, which may be NULL
 * with QSA_FLAG_NO_ROPE, and an optional learned weight for the pooled-key
 * normalization ([SGL]: the averaged keys are "normalized" before the
 * rotation; the pages give no norm or weight).  Reading: with
 * QSA_FLAG_POOL_RMSNORM the mean m becomes (m / sqrt(mean(m^2) + 1e-6)) * w
 * element by element, w = norm_weight (fp32 [128], device memory, 4-byte
 * aligned), or unit weight when norm_weight is NULL.  A weight without
 * QSA_FLAG_POOL_RMSNORM is QSA_ERR_INVALID_ARG.  With a NULL weight and
 * yarn_factor 1 this is exactly qsa_pool_index_keys; the weight costs one
 * multiply per element, the YaRN table nothing (it is formed on the host).
 */
qsa_status_t qsa_pool_index_keys_ex(const void *raw_keys, int64_t raw_seq_stride, void *pooled,
                                    int64_t pooled_seq_stride, int32_t batch, int32_t block_begin,
                                    int32_t block_end, const qsa_rope_t *rope,
                                    const float *norm_weight, uint32_t flags, qsa_dtype_t dtype,
                                    void *stream);

/*
 * Steps a1-a3 with the compressed keys stored in FP8 ([LBL] section "Serving
 * it": the deployment keeps the indexer's keys in FP8).  Each block is pooled
 * and rotated exactly as by qsa_pool_index_keys, then rounded to FP32; with
 * amax its largest magnitude, inv = 448 / amax and scale = amax / 448 (IEEE
 * FP32 quotients), and element d is stored as the OCP FP8 E4M3 code of
 * k_d * inv (FP32 product, nearest-even).  The key stands for code * scale.
 * A zero key gets scale 0 and zero codes.
 *   raw_keys  [batch][raw_seq_stride] of raw_dtype (bf16 or fp32), as above.
 *   codes     [batch][pooled_seq_stride][128] bytes; block b of sequence s at
 *             codes + (s*pooled_seq_stride + b)*128.  16-byte aligned.
 *   scales    [batch][pooled_seq_stride] fp32, one per key.  4-byte aligned.
 *   pooled_seq_stride counts keys (blocks), not bytes.  Blocks outside
 *   [block_begin, block_end) are not touched.
 */
qsa_status_t qsa_pool_index_keys_fp8(const void *raw_keys, int64_t raw_seq_stride, uint8_t *codes,
                                     float *scales, int64_t pooled_seq_stride, int32_t batch,
                                     int32_t block_begin, int32_t block_end, double rope_theta,
                                     uint32_t flags, qsa_dtype_t raw_dtype, void *stream);

/*
 * Incremental pooling for decode ([SGL] section "Qwen Sparse Attention": the
 * raw index keys of a request's unfinished block live in a four-slot
 * per-request ring, and the compressed cache is addressed by page-aligned
 * full_slot / 4).  For each request r, with its new token at position
 * t = positions[r] and physical KV slot full_slots[r]:
 *   - ring[r][t mod 4] = new_keys[r];
 *   - if t mod 4 == 3 (block b = t / 4 is complete): the four ring keys, which
 *     are tokens 4b..4b+3, are pooled exactly as qsa_pool_index_keys pools a
 *     block (FP32 sum in token order times 1/4, QSA_FLAG_POOL_RMSNORM, RoPE
 *     at position 4b unless QSA_FLAG_NO_ROPE, rounding to dtype) and stored
 *     at compressed[full_slots[r] / 4].
 *   new_keys   [batch][128], read only.
 *   positions  [batch] int32 (device), t >= 0.
 *   full_slots [batch] int64 (device).  Contract: pages are aligned to 4
 *              tokens, so full_slots[r] mod 4 == t mod 4 and the block's four
 *              tokens share compressed slot full_slots[r] / 4.  Not checked.
 *   ring       [batch][4][128], updated in place (slot t mod 4 written).
 *   compressed [slots][128]: one compressed key per 4 physical KV slots.
 *   Slots and positions are the caller's; the library keeps no state.
 */
qsa_status_t qsa_pool_append(const void *new_keys, const int32_t *positions, const int64_t *full_slots,
                             void *ring, void *compressed, int32_t batch, double rope_theta, uint32_t flags,
                             qsa_dtype_t dtype, void *stream);

/*
 * Bytes of device workspace qsa_score_topk needs for `rows` rows whose visible
 * block counts are at most `max_visible_blocks`, with the same `flags` the
 * call will get (the scoring kernel decides the layout).  0 when rows == 0 or
 * an argument is out of range.
 */
size_t qsa_score_topk_workspace_size(int32_t rows, int32_t max_visible_blocks, int32_t top_k,
                                     qsa_dtype_t dtype, uint32_t flags);

/*
 * Steps a4-a6 ([SGL] score equation and top-512; [LBL]).  For every row r with
 * sequence s = row_seq[r] and position t = row_pos[r]:
 *   - q~_h = round_dtype(RoPE(q_index[r][h], t)) for the 4 index heads;
 *   - raw(t,b) = sum_h max(0, <q~_h, pooled[s][b]>) for the visible blocks
 *     b < nc(t);
 *   - keep all visible blocks if nc(t) <= top_k, else the top_k best under
 *     (raw descending, block ascending).
 *   sel_blocks [rows][top_k] (out): kept blocks ascending, padded with -1.
 *   sel_count  [rows] (out): number kept = min(top_k, nc(t)).
 *   sel_scores [rows][top_k] (out, may be NULL): s_{t,b} = raw / sqrt(128) of
 *              each kept block, in the order of sel_blocks (0 for padding).
 *   q_index    [rows][4][128], un-rotated.  row_seq, row_pos: device int32.
 *   pooled     as written by qsa_pool_index_keys.
 *   max_visible_blocks: an upper bound of nc(row_pos[r]) over all rows; it
 *              sizes the grid and the workspace (positions live on the device,
 *              so the host cannot read them without a synchronization).
 *   workspace: device memory of at least qsa_score_topk_workspace_size()
 *              bytes, 256-byte aligned; its contents on entry do not matter.
 *   1 <= top_k <= QSA_MAX_TOP_K.  flags: QSA_FLAG_NO_ROPE, QSA_FLAG_SCORE_*.
 */
qsa_status_t qsa_score_topk(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                            int32_t rows, const void *pooled, int64_t pooled_seq_stride,
                            int32_t max_visible_blocks, int32_t top_k, double rope_theta,
                            uint32_t flags, qsa_dtype_t dtype, int32_t *sel_blocks,
                            int32_t *sel_count, float *sel_scores, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * qsa_score_topk with the index queries rotated by a qsa_rope_t, which may be NULL
 * with QSA_FLAG_NO_ROPE; the keys must have been pooled with the same
 * rotation (qsa_pool_index_keys_ex).  Workspace:
 * qsa_score_topk_workspace_size().  Everything else as qsa_score_topk.
 */
qsa_status_t qsa_score_topk_ex(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                               int32_t rows, const void *pooled, int64_t pooled_seq_stride,
                               int32_t max_visible_blocks, int32_t top_k, const qsa_rope_t *rope,
                               uint32_t flags, qsa_dtype_t dtype, int32_t *sel_blocks,
                               int32_t *sel_count, float *sel_scores, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Diagnostics of the many-rows scorer.  When qsa_score_topk (or its FP8 and
 * paged forms) runs the fused MFMA scorer for these arguments, the call
 * leaves in its workspace, at this byte offset, int32 [rows]: how the merge
 * ranked each row -- 0 no visible block; 1 all of the row's candidate pairs
 * ranked in LDS; 2 a histogram first narrowed the candidates to those that
 * can be kept; 3 radix passes over the candidate lists (the k-th score's bin
 * too crowded to stage); 4 the row's scores recomputed and ranked (too few
 * candidates, a full candidate list, or too many exact ties).  The selection
 * is the same whatever the mode.  Returns (size_t)-1 when the arguments are
 * invalid or the call would use the per-row scorer (no such record).
 */
size_t qsa_score_topk_merge_modes_offset(int32_t rows, int32_t max_visible_blocks, int32_t top_k,
                                         qsa_dtype_t dtype, uint32_t flags);

/*
 * qsa_score_topk on FP8 keys (as written by qsa_pool_index_keys_fp8).  The
 * index queries are bf16 and rotated as in qsa_score_topk; the key of block b
 * is code_b * scale_b, so raw(t,b) = scale_b * sum_h max(0, <q~_h, code_b>)
 * (a non-negative scale commutes with the ReLUs).  Selection, outputs and
 * workspace rules are those of qsa_score_topk; pooled_seq_stride counts keys.
 */
size_t qsa_score_topk_fp8_workspace_size(int32_t rows, int32_t max_visible_blocks, int32_t top_k,
                                         uint32_t flags);
qsa_status_t qsa_score_topk_fp8(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                                int32_t rows, const uint8_t *codes, const float *scales,
                                int64_t pooled_seq_stride, int32_t max_visible_blocks, int32_t top_k,
                                double rope_theta, uint32_t flags, int32_t *sel_blocks,
                                int32_t *sel_count, float *sel_scores, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Steps a7+a8 ([SGL]: expansion of the kept blocks to token positions, the
 * zero-to-three tail tokens, attention on the original K/V).  Row r (sequence
 * row_seq[r], position t = row_pos[r]) attends P = {4b+i : b in
 * sel_blocks[r][0..sel_count[r]), i < 4} U [4*nc(t), t]; query head h uses KV
 * head floor(h / (Hq/Hkv)); out = softmax(softmax_scale * q K_P^T) V_P.
 *   q        [rows][Hq][D]; k_cache, v_cache [B][kv_seq_stride]: token p of
 *            sequence s, KV head g at s*kv_seq_stride + (p*Hkv + g)*D.
 *   sel_blocks [rows][top_k], sel_count [rows] as written by qsa_score_topk.
 *   out      [rows][Hq][D], dtype.  lse [rows][Hq] fp32 natural-log
 *            log-sum-exp of the scaled logits, or NULL.
 *   D == 128, or D == 256 with dtype QSA_BF16; Hq % Hkv == 0;
 *   Hq/Hkv <= QSA_MAX_QUERY_GROUP; 1 <= top_k <= QSA_MAX_TOP_K.
 */
qsa_status_t qsa_sparse_attn_prefill(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                     int32_t rows, const void *k_cache, const void *v_cache,
                                     int64_t kv_seq_stride, const int32_t *sel_blocks,
                                     const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                     int32_t Hkv, int32_t D, float softmax_scale,
                                     qsa_dtype_t dtype, void *out, float *lse, void *stream);

/*
 * Paged KV pool ([SGL] section "Qwen Sparse Attention": the compressed keys
 * live in the paged KV pool, one per four token slots, addressed by
 * page-aligned full_slot / 4).  A sequence's tokens sit in pages of
 * page_tokens slots (a multiple of 4, so a block never straddles pages):
 * token p of sequence s is slot page_table[s*page_table_stride + p/page_tokens]
 * * page_tokens + p % page_tokens.  The paged variants below read
 *   - compressed keys [slots / 4][128]: block b of s is key
 *     slot(4b) / 4 (qsa_pool_append writes exactly there);
 *   - K/V caches [slots][Hkv][D].
 * page_table [n_seq][page_table_stride] int32 (device); its rows must cover
 * every position the call reads.  Everything else is as in the contiguous
 * entry points.
 */
/* qsa_pool_index_keys into a paged compressed-key pool: block b of sequence s
 * (raw keys contiguous as in qsa_pool_index_keys) is stored at key
 * slot(4b) / 4 -- into `pooled` (dtype = raw_dtype) or, for FP8 keys, into
 * `codes` + `scales` (as qsa_pool_index_keys_fp8; pass pooled = NULL).  The
 * table must cover block_end blocks (page_table_stride * page_tokens / 4 >=
 * block_end). */
qsa_status_t qsa_pool_index_keys_paged(const void *raw_keys, int64_t raw_seq_stride, void *pooled,
                                       uint8_t *codes, float *scales, const int32_t *page_table,
                                       int64_t page_table_stride, int32_t page_tokens, int32_t batch,
                                       int32_t block_begin, int32_t block_end, double rope_theta,
                                       uint32_t flags, qsa_dtype_t raw_dtype, void *stream);
/* qsa_score_topk on paged compressed keys: `pooled` (dtype) or, for FP8 keys,
 * `codes` + `scales` (with dtype QSA_BF16 for the index queries; pass
 * pooled = NULL).  Workspace: qsa_score_topk_workspace_size(..., dtype, flags). */
qsa_status_t qsa_score_topk_paged(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                                  int32_t rows, const void *pooled, const uint8_t *codes,
                                  const float *scales, const int32_t *page_table,
                                  int64_t page_table_stride, int32_t page_tokens,
                                  int32_t max_visible_blocks, int32_t top_k, double rope_theta,
                                  uint32_t flags, qsa_dtype_t dtype, int32_t *sel_blocks,
                                  int32_t *sel_count, float *sel_scores, void *workspace,
                                  size_t workspace_bytes, void *stream);
/* qsa_sparse_attn_prefill on a paged K/V pool (bf16 only, else
 * QSA_ERR_UNSUPPORTED). */
qsa_status_t qsa_sparse_attn_prefill_paged(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                           int32_t rows, const void *k_cache, const void *v_cache,
                                           const int32_t *page_table, int64_t page_table_stride,
                                           int32_t page_tokens, const int32_t *sel_blocks,
                                           const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                           int32_t Hkv, int32_t D, float softmax_scale,
                                           qsa_dtype_t dtype, void *out, float *lse, void *stream);

/*
 * Bytes of device workspace qsa_sparse_attn_decode needs (fp32 partial
 * softmax states, one per row, head and split of the positions; sized for one
 * split per 16 kept blocks, which bounds every launch: large bf16 launches
 * merge splits and use less).
 */
size_t qsa_sparse_attn_decode_workspace_size(int32_t batch, int32_t q_per_seq, int32_t Hq,
                                             int32_t D, int32_t top_k);

/*
 * Steps a7+a9 ([SGL] attention on the original K/V; [SGL] "IndexShare MTP":
 * rows of one sequence share that sequence's selection plus the positions
 * since it was taken).  Row j of sequence s sits at t = row_pos[s][j] and
 * attends P = {4b+i : b in sel_blocks[s][0..sel_count[s]), i < 4} U
 * [tail_start[s], t].  tail_start == NULL means 4*nc(t) for every row (plain
 * decode).  Contract: every position in P is < the cache length, and
 * tail_start[s] >= 4*(largest kept block + 1).
 *   q, out   [batch][q_per_seq][Hq][D]; lse [batch][q_per_seq][Hq] or NULL.
 *   row_pos  [batch][q_per_seq]; tail_start [batch] or NULL.
 *   sel_blocks [batch][top_k], sel_count [batch].
 *   workspace: at least qsa_sparse_attn_decode_workspace_size() bytes,
 *   256-byte aligned.  q_per_seq * (Hq/Hkv) <= QSA_MAX_QUERY_GROUP.
 *   Other arguments as in qsa_sparse_attn_prefill.
 */
qsa_status_t qsa_sparse_attn_decode(const void *q, const int32_t *row_pos, int32_t batch,
                                    int32_t q_per_seq, const int32_t *tail_start,
                                    const void *k_cache, const void *v_cache,
                                    int64_t kv_seq_stride, const int32_t *sel_blocks,
                                    const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                    int32_t Hkv, int32_t D, float softmax_scale,
                                    qsa_dtype_t dtype, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * qsa_sparse_attn_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc.  The split partials go to a static
 * device array of QSA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends (the copy of the calling thread's
 * current device is used; `stream` must belong to that device).  The call
 * allocates nothing (with kernel timing enabled, timing events are created
 * as for every entry point).  Arguments, results and errors are those of
 * qsa_sparse_attn_decode; a call whose workspace
 * (qsa_sparse_attn_decode_workspace_size) would exceed the array returns
 * QSA_ERR_WORKSPACE before any HIP call.  Every call on one GPU shares that
 * GPU's array, and nothing in it needs to start at zero: calls that overlap
 * on one GPU (concurrent streams or threads) race and are the caller's to
 * order.
 */
#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)
qsa_status_t qsa_sparse_attn_decode_noalloc(const void *q, const int32_t *row_pos, int32_t batch,
                                            int32_t q_per_seq, const int32_t *tail_start,
                                            const void *k_cache, const void *v_cache,
                                            int64_t kv_seq_stride, const int32_t *sel_blocks,
                                            const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                            int32_t Hkv, int32_t D, float softmax_scale,
                                            qsa_dtype_t dtype, void *out, float *lse, void *stream);

/* qsa_sparse_attn_decode on a paged K/V pool (bf16 with q_per_seq <= 32,
 * else QSA_ERR_UNSUPPORTED). */
qsa_status_t qsa_sparse_attn_decode_paged(const void *q, const int32_t *row_pos, int32_t batch,
                                          int32_t q_per_seq, const int32_t *tail_start,
                                          const void *k_cache, const void *v_cache,
                                          const int32_t *page_table, int64_t page_table_stride,
                                          int32_t page_tokens, const int32_t *sel_blocks,
                                          const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                          int32_t Hkv, int32_t D, float softmax_scale,
                                          qsa_dtype_t dtype, void *out, float *lse, void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * FP8 K/V cache ("Qwen3.8-Flash-Next, Layer by Layer", section "Serving it":
 * the KV cache kept in FP8).  k_codes / v_codes hold OCP E4M3 codes (the bit
 * layout of torch.float8_e4m3fn), one byte per element, laid out as the bf16
 * caches of qsa_sparse_attn_prefill / _decode (contiguous with kv_seq_stride,
 * in elements = bytes, a multiple of 16), or paged when page_table is not
 * NULL (then kv_seq_stride is ignored; see the paged pool above).  An
 * element's value is k_scale * E4M3(code) for K and v_scale * E4M3(code) for
 * V: one positive finite FP32 scale per cache tensor.  q, out are bf16;
 * lse as in the bf16 calls.  Head dim 128 or 256, Hq/Hkv <= 64, decode
 * q_per_seq <= 32 and q_per_seq * Hq/Hkv <= 64 (else QSA_ERR_UNSUPPORTED);
 * code arrays 16-byte aligned.  Decode workspace:
 * qsa_sparse_attn_decode_workspace_size().  Everything else as in the bf16
 * entry points.
 */
qsa_status_t qsa_sparse_attn_prefill_fp8kv(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                           int32_t rows, const uint8_t *k_codes, const uint8_t *v_codes,
                                           int64_t kv_seq_stride, const int32_t *page_table,
                                           int64_t page_table_stride, int32_t page_tokens, float k_scale,
                                           float v_scale, const int32_t *sel_blocks,
                                           const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                           int32_t Hkv, int32_t D, float softmax_scale, void *out,
                                           float *lse, void *stream);
qsa_status_t qsa_sparse_attn_decode_fp8kv(const void *q, const int32_t *row_pos, int32_t batch,
                                          int32_t q_per_seq, const int32_t *tail_start,
                                          const uint8_t *k_codes, const uint8_t *v_codes,
                                          int64_t kv_seq_stride, const int32_t *page_table,
                                          int64_t page_table_stride, int32_t page_tokens, float k_scale,
                                          float v_scale, const int32_t *sel_blocks,
                                          const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                          int32_t Hkv, int32_t D, float softmax_scale, void *out,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream);

/* Static description of a status code. */
const char *qsa_status_string(qsa_status_t status);

/*
 * HIP's description of the error behind the last QSA_ERR_DEVICE returned on
 * the calling thread ("none" if there was none).  Static string; the record
 * is per thread and kept until the next failure.
 */
const char *qsa_last_device_error(void);

/*
 * Kernel timing, for benchmarks.  While enabled, every kernel the library
 * launches is bracketed by a pair of hipEvents recorded on its stream.
 * qsa_profile_kernel_ms() waits for the recorded events, then returns how many
 * launches of kernel `name` were recorded and their total duration in
 * milliseconds (*total_ms).  qsa_profile_reset() drops the records.  A kernel
 * name not launched returns 0.  Timing is off by default and costs nothing
 * then.  Thread-safe: the flag is atomic and the records are kept under a
 * lock, so calls from several threads are all recorded in one list; a
 * qsa_profile_reset() while another thread is launching may drop that
 * launch's record.  The per-kernel sums read the records of every thread.
 */
qsa_status_t qsa_profile_enable(int enable);
qsa_status_t qsa_profile_reset(void);
int32_t qsa_profile_kernel_ms(const char *name, double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
