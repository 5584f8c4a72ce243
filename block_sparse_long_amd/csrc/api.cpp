// api.cpp -- the C-ABI of libqsa: argument validation (on the host, before
// any HIP call), workspace layout, kernel launches on the caller's stream,
// status strings and optional per-kernel timing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "qsa.h"
#include "qsa_internal.h"

namespace qsa {

// ---------------------------------------------------------------------------
// launch bookkeeping
// ---------------------------------------------------------------------------
static thread_local hipError_t g_launch_err = hipSuccess;
static thread_local hipError_t g_last_failure = hipSuccess;  // kept until the next failure

void note_launch(hipError_t err)
{
    if (err != hipSuccess && g_launch_err == hipSuccess) g_launch_err = g_last_failure = err;
}

// Drops an error another caller left pending in this thread (hipGetLastError
// reports the last error of any HIP call), so a launch reports only its own.
static void clear_launch_err()
{
    (void)hipGetLastError();
    g_launch_err = hipSuccess;
}
static qsa_status_t launch_status() { return g_launch_err == hipSuccess ? QSA_OK : QSA_ERR_DEVICE; }

// Timing records.  The enable flag is atomic; a launch's pending start event
// and name belong to the launching thread; the finished records and the pool
// of free events are shared and guarded by one mutex.  Timing is meant for
// benchmarks: records from several threads land in one list.
struct ProfRecord {
    std::string name;
    hipEvent_t start, stop;
};
static std::atomic<bool> g_prof{false};
static std::mutex g_prof_mutex;
static std::vector<ProfRecord> g_records;        // guarded by g_prof_mutex
static std::vector<hipEvent_t> g_free_events;    // guarded by g_prof_mutex
static thread_local std::string g_pending_name;
static thread_local hipEvent_t g_pending_start = nullptr;

static hipEvent_t take_event()
{
    {
        std::lock_guard<std::mutex> lock(g_prof_mutex);
        if (!g_free_events.empty()) {
            hipEvent_t e = g_free_events.back();
            g_free_events.pop_back();
            return e;
        }
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

bool profiling_enabled() { return g_prof.load(std::memory_order_relaxed); }

void prof_begin(const char *name, hipStream_t stream)
{
    g_pending_name = name;
    g_pending_start = take_event();
    if (g_pending_start) (void)hipEventRecord(g_pending_start, stream);
}

void prof_end(hipStream_t stream)
{
    hipEvent_t stop = take_event();
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    if (!g_pending_start || !stop) {  // no record: an event that was taken goes back to the pool
        if (g_pending_start) g_free_events.push_back(g_pending_start);
        if (stop) g_free_events.push_back(stop);
        g_pending_start = nullptr;
        return;
    }
    (void)hipEventRecord(stop, stream);
    g_records.push_back({g_pending_name, g_pending_start, stop});
    g_pending_start = nullptr;
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
static bool aligned16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool dtype_ok(qsa_dtype_t d) { return d == QSA_F32 || d == QSA_BF16; }
static size_t elem_bytes(qsa_dtype_t d) { return d == QSA_BF16 ? 2 : 4; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Rows up to this count use the per-row streaming scorer; more rows use the
// MFMA GEMM scorer, which shares each key tile among 16 rows.
constexpr int32_t kRowsPathMax = 64;

// Which kernels qsa_score_topk runs: many bf16 rows take the fused MFMA
// scorer + merge; few rows (or QSA_FLAG_SCORE_ROWS) the per-row streaming
// scorer, followed by the split selection (few rows) or the per-row select.
struct ScorePlan {
    bool fused, split;
};

static ScorePlan score_plan(int32_t rows, qsa_dtype_t dtype, uint32_t flags)
{
    const bool few = rows <= kRowsPathMax || dtype != QSA_BF16;
    ScorePlan p;
    p.fused = !few;
    if (flags & QSA_FLAG_SCORE_ROWS) p.fused = false;
    if (flags & QSA_FLAG_SCORE_GEMM) p.fused = true;
    p.split = few && !p.fused;
    return p;
}

// Workspace of qsa_score_topk: rotated index queries, then either the fp32
// scores (+ the split selection's per-row scratch, kept-for-sure and
// candidate lists) or the fused scorer's per-(row, split) pair buffers,
// counts and thresholds.
struct ScoreLayout {
    ScorePlan plan;
    int64_t sc_stride;
    size_t qrot_off, scores_off, scratch_off, sure_off, cand_off;
    int32_t nsplit, split_len, subcap, nsample, ssplit;
    size_t buf_off, cnt_off, scand_off, tau_off, mode_off;
    size_t total;
};

static ScoreLayout score_layout(int32_t rows, int32_t max_nb, int32_t top_k, qsa_dtype_t dtype, uint32_t flags)
{
    ScoreLayout L{};
    L.plan = score_plan(rows, dtype, flags);
    L.sc_stride = ((int64_t)max_nb + 63) / 64 * 64;
    L.qrot_off = 0;
    const size_t off = align256((size_t)rows * kIdxHeads * kDim * elem_bytes(dtype));
    if (L.plan.fused) {
        L.nsplit = fused_score_splits(rows, max_nb);
        L.split_len = fused_score_split_len(max_nb, L.nsplit);
        L.subcap = fused_score_subcap(top_k, L.nsplit);
        L.nsample = fused_score_nsample(max_nb);
        L.ssplit = fused_score_ssplit(rows, L.nsample);
        L.buf_off = off;
        L.cnt_off = L.buf_off + align256((size_t)rows * L.nsplit * 16 * (size_t)L.subcap * sizeof(uint2));
        L.scand_off = L.cnt_off + align256((size_t)rows * L.nsplit * 16 * sizeof(uint32_t));
        L.tau_off = L.scand_off + align256((size_t)rows * L.ssplit * 64 * sizeof(uint32_t));
        L.mode_off = L.tau_off + align256((size_t)rows * sizeof(uint32_t));
        L.total = L.mode_off + align256((size_t)rows * sizeof(int32_t));
        return L;
    }
    L.scores_off = off;
    L.total = L.scores_off + align256((size_t)rows * (size_t)L.sc_stride * sizeof(float));
    if (L.plan.split) {
        L.scratch_off = L.total;
        L.sure_off = L.scratch_off + align256((size_t)rows * kRowScratch * sizeof(uint32_t));
        L.cand_off = L.sure_off + align256((size_t)rows * (size_t)top_k * sizeof(uint2));
        L.total = L.cand_off + align256((size_t)rows * (size_t)L.sc_stride * sizeof(uint2));
    }
    return L;
}

static bool score_flags_ok(uint32_t flags, qsa_dtype_t dtype)
{
    const uint32_t known = QSA_FLAG_NO_ROPE | QSA_FLAG_SCORE_ROWS | QSA_FLAG_SCORE_GEMM;
    if (flags & ~known) return false;
    if ((flags & QSA_FLAG_SCORE_ROWS) && (flags & QSA_FLAG_SCORE_GEMM)) return false;
    return true;
}

}  // namespace qsa

using namespace qsa;

// Where qsa_score_topk's keys come from: `pooled` of the call's dtype, or FP8
// codes with one scale per key.
struct KeySource {
    const void *pooled;
    const uint8_t *codes;
    const float *scales;
    KeyPages kp;  // table null: contiguous
};
static qsa_status_t score_topk_run(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                                   int32_t rows, const KeySource &keys, int64_t pooled_seq_stride,
                                   int32_t max_visible_blocks, int32_t top_k, const RopeFreq &rf, uint32_t flags,
                                   qsa_dtype_t dtype, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                                   void *workspace, size_t workspace_bytes, void *stream);

extern "C" {

const char *qsa_status_string(qsa_status_t s)
{
    switch (s) {
    case QSA_OK: return "ok";
    case QSA_ERR_INVALID_ARG: return "invalid argument";
    case QSA_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case QSA_ERR_WORKSPACE: return "workspace too small";
    case QSA_ERR_DEVICE: return "HIP launch or runtime error";
    }
    return "unknown status";
}

const char *qsa_last_device_error(void)
{
    return g_last_failure == hipSuccess ? "none" : hipGetErrorString(g_last_failure);
}

qsa_status_t qsa_pool_index_keys(const void *raw_keys, int64_t raw_seq_stride, void *pooled,
                                 int64_t pooled_seq_stride, int32_t batch, int32_t block_begin,
                                 int32_t block_end, double rope_theta, uint32_t flags, qsa_dtype_t dtype,
                                 void *stream)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (batch < 0 || block_begin < 0 || block_end < block_begin) return QSA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(QSA_FLAG_NO_ROPE | QSA_FLAG_POOL_RMSNORM)) return QSA_ERR_INVALID_ARG;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (batch == 0 || block_end == block_begin) return QSA_OK;
    if (!aligned16(raw_keys) || !aligned16(pooled)) return QSA_ERR_INVALID_ARG;
    if (raw_seq_stride % 8 || pooled_seq_stride % 8) return QSA_ERR_INVALID_ARG;
    if (batch > 1 && (raw_seq_stride < (int64_t)kBlock * block_end * kDim || pooled_seq_stride < (int64_t)block_end * kDim))
        return QSA_ERR_INVALID_ARG;
    clear_launch_err();
    launch_pool(raw_keys, raw_seq_stride, pooled, pooled_seq_stride, KeyPages{nullptr, 0, 0}, batch, block_begin,
                block_end, rope_freq_plain(rope_theta), flags, dtype == QSA_BF16, (hipStream_t)stream);
    return launch_status();
}

qsa_status_t qsa_pool_index_keys_fp8(const void *raw_keys, int64_t raw_seq_stride, uint8_t *codes, float *scales,
                                     int64_t pooled_seq_stride, int32_t batch, int32_t block_begin, int32_t block_end,
                                     double rope_theta, uint32_t flags, qsa_dtype_t raw_dtype, void *stream)
{
    if (!dtype_ok(raw_dtype)) return QSA_ERR_UNSUPPORTED;
    if (batch < 0 || block_begin < 0 || block_end < block_begin) return QSA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(QSA_FLAG_NO_ROPE | QSA_FLAG_POOL_RMSNORM)) return QSA_ERR_INVALID_ARG;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (batch == 0 || block_end == block_begin) return QSA_OK;
    if (!aligned16(raw_keys) || !aligned16(codes) || !scales || (reinterpret_cast<uintptr_t>(scales) & 3u))
        return QSA_ERR_INVALID_ARG;
    if (raw_seq_stride % 8 || pooled_seq_stride < 0) return QSA_ERR_INVALID_ARG;
    if (batch > 1 && (raw_seq_stride < (int64_t)kBlock * block_end * kDim || pooled_seq_stride < (int64_t)block_end))
        return QSA_ERR_INVALID_ARG;
    clear_launch_err();
    launch_pool_fp8(raw_keys, raw_seq_stride, codes, scales, pooled_seq_stride, KeyPages{nullptr, 0, 0}, batch,
                    block_begin, block_end, rope_freq_plain(rope_theta), flags, raw_dtype == QSA_BF16,
                    (hipStream_t)stream);
    return launch_status();
}

qsa_status_t qsa_pool_index_keys_paged(const void *raw_keys, int64_t raw_seq_stride, void *pooled, uint8_t *codes,
                                       float *scales, const int32_t *page_table, int64_t page_table_stride,
                                       int32_t page_tokens, int32_t batch, int32_t block_begin, int32_t block_end,
                                       double rope_theta, uint32_t flags, qsa_dtype_t raw_dtype, void *stream)
{
    const bool fp8 = codes != nullptr;
    if (!dtype_ok(raw_dtype)) return QSA_ERR_UNSUPPORTED;
    if (batch < 0 || block_begin < 0 || block_end < block_begin) return QSA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(QSA_FLAG_NO_ROPE | QSA_FLAG_POOL_RMSNORM)) return QSA_ERR_INVALID_ARG;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (page_tokens < kBlock || page_tokens % kBlock || page_table_stride < 0) return QSA_ERR_INVALID_ARG;
    if (batch == 0 || block_end == block_begin) return QSA_OK;
    if (!aligned16(raw_keys) || raw_seq_stride % 8 || !page_table) return QSA_ERR_INVALID_ARG;
    if (fp8 ? (!aligned16(codes) || !scales || (reinterpret_cast<uintptr_t>(scales) & 3u) || pooled)
            : (!aligned16(pooled) || scales))
        return QSA_ERR_INVALID_ARG;
    if (batch > 1 && raw_seq_stride < (int64_t)kBlock * block_end * kDim) return QSA_ERR_INVALID_ARG;
    const int32_t bpp = page_tokens / kBlock;
    if ((int64_t)block_end > page_table_stride * bpp) return QSA_ERR_INVALID_ARG;  // the table covers the blocks
    const KeyPages kp{page_table, page_table_stride, bpp};
    clear_launch_err();
    if (fp8)
        launch_pool_fp8(raw_keys, raw_seq_stride, codes, scales, 0, kp, batch, block_begin, block_end,
                        rope_freq_plain(rope_theta), flags, raw_dtype == QSA_BF16, (hipStream_t)stream);
    else
        launch_pool(raw_keys, raw_seq_stride, pooled, 0, kp, batch, block_begin, block_end,
                    rope_freq_plain(rope_theta), flags, raw_dtype == QSA_BF16, (hipStream_t)stream);
    return launch_status();
}

qsa_status_t qsa_pool_append(const void *new_keys, const int32_t *positions, const int64_t *full_slots, void *ring,
                             void *compressed, int32_t batch, double rope_theta, uint32_t flags, qsa_dtype_t dtype,
                             void *stream)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (batch < 0) return QSA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(QSA_FLAG_NO_ROPE | QSA_FLAG_POOL_RMSNORM)) return QSA_ERR_INVALID_ARG;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (batch == 0) return QSA_OK;
    if (!aligned16(new_keys) || !aligned16(ring) || !aligned16(compressed) || !positions || !full_slots)
        return QSA_ERR_INVALID_ARG;
    clear_launch_err();
    launch_pool_append(new_keys, positions, full_slots, ring, compressed, batch, rope_freq_plain(rope_theta), flags,
                       dtype == QSA_BF16, (hipStream_t)stream);
    return launch_status();
}

// qsa_rope_t: a valid rotation (unused with QSA_FLAG_NO_ROPE, where it may be NULL).
static bool rope_ok(const qsa_rope_t *r, uint32_t flags)
{
    if (flags & QSA_FLAG_NO_ROPE) return true;
    if (!r || !(r->theta > 1.0 && std::isfinite(r->theta))) return false;
    if (!(r->yarn_factor >= 1.0 && std::isfinite(r->yarn_factor))) return false;
    if (r->yarn_factor == 1.0) return true;
    return r->yarn_original_context > 0.0 && std::isfinite(r->yarn_original_context) && r->yarn_alpha >= 0.0 &&
           std::isfinite(r->yarn_beta) && r->yarn_beta > r->yarn_alpha;
}

static RopeFreq rope_freq_of(const qsa_rope_t *r, uint32_t flags)
{
    if ((flags & QSA_FLAG_NO_ROPE) || !r) return RopeFreq{};  // not read by the kernels
    return rope_freq_yarn(r->theta, r->yarn_factor, r->yarn_original_context, r->yarn_alpha, r->yarn_beta);
}

qsa_status_t qsa_pool_index_keys_ex(const void *raw_keys, int64_t raw_seq_stride, void *pooled,
                                    int64_t pooled_seq_stride, int32_t batch, int32_t block_begin, int32_t block_end,
                                    const qsa_rope_t *rope, const float *norm_weight, uint32_t flags,
                                    qsa_dtype_t dtype, void *stream)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (batch < 0 || block_begin < 0 || block_end < block_begin) return QSA_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)(QSA_FLAG_NO_ROPE | QSA_FLAG_POOL_RMSNORM)) return QSA_ERR_INVALID_ARG;
    if (!rope_ok(rope, flags)) return QSA_ERR_INVALID_ARG;
    if (norm_weight && (!(flags & QSA_FLAG_POOL_RMSNORM) || (reinterpret_cast<uintptr_t>(norm_weight) & 3u)))
        return QSA_ERR_INVALID_ARG;
    if (batch == 0 || block_end == block_begin) return QSA_OK;
    if (!aligned16(raw_keys) || !aligned16(pooled)) return QSA_ERR_INVALID_ARG;
    if (raw_seq_stride % 8 || pooled_seq_stride % 8) return QSA_ERR_INVALID_ARG;
    if (batch > 1 && (raw_seq_stride < (int64_t)kBlock * block_end * kDim || pooled_seq_stride < (int64_t)block_end * kDim))
        return QSA_ERR_INVALID_ARG;
    clear_launch_err();
    launch_pool(raw_keys, raw_seq_stride, pooled, pooled_seq_stride, KeyPages{nullptr, 0, 0}, batch, block_begin,
                block_end, rope_freq_of(rope, flags), flags, dtype == QSA_BF16, (hipStream_t)stream, norm_weight);
    return launch_status();
}

size_t qsa_score_topk_workspace_size(int32_t rows, int32_t max_visible_blocks, int32_t top_k, qsa_dtype_t dtype,
                                     uint32_t flags)
{
    if (rows <= 0 || max_visible_blocks < 0 || top_k < 1 || top_k > QSA_MAX_TOP_K || !dtype_ok(dtype)) return 0;
    if (!score_flags_ok(flags, dtype)) return 0;
    return score_layout(rows, max_visible_blocks, top_k, dtype, flags).total;
}

size_t qsa_score_topk_merge_modes_offset(int32_t rows, int32_t max_visible_blocks, int32_t top_k, qsa_dtype_t dtype,
                                         uint32_t flags)
{
    if (qsa_score_topk_workspace_size(rows, max_visible_blocks, top_k, dtype, flags) == 0) return (size_t)-1;
    const ScoreLayout L = score_layout(rows, max_visible_blocks, top_k, dtype, flags);
    return L.plan.fused ? L.mode_off : (size_t)-1;
}

size_t qsa_score_topk_fp8_workspace_size(int32_t rows, int32_t max_visible_blocks, int32_t top_k, uint32_t flags)
{
    return qsa_score_topk_workspace_size(rows, max_visible_blocks, top_k, QSA_BF16, flags);
}

qsa_status_t qsa_score_topk(const void *q_index, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                            const void *pooled, int64_t pooled_seq_stride, int32_t max_visible_blocks, int32_t top_k,
                            double rope_theta, uint32_t flags, qsa_dtype_t dtype, int32_t *sel_blocks,
                            int32_t *sel_count, float *sel_scores, void *workspace, size_t workspace_bytes,
                            void *stream)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (rows < 0 || max_visible_blocks < 0 || top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
    if (!score_flags_ok(flags, dtype)) return QSA_ERR_INVALID_ARG;
    if ((flags & QSA_FLAG_SCORE_GEMM) && dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (rows == 0) return QSA_OK;
    if (!aligned16(q_index) || !aligned16(pooled) || !row_seq || !row_pos || !sel_blocks || !sel_count)
        return QSA_ERR_INVALID_ARG;
    if (pooled_seq_stride % 8 || pooled_seq_stride < 0) return QSA_ERR_INVALID_ARG;
    const KeySource keys{pooled, nullptr, nullptr, KeyPages{nullptr, 0, 1}};
    return score_topk_run(q_index, row_seq, row_pos, rows, keys, pooled_seq_stride, max_visible_blocks, top_k,
                          rope_freq_plain(rope_theta), flags, dtype, sel_blocks, sel_count, sel_scores, workspace,
                          workspace_bytes, stream);
}

qsa_status_t qsa_score_topk_ex(const void *q_index, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                               const void *pooled, int64_t pooled_seq_stride, int32_t max_visible_blocks,
                               int32_t top_k, const qsa_rope_t *rope, uint32_t flags, qsa_dtype_t dtype,
                               int32_t *sel_blocks, int32_t *sel_count, float *sel_scores, void *workspace,
                               size_t workspace_bytes, void *stream)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (rows < 0 || max_visible_blocks < 0 || top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
    if (!score_flags_ok(flags, dtype)) return QSA_ERR_INVALID_ARG;
    if ((flags & QSA_FLAG_SCORE_GEMM) && dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
    if (!rope_ok(rope, flags)) return QSA_ERR_INVALID_ARG;
    if (rows == 0) return QSA_OK;
    if (!aligned16(q_index) || !aligned16(pooled) || !row_seq || !row_pos || !sel_blocks || !sel_count)
        return QSA_ERR_INVALID_ARG;
    if (pooled_seq_stride % 8 || pooled_seq_stride < 0) return QSA_ERR_INVALID_ARG;
    const KeySource keys{pooled, nullptr, nullptr, KeyPages{nullptr, 0, 1}};
    return score_topk_run(q_index, row_seq, row_pos, rows, keys, pooled_seq_stride, max_visible_blocks, top_k,
                          rope_freq_of(rope, flags), flags, dtype, sel_blocks, sel_count, sel_scores, workspace,
                          workspace_bytes, stream);
}

qsa_status_t qsa_score_topk_fp8(const void *q_index, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                                const uint8_t *codes, const float *scales, int64_t pooled_seq_stride,
                                int32_t max_visible_blocks, int32_t top_k, double rope_theta, uint32_t flags,
                                int32_t *sel_blocks, int32_t *sel_count, float *sel_scores, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    if (rows < 0 || max_visible_blocks < 0 || top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
    if (!score_flags_ok(flags, QSA_BF16)) return QSA_ERR_INVALID_ARG;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (rows == 0) return QSA_OK;
    if (!aligned16(q_index) || !aligned16(codes) || !scales || (reinterpret_cast<uintptr_t>(scales) & 3u) || !row_seq ||
        !row_pos || !sel_blocks || !sel_count)
        return QSA_ERR_INVALID_ARG;
    if (pooled_seq_stride < 0) return QSA_ERR_INVALID_ARG;
    const KeySource keys{nullptr, codes, scales, KeyPages{nullptr, 0, 1}};
    return score_topk_run(q_index, row_seq, row_pos, rows, keys, pooled_seq_stride, max_visible_blocks, top_k,
                          rope_freq_plain(rope_theta), flags, QSA_BF16, sel_blocks, sel_count, sel_scores, workspace,
                          workspace_bytes, stream);
}

qsa_status_t qsa_score_topk_paged(const void *q_index, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                                  const void *pooled, const uint8_t *codes, const float *scales,
                                  const int32_t *page_table, int64_t page_table_stride, int32_t page_tokens,
                                  int32_t max_visible_blocks, int32_t top_k, double rope_theta, uint32_t flags,
                                  qsa_dtype_t dtype, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    const bool fp8 = codes != nullptr;
    if (!fp8 && !dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (fp8 && dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;  // FP8 keys go with bf16 index queries
    if (rows < 0 || max_visible_blocks < 0 || top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
    if (!score_flags_ok(flags, dtype)) return QSA_ERR_INVALID_ARG;
    if ((flags & QSA_FLAG_SCORE_GEMM) && dtype != QSA_BF16) return QSA_ERR_UNSUPPORTED;
    if (!(flags & QSA_FLAG_NO_ROPE) && !(rope_theta > 1.0 && std::isfinite(rope_theta))) return QSA_ERR_INVALID_ARG;
    if (page_tokens < kBlock || page_tokens % kBlock || page_table_stride < 0) return QSA_ERR_INVALID_ARG;
    if (rows == 0) return QSA_OK;
    if (!aligned16(q_index) || !row_seq || !row_pos || !sel_blocks || !sel_count || !page_table)
        return QSA_ERR_INVALID_ARG;
    if (fp8 ? (!aligned16(codes) || !scales || (reinterpret_cast<uintptr_t>(scales) & 3u) || pooled)
            : (!aligned16(pooled) || scales))
        return QSA_ERR_INVALID_ARG;
    if ((int64_t)max_visible_blocks * kBlock > page_table_stride * (int64_t)page_tokens) return QSA_ERR_INVALID_ARG;
    const KeySource keys{fp8 ? nullptr : pooled, codes, scales, KeyPages{page_table, page_table_stride, page_tokens / kBlock}};
    return score_topk_run(q_index, row_seq, row_pos, rows, keys, 0, max_visible_blocks, top_k,
                          rope_freq_plain(rope_theta), flags, dtype, sel_blocks, sel_count, sel_scores, workspace,
                          workspace_bytes, stream);
}

}  // extern "C"

// The launches of qsa_score_topk / qsa_score_topk_fp8 after validation.
// FP8 keys go with bf16 index queries (the same layout and kernels, with the
// codes converted to bf16 on the way to the MFMA).
static qsa_status_t score_topk_run(const void *q_index, const int32_t *row_seq, const int32_t *row_pos,
                                   int32_t rows, const KeySource &keys, int64_t pooled_seq_stride,
                                   int32_t max_visible_blocks, int32_t top_k, const RopeFreq &rf, uint32_t flags,
                                   qsa_dtype_t dtype, int32_t *sel_blocks, int32_t *sel_count, float *sel_scores,
                                   void *workspace, size_t workspace_bytes, void *stream)
{
    const ScoreLayout L = score_layout(rows, max_visible_blocks, top_k, dtype, flags);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return QSA_ERR_INVALID_ARG;
    if (workspace_bytes < L.total) return QSA_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const bool bf16 = dtype == QSA_BF16;
    char *ws = (char *)workspace;
    void *qrot = ws + L.qrot_off;
    SplitSelect ss{};
    if (L.plan.split) {
        ss.scratch = (uint32_t *)(ws + L.scratch_off);
        ss.sure = (uint2 *)(ws + L.sure_off);
        ss.cand = (uint2 *)(ws + L.cand_off);
        ss.cand_stride = L.sc_stride;
    }
    clear_launch_err();
    launch_rope_query(q_index, row_pos, rows, qrot, rf, flags & QSA_FLAG_NO_ROPE, bf16,
                      L.plan.split ? ss.scratch : nullptr, kRowScratch, st);
    if (L.plan.fused) {
        FusedScoreArgs fa{};
        fa.qrot = (const uint16_t *)qrot;
        fa.row_seq = row_seq;
        fa.row_pos = row_pos;
        fa.rows = rows;
        fa.pooled = (const uint16_t *)keys.pooled;
        fa.codes = keys.codes;
        fa.scales = keys.scales;
        fa.kp = keys.kp;
        fa.pooled_stride = pooled_seq_stride;
        fa.max_nb = max_visible_blocks;
        fa.top_k = top_k;
        fa.nsplit = L.nsplit;
        fa.split_len = L.split_len;
        fa.subcap = L.subcap;
        fa.buf = (uint2 *)(ws + L.buf_off);
        fa.cnt = (uint32_t *)(ws + L.cnt_off);
        fa.nsample = L.nsample;
        fa.ssplit = L.ssplit;
        fa.cand = (uint32_t *)(ws + L.scand_off);
        fa.tau = (uint32_t *)(ws + L.tau_off);
        fa.mode = (int32_t *)(ws + L.mode_off);
        launch_score_fused(fa, sel_blocks, sel_count, sel_scores, st);
        return launch_status();
    }
    float *scores = (float *)(ws + L.scores_off);
    if (max_visible_blocks > 0) {
        if (keys.codes)
            launch_score_rows_fp8(qrot, row_seq, row_pos, rows, keys.codes, keys.scales, pooled_seq_stride, keys.kp,
                                  max_visible_blocks, scores, L.sc_stride, L.plan.split ? ss.scratch : nullptr, st);
        else
            launch_score_rows(qrot, row_seq, row_pos, rows, keys.pooled, pooled_seq_stride, keys.kp,
                              max_visible_blocks, scores, L.sc_stride, L.plan.split ? ss.scratch : nullptr, bf16, st);
    }
    if (L.plan.split)
        launch_select_split(scores, L.sc_stride, row_pos, rows, max_visible_blocks, top_k, ss, sel_blocks, sel_count,
                            sel_scores, st);
    else
        launch_select_rows(scores, L.sc_stride, row_pos, rows, max_visible_blocks, top_k, sel_blocks, sel_count,
                           sel_scores, st);
    return launch_status();
}

// ---------------------------------------------------------------------------
// Allocation-free decode (qsa_sparse_attn_decode_noalloc): the split partials
// live in this file-scope device array instead of a caller's workspace.  Every
// GPU the library runs on holds its own copy until the process ends.  In host
// code `scratch` names a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is ever handed to a kernel.  Calls that overlap on one
// GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once known
std::mutex g_scratch_mutex;
}  // namespace

// The current device's copy of `scratch` (null if it cannot be resolved).
static void *noalloc_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void *addr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !addr) {
        g_launch_err = g_last_failure = err != hipSuccess ? err : hipErrorInvalidSymbol;
        return nullptr;
    }
    g_scratch_ptr[dev].store(addr, std::memory_order_release);
    return addr;
}

extern "C" {

static qsa_status_t check_attn_common(const void *q, const void *k_cache, const void *v_cache, int64_t kv_seq_stride,
                                      const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                      int32_t Hkv, int32_t D, float softmax_scale, qsa_dtype_t dtype, const void *out,
                                      bool kv_fp8 = false)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return QSA_ERR_INVALID_ARG;
    if (top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
    if (!std::isfinite(softmax_scale)) return QSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !sel_blocks || !sel_count || !out)
        return QSA_ERR_INVALID_ARG;
    if (kv_seq_stride < 0 || kv_seq_stride % (kv_fp8 ? 16 : 8)) return QSA_ERR_INVALID_ARG;  // 16-byte rows
    return QSA_OK;
}

// FP8 K/V: the two per-tensor scales must be positive and finite.
static bool kv_scales_ok(float k_scale, float v_scale)
{
    return std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.0f && v_scale > 0.0f;
}

static qsa_status_t attn_prefill_impl(const void *q, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                                     const void *k_cache, const void *v_cache, int64_t kv_seq_stride,
                                     const int32_t *page_table, int64_t pt_stride, int32_t page_tokens,
                                     const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                     int32_t Hkv, int32_t D, float softmax_scale, qsa_dtype_t dtype, void *out,
                                     float *lse, void *stream, bool kv_fp8 = false, float k_scale = 1.0f,
                                     float v_scale = 1.0f)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (rows < 0) return QSA_ERR_INVALID_ARG;
    if (D != kDim && D != kDimWide) return QSA_ERR_UNSUPPORTED;
    if (Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && Hq / Hkv > QSA_MAX_QUERY_GROUP) return QSA_ERR_UNSUPPORTED;
    const bool mfma = attn_mfma_supported(Hq, Hkv, 1, D, dtype == QSA_BF16);
    if (D == kDimWide && !mfma) return QSA_ERR_UNSUPPORTED;  // D = 256 lives in the bf16 MFMA kernels
    if (kv_fp8 && !mfma) return QSA_ERR_UNSUPPORTED;         // and so do FP8 K/V
    if (kv_fp8 && !kv_scales_ok(k_scale, v_scale)) return QSA_ERR_INVALID_ARG;
    if (rows == 0) {
        if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
        return QSA_OK;
    }
    qsa_status_t st = check_attn_common(q, k_cache, v_cache, kv_seq_stride, sel_blocks, sel_count, top_k, Hq, Hkv, D,
                                        softmax_scale, dtype, out, kv_fp8);
    if (st != QSA_OK) return st;
    if (!row_seq || !row_pos) return QSA_ERR_INVALID_ARG;
    AttnArgs a{};
    a.q = q;
    a.row_seq = row_seq;
    a.row_pos = row_pos;
    a.tail_start = nullptr;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.kv_seq_stride = kv_seq_stride;
    a.sel_blocks = sel_blocks;
    a.sel_count = sel_count;
    a.top_k = top_k;
    a.n_sel = rows;
    a.q_per_sel = 1;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.scale = softmax_scale;
    a.out = out;
    a.lse = lse;
    a.partial = nullptr;
    a.nsplit = 1;
    a.page_table = page_table;
    a.pt_stride = pt_stride;
    a.page_tokens = page_tokens;
    a.kv_fp8 = kv_fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    if (page_table && !mfma) return QSA_ERR_UNSUPPORTED;  // the paged gather lives in the MFMA kernels
    clear_launch_err();
    if (mfma)
        launch_attn_prefill_mfma(a, (hipStream_t)stream);
    else
        launch_attn_prefill(a, dtype == QSA_BF16, (hipStream_t)stream);
    return launch_status();
}

qsa_status_t qsa_sparse_attn_prefill(const void *q, const int32_t *row_seq, const int32_t *row_pos, int32_t rows,
                                     const void *k_cache, const void *v_cache, int64_t kv_seq_stride,
                                     const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k, int32_t Hq,
                                     int32_t Hkv, int32_t D, float softmax_scale, qsa_dtype_t dtype, void *out,
                                     float *lse, void *stream)
{
    return attn_prefill_impl(q, row_seq, row_pos, rows, k_cache, v_cache, kv_seq_stride, nullptr, 0, 0, sel_blocks,
                             sel_count, top_k, Hq, Hkv, D, softmax_scale, dtype, out, lse, stream);
}

qsa_status_t qsa_sparse_attn_prefill_paged(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                           int32_t rows, const void *k_cache, const void *v_cache,
                                           const int32_t *page_table, int64_t page_table_stride, int32_t page_tokens,
                                           const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k,
                                           int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale, qsa_dtype_t dtype,
                                           void *out, float *lse, void *stream)
{
    if (page_tokens < kBlock || page_tokens % kBlock || page_table_stride < 0) return QSA_ERR_INVALID_ARG;
    if (rows > 0 && !page_table) return QSA_ERR_INVALID_ARG;
    return attn_prefill_impl(q, row_seq, row_pos, rows, k_cache, v_cache, 0, page_table, page_table_stride,
                             page_tokens, sel_blocks, sel_count, top_k, Hq, Hkv, D, softmax_scale, dtype, out, lse,
                             stream);
}

size_t qsa_sparse_attn_decode_workspace_size(int32_t batch, int32_t q_per_seq, int32_t Hq, int32_t D, int32_t top_k)
{
    if (batch <= 0 || q_per_seq <= 0 || Hq <= 0 || (D != kDim && D != kDimWide) || top_k < 1 ||
        top_k > QSA_MAX_TOP_K)
        return 0;
    const size_t nsplit = (size_t)attn_decode_splits(top_k);
    return align256((size_t)batch * q_per_seq * Hq * nsplit * (D + 2) * sizeof(float));
}

// Splits of the MFMA decode attention.  One split of 16 kept blocks per
// workgroup while the launch fits one round of resident workgroups (two per CU
// at this kernel's register use, 256 CUs).  A launch of two to four rounds
// whose splits, merged `rounds` at a time, fit one round gives each workgroup
// that many 16-block groups instead (a workgroup's chunks then run back to
// back, and the last rounds' start-up waits are gone); larger launches keep
// one group per workgroup.  The kernel derives a split's length from the
// count; the workspace of qsa_sparse_attn_decode_workspace_size (one split per
// 16 blocks) covers any of these.
constexpr int64_t kDecodeResident = 2 * 256;
static int32_t attn_decode_mfma_splits(int32_t top_k, int32_t batch, int32_t Hkv)
{
    const int64_t n16 = attn_decode_splits(top_k) - 1;  // 16-block groups of the selection
    const int64_t rows = (int64_t)batch * Hkv;
    const int64_t rounds = ((n16 + 1) * rows + kDecodeResident - 1) / kDecodeResident;
    if (rounds <= 1 || rounds > 4) return (int32_t)(n16 + 1);
    const int64_t merged = (n16 + rounds - 1) / rounds + 1;
    return merged * rows <= kDecodeResident ? (int32_t)merged : (int32_t)(n16 + 1);
}

static qsa_status_t attn_decode_impl(const void *q, const int32_t *row_pos, int32_t batch, int32_t q_per_seq,
                                    const int32_t *tail_start, const void *k_cache, const void *v_cache,
                                    int64_t kv_seq_stride, const int32_t *page_table, int64_t pt_stride,
                                    int32_t page_tokens, const int32_t *sel_blocks, const int32_t *sel_count,
                                    int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                    qsa_dtype_t dtype, void *out, float *lse, void *workspace, size_t workspace_bytes,
                                    void *stream, bool kv_fp8 = false, float k_scale = 1.0f, float v_scale = 1.0f,
                                    bool static_scratch = false)
{
    if (!dtype_ok(dtype)) return QSA_ERR_UNSUPPORTED;
    if (batch < 0 || q_per_seq < 1) return QSA_ERR_INVALID_ARG;
    if (D != kDim && D != kDimWide) return QSA_ERR_UNSUPPORTED;
    if (Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && (int64_t)q_per_seq * (Hq / Hkv) > QSA_MAX_QUERY_GROUP)
        return QSA_ERR_UNSUPPORTED;
    const bool mfma = attn_mfma_supported(Hq, Hkv, q_per_seq, D, dtype == QSA_BF16);
    if (D == kDimWide && !mfma) return QSA_ERR_UNSUPPORTED;  // D = 256 lives in the bf16 MFMA kernels
    if (kv_fp8 && !mfma) return QSA_ERR_UNSUPPORTED;         // and so do FP8 K/V
    if (kv_fp8 && !kv_scales_ok(k_scale, v_scale)) return QSA_ERR_INVALID_ARG;
    if (batch == 0) {
        if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || top_k < 1 || top_k > QSA_MAX_TOP_K) return QSA_ERR_INVALID_ARG;
        return QSA_OK;
    }
    qsa_status_t st = check_attn_common(q, k_cache, v_cache, kv_seq_stride, sel_blocks, sel_count, top_k, Hq, Hkv, D,
                                        softmax_scale, dtype, out, kv_fp8);
    if (st != QSA_OK) return st;
    if (!row_pos) return QSA_ERR_INVALID_ARG;
    const size_t need = qsa_sparse_attn_decode_workspace_size(batch, q_per_seq, Hq, D, top_k);
    if (static_scratch) {  // the library's own scratch array; the first HIP call of this path
        if (need > (size_t)QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_WORKSPACE;
        workspace = noalloc_scratch();
        if (!workspace) return QSA_ERR_DEVICE;
        workspace_bytes = QSA_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return QSA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return QSA_ERR_WORKSPACE;
    AttnArgs a{};
    a.q = q;
    a.row_seq = nullptr;
    a.row_pos = row_pos;
    a.tail_start = tail_start;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.kv_seq_stride = kv_seq_stride;
    a.sel_blocks = sel_blocks;
    a.sel_count = sel_count;
    a.top_k = top_k;
    a.n_sel = batch;
    a.q_per_sel = q_per_seq;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.scale = softmax_scale;
    a.out = out;
    a.lse = lse;
    a.partial = (float *)workspace;
    a.nsplit = mfma ? attn_decode_mfma_splits(top_k, batch, Hkv) : attn_decode_splits(top_k);
    a.page_table = page_table;
    a.pt_stride = pt_stride;
    a.page_tokens = page_tokens;
    a.kv_fp8 = kv_fp8;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    if (page_table && !mfma) return QSA_ERR_UNSUPPORTED;  // the paged gather lives in the MFMA kernels
    clear_launch_err();
    if (mfma) {
        launch_attn_decode_mfma(a, (hipStream_t)stream);
        launch_attn_combine(a, true, (hipStream_t)stream);
    } else {
        launch_attn_decode(a, dtype == QSA_BF16, (hipStream_t)stream);
    }
    return launch_status();
}

qsa_status_t qsa_sparse_attn_decode(const void *q, const int32_t *row_pos, int32_t batch, int32_t q_per_seq,
                                    const int32_t *tail_start, const void *k_cache, const void *v_cache,
                                    int64_t kv_seq_stride, const int32_t *sel_blocks, const int32_t *sel_count,
                                    int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                    qsa_dtype_t dtype, void *out, float *lse, void *workspace, size_t workspace_bytes,
                                    void *stream)
{
    return attn_decode_impl(q, row_pos, batch, q_per_seq, tail_start, k_cache, v_cache, kv_seq_stride, nullptr, 0, 0,
                            sel_blocks, sel_count, top_k, Hq, Hkv, D, softmax_scale, dtype, out, lse, workspace,
                            workspace_bytes, stream);
}

qsa_status_t qsa_sparse_attn_decode_noalloc(const void *q, const int32_t *row_pos, int32_t batch, int32_t q_per_seq,
                                            const int32_t *tail_start, const void *k_cache, const void *v_cache,
                                            int64_t kv_seq_stride, const int32_t *sel_blocks, const int32_t *sel_count,
                                            int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                            qsa_dtype_t dtype, void *out, float *lse, void *stream)
{
    return attn_decode_impl(q, row_pos, batch, q_per_seq, tail_start, k_cache, v_cache, kv_seq_stride, nullptr, 0, 0,
                            sel_blocks, sel_count, top_k, Hq, Hkv, D, softmax_scale, dtype, out, lse, nullptr, 0,
                            stream, false, 1.0f, 1.0f, true);
}

qsa_status_t qsa_sparse_attn_decode_paged(const void *q, const int32_t *row_pos, int32_t batch, int32_t q_per_seq,
                                          const int32_t *tail_start, const void *k_cache, const void *v_cache,
                                          const int32_t *page_table, int64_t page_table_stride, int32_t page_tokens,
                                          const int32_t *sel_blocks, const int32_t *sel_count, int32_t top_k,
                                          int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale, qsa_dtype_t dtype,
                                          void *out, float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    if (page_tokens < kBlock || page_tokens % kBlock || page_table_stride < 0) return QSA_ERR_INVALID_ARG;
    if (batch > 0 && !page_table) return QSA_ERR_INVALID_ARG;
    return attn_decode_impl(q, row_pos, batch, q_per_seq, tail_start, k_cache, v_cache, 0, page_table,
                            page_table_stride, page_tokens, sel_blocks, sel_count, top_k, Hq, Hkv, D, softmax_scale,
                            dtype, out, lse, workspace, workspace_bytes, stream);
}

qsa_status_t qsa_sparse_attn_prefill_fp8kv(const void *q, const int32_t *row_seq, const int32_t *row_pos,
                                           int32_t rows, const uint8_t *k_codes, const uint8_t *v_codes,
                                           int64_t kv_seq_stride, const int32_t *page_table,
                                           int64_t page_table_stride, int32_t page_tokens, float k_scale,
                                           float v_scale, const int32_t *sel_blocks, const int32_t *sel_count,
                                           int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                           void *out, float *lse, void *stream)
{
    if (page_table && (page_tokens < kBlock || page_tokens % kBlock || page_table_stride < 0))
        return QSA_ERR_INVALID_ARG;
    return attn_prefill_impl(q, row_seq, row_pos, rows, k_codes, v_codes, page_table ? 0 : kv_seq_stride,
                             page_table, page_table_stride, page_tokens, sel_blocks, sel_count, top_k, Hq, Hkv, D,
                             softmax_scale, QSA_BF16, out, lse, stream, true, k_scale, v_scale);
}

qsa_status_t qsa_sparse_attn_decode_fp8kv(const void *q, const int32_t *row_pos, int32_t batch, int32_t q_per_seq,
                                          const int32_t *tail_start, const uint8_t *k_codes, const uint8_t *v_codes,
                                          int64_t kv_seq_stride, const int32_t *page_table,
                                          int64_t page_table_stride, int32_t page_tokens, float k_scale,
                                          float v_scale, const int32_t *sel_blocks, const int32_t *sel_count,
                                          int32_t top_k, int32_t Hq, int32_t Hkv, int32_t D, float softmax_scale,
                                          void *out, float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream)
{
    if (page_table && (page_tokens < kBlock || page_tokens % kBlock || page_table_stride < 0))
        return QSA_ERR_INVALID_ARG;
    return attn_decode_impl(q, row_pos, batch, q_per_seq, tail_start, k_codes, v_codes,
                            page_table ? 0 : kv_seq_stride, page_table, page_table_stride, page_tokens, sel_blocks,
                            sel_count, top_k, Hq, Hkv, D, softmax_scale, QSA_BF16, out, lse, workspace,
                            workspace_bytes, stream, true, k_scale, v_scale);
}

qsa_status_t qsa_profile_enable(int enable)
{
    g_prof.store(enable != 0, std::memory_order_relaxed);
    return QSA_OK;
}

qsa_status_t qsa_profile_reset(void)
{
    std::lock_guard<std::mutex> lock(g_prof_mutex);
    for (auto &r : g_records) {
        g_free_events.push_back(r.start);
        g_free_events.push_back(r.stop);
    }
    g_records.clear();
    return QSA_OK;
}

int32_t qsa_profile_kernel_ms(const char *name, double *total_ms)
{
    double total = 0.0;
    int32_t n = 0;
    if (name) {
        std::vector<ProfRecord> mine;
        {
            std::lock_guard<std::mutex> lock(g_prof_mutex);
            for (auto &r : g_records)
                if (r.name == name) mine.push_back(r);
        }
        for (auto &r : mine) {  // waits outside the lock
            if (hipEventSynchronize(r.stop) != hipSuccess) continue;
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) continue;
            total += ms;
            ++n;
        }
    }
    if (total_ms) *total_ms = total;
    return n;
}

}  // extern "C"
