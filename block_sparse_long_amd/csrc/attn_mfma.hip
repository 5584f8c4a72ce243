// attn_mfma.hip -- steps a7-a9 on bf16 MFMA: gather attention over the kept
// blocks plus the tail, shared by the query rows of a workgroup.
//
// "Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
// Attention": each kept block stands for its 4 token positions, the
// zero-to-three tail tokens of the query's incomplete block are appended, and
// attention reads the original K/V at those positions.  Section "IndexShare
// MTP": draft rows share one selection plus the positions drafted since.
// Readings: query head h uses KV head floor(h / (Hq/Hkv)); logits are
// softmax_scale * <q, k>; P is rounded to bf16 as an MFMA operand.  K/V are
// bf16, or FP8 E4M3 codes with one scale per cache tensor ("Qwen3.8-Flash-
// Next, Layer by Layer", section "Serving it"), widened to bf16 on their way
// into LDS; the caches are contiguous per sequence or a paged pool.
//
// Layout of the work.  A workgroup owns up to 64 queries that share one KV
// head: (rows of the tile) x (Hq/Hkv heads), as 4 MFMA tiles of 16 queries,
// one per wave.  It walks a list of positions in chunks (64 positions at head
// dim D = 128, 32 at D = 256, so a chunk is 16 KiB of K and of V either way):
// the chunk's K rows (row-major) and V rows (transposed) are gathered into LDS
// once and every wave computes S^T = K Q^T for its 16 queries
// (v_mfma_f32_16x16x32_bf16, positions on M, queries on N), an online
// softmax, then O += P V (queries on M, head dims on N).  Each position of a chunk carries a mask of the query
// rows that attend it, so one gathered chunk serves every row of the tile:
//   - prefill: the tile is up to 64/(Hq/Hkv) consecutive rows; the position
//     list is the union of their kept blocks (built in LDS with a bitmap per
//     window of 65,536 blocks) followed by each row's tail tokens;
//   - decode: the rows of one sequence share its selection; a workgroup takes
//     a split of 16 kept blocks (one or two chunks; several 16-block groups
//     when the caller merges splits) or the tail, and a combine kernel merges
//     the splits' partial softmaxes.
// A wave skips the MFMAs of a 16-position sub-tile that none of its rows
// attends, so disjoint selections cost gathers but not matrix work.
//
// MFMA operand layout (16x16x32): lane l supplies A[m = l%16][8 k-slots of
// group l/16] and B[8 k-slots of group l/16][n = l%16] and receives
// C[4*(l/16) + j][l%16].  For S^T = K Q^T the k-slots of group g at step s
// are head dims (D/4)g + 8s .. +7.  For O = P V, a 32-position step covers
// sub-tiles 2i and 2i+1; group g's slots 0-3 are positions 4g..4g+3 of
// sub-tile 2i and slots 4-7 those of sub-tile 2i+1 -- exactly the S^T values
// the lane already holds, so P needs no shuffle.
#include <type_traits>

#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

// Shapes of one chunk at head dim DIM.
template <int DIM>
struct Geo {
    static_assert(DIM == 128 || DIM == 256, "head dims 128 and 256");
    static constexpr int kCh = 8192 / DIM;    // positions per chunk: 64 or 32
    static constexpr int kKRow = DIM + 8;     // LDS row stride of K (bf16): 4 banks of skew per row
    static constexpr int kVRow = kCh + 8;     // LDS row stride of V^T (bf16), a multiple of 16 bytes
    static constexpr int kSub = kCh / 16;     // 16-position sub-tiles of S^T
    static constexpr int kKs = DIM / 32;      // k-steps of S^T
    static constexpr int kNt = DIM / 16;      // 16-column tiles of O
    static constexpr int kTpp = 256 / kCh;    // gather threads per K row, 32 dims each
    static constexpr int kChB = kCh / kBlock; // whole blocks per chunk
};
constexpr int kSplitBlocks = 16;    // kept blocks of one decode split group (64 positions)
constexpr int kWin = 1 << 16;       // union bitmap window, in blocks
constexpr int kWinWords = kWin / 32;
constexpr int kMaxUnionBlocks = 8192;  // rows per tile x top_k is kept at or below this
constexpr int kMaxTileRows = 16;       // row masks are 16 bits, two per LDS word

// Column of chunk position p in a V^T row.  The P V MFMA of 32-position step
// i takes, in lane group g, positions 32i + 4g .. +3 and 32i + 16 + 4g .. +3;
// they are stored side by side at 32i + 8g .. +7, so one 16-byte read fetches
// the lane's B operand.
__device__ __forceinline__ int vt_col(int p)
{
    const int i = p >> 5, h = (p >> 4) & 1, g = (p >> 2) & 3, j = p & 3;
    return 32 * i + 8 * g + 4 * h + j;
}

template <int DIM>
struct alignas(16) ChunkSmem {
    bf16_t k[Geo<DIM>::kCh][Geo<DIM>::kKRow];
    bf16_t vt[DIM][Geo<DIM>::kVRow];
    int32_t pos[Geo<DIM>::kCh];
    uint32_t pmask[Geo<DIM>::kCh];
};

// The union of a tile's kept blocks in one window of kWin blocks.  The bitmap
// and its word prefix counts are needed only while the union is built, so
// they share LDS with the chunk buffer; the union's block list (offsets from
// the window's first block) and row masks stay for the window's chunks.
struct alignas(16) UnionBuild {
    uint32_t bitmap[kWinWords];
    uint16_t wprefix[kWinWords];          // < kMaxUnionBlocks
};
struct alignas(16) UnionSmem {
    // union block i is block w0 + blk[i]; slot kMaxUnionBlocks takes the
    // stores of entries that are not kept
    uint16_t blk[kMaxUnionBlocks + 8];
    uint32_t mask2[kMaxUnionBlocks / 2 + 4];  // union block i: bits 16(i%2) + r of word i/2, r = tile row keeping it
    uint32_t count;
};

__device__ __forceinline__ uint32_t union_mask(const UnionSmem &us, int i)
{
    return (us.mask2[i >> 1] >> (16 * (i & 1))) & 0xffffu;
}

// Logits are kept in base-2 units (softmax_scale * log2(e) * <q, k>).  The
// softmax reference max of a query moves only when a logit exceeds it by more
// than kLazy: until then P = 2^(s - m) <= 2^kLazy, and O and l keep their
// scale (the final O / l and lse = m + log2(l) are the same either way).
constexpr float kLazy = 8.0f;
constexpr float kNoMax = -1.0e30f;  // reference max before a query's first logit: finite, so 2^(-inf - m) = 0
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Reductions over the 4 lane groups of a query: v_permlane16_swap /
// v_permlane32_swap of a register with itself give every lane its own value
// and that of lane l ^ 16 (l ^ 32), without a trip through LDS.
__device__ __forceinline__ float max_xor16(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_xor16(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Per-wave attention state: 16 queries, lane l <-> query l%16 for m / l,
// O[q = 4*(l/16) + j][dim 16*nt + l%16] in o[nt][j].
template <int DIM>
struct WaveState {
    f32x4_t o[Geo<DIM>::kNt];
    float m, l;
};

// K/V elements: bf16 values, or FP8 E4M3 codes (one byte; their values are
// a per-tensor k_scale / v_scale times E4M3(code), applied to the logits and
// the output).  Codes are widened to bf16 on their way into LDS, exactly, so
// the chunk in LDS and everything after it are the same for both.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// A thread's share of one chunk's gather, 32 elements of K and 32 of V: K row
// t/kTpp at dims 32*(t%kTpp) .. +31, and V of positions 4q .. 4q+3 at dims
// 8*(t/(kCh/4)) .. +7, q = t%(kCh/4).  64 + 64 bytes in bf16, 32 + 32 as codes.
template <typename KV>
struct ChunkRegs;
template <>
struct ChunkRegs<bf16_t> {
    uint4 k[4];
    uint4 v[4];
};
template <>
struct ChunkRegs<uint8_t> {
    uint4 k[2];
    uint2 v[4];
};

// Element-wise vector loads (a struct copy from global memory can be lowered
// to a copy through scratch).
__device__ __forceinline__ uint4 load_u4(const void *p)
{
    const u32x4_t x = *(const u32x4_t *)p;
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ uint2 load_u2(const void *p)
{
    const u32x2_t x = *(const u32x2_t *)p;
    return make_uint2(x.x, x.y);
}

// A thread's 32 K elements, and V elements [4 positions x 8 dims] (piece i).
template <typename KV>
__device__ __forceinline__ void load_k(ChunkRegs<KV> &cr, const KV *src)
{
    constexpr int n = sizeof(KV) == 2 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < n; ++i) cr.k[i] = load_u4(src + i * (16 / sizeof(KV)));
}
template <typename KV>
__device__ __forceinline__ void zero_k(ChunkRegs<KV> &cr)
{
    constexpr int n = sizeof(KV) == 2 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < n; ++i) cr.k[i] = make_uint4(0, 0, 0, 0);
}
template <typename KV>
__device__ __forceinline__ void load_v(ChunkRegs<KV> &cr, int i, const KV *src)
{
    if constexpr (sizeof(KV) == 2)
        cr.v[i] = load_u4(src);
    else
        cr.v[i] = load_u2(src);
}
template <typename KV>
__device__ __forceinline__ void zero_v(ChunkRegs<KV> &cr, int i)
{
    if constexpr (sizeof(KV) == 2)
        cr.v[i] = make_uint4(0, 0, 0, 0);
    else
        cr.v[i] = make_uint2(0, 0);
}

// Load the chunk of positions pos(0..n) into registers (zeros beyond n).  The
// loads are only consumed by chunk_store, so they can stay in flight while
// the previous chunk is computed.
template <int DIM, typename KV, class PosFn>
__device__ __forceinline__ void chunk_load(ChunkRegs<KV> &cr, const KV *__restrict__ kbase,
                                           const KV *__restrict__ vbase, int64_t row_stride, int n, PosFn pos)
{
    using G = Geo<DIM>;
    const int t = threadIdx.x;
    const int p = t / G::kTpp, dk = (t % G::kTpp) * 32;
    if (p < n)
        load_k(cr, kbase + (int64_t)pos(p) * row_stride + dk);
    else
        zero_k(cr);
    const int p0 = (t % (G::kCh / 4)) * 4, dv = (t / (G::kCh / 4)) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (p0 + i < n)
            load_v(cr, i, vbase + (int64_t)pos(p0 + i) * row_stride + dv);
        else
            zero_v(cr, i);
    }
}

// Slot of token p of sequence s in the K/V arrays: p itself when the caches
// are contiguous (the sequence's base is then part of the pointers), else the
// slot of p's page ([SGL]: the paged KV pool, addressed by physical slots).
__device__ __forceinline__ int64_t kv_slot(const AttnArgs &a, int64_t s, int64_t p)
{
    if (!a.page_table) return p;
    return (int64_t)a.page_table[s * a.pt_stride + p / a.page_tokens] * a.page_tokens + p % a.page_tokens;
}

// The same share of a chunk of whole blocks: w0 + ublk[0..nb) are the
// chunk's blocks (kChB at most, nb >= 1).  Thread t's K position is token (t/kTpp)%4
// of block t/(4 kTpp) and its V positions are tokens 0..3 of block t%kChB, so
// one block id serves each; a thread past the chunk's blocks reads the last
// one instead (its positions carry no mask bit, so their P is exactly 0).
// Every load is unconditional.
template <int DIM, typename KV>
__device__ __forceinline__ void chunk_load_blocks(ChunkRegs<KV> &cr, const KV *__restrict__ kbase,
                                                  const KV *__restrict__ vbase, uint32_t row_stride,
                                                  const uint16_t *ublk, int32_t w0, int nb, const AttnArgs &a,
                                                  int64_t seq)
{
    using G = Geo<DIM>;
    const int t = threadIdx.x;
    const int32_t bk = w0 + ublk[min(t / (4 * G::kTpp), nb - 1)], bv = w0 + ublk[min(t % G::kChB, nb - 1)];
    // first slot of each block: its 4 tokens are consecutive slots
    const uint32_t sk = (uint32_t)kv_slot(a, seq, (int64_t)kBlock * bk), sv = (uint32_t)kv_slot(a, seq, (int64_t)kBlock * bv);
    load_k(cr, kbase + (uint64_t)sk * row_stride + ((t / G::kTpp) & 3) * row_stride + (t % G::kTpp) * 32);
    const KV *vs = vbase + (uint64_t)sv * row_stride + (t / G::kChB) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_v(cr, i, vs + i * row_stride);
}

// Registers -> LDS: K row-major, V transposed.
template <int DIM>
__device__ __forceinline__ void chunk_store(ChunkSmem<DIM> &cs, const ChunkRegs<bf16_t> &cr)
{
    using G = Geo<DIM>;
    const int t = threadIdx.x;
    const int p = t / G::kTpp, dk = (t % G::kTpp) * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(uint4 *)&cs.k[p][dk + 8 * i] = cr.k[i];
    // the kCh/4 lanes sharing dv write distinct 8-byte pieces of a V^T row;
    // position p0 + j is stored at vt_col(p0) + j
    const int q = t % (G::kCh / 4), dv = (t / (G::kCh / 4)) * 8;
    const int c0 = vt_col(4 * q);
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // dims dv + 2w (low halves) and dv + 2w + 1 (high halves)
        uint32_t x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = w == 0 ? cr.v[i].x : w == 1 ? cr.v[i].y : w == 2 ? cr.v[i].z : cr.v[i].w;
        *(uint2 *)&cs.vt[dv + 2 * w][c0] = make_uint2(__builtin_amdgcn_perm(x[1], x[0], 0x05040100u),
                                                      __builtin_amdgcn_perm(x[3], x[2], 0x05040100u));
        *(uint2 *)&cs.vt[dv + 2 * w + 1][c0] = make_uint2(__builtin_amdgcn_perm(x[1], x[0], 0x07060302u),
                                                          __builtin_amdgcn_perm(x[3], x[2], 0x07060302u));
    }
}

// FP8 codes: widen to bf16 (exact), then store as above.
template <int DIM>
__device__ __forceinline__ void chunk_store(ChunkSmem<DIM> &cs, const ChunkRegs<uint8_t> &c8)
{
    ChunkRegs<bf16_t> cr;
    cr.k[0] = fp8x8_to_bf16_words(c8.k[0].x, c8.k[0].y);
    cr.k[1] = fp8x8_to_bf16_words(c8.k[0].z, c8.k[0].w);
    cr.k[2] = fp8x8_to_bf16_words(c8.k[1].x, c8.k[1].y);
    cr.k[3] = fp8x8_to_bf16_words(c8.k[1].z, c8.k[1].w);
#pragma unroll
    for (int i = 0; i < 4; ++i) cr.v[i] = fp8x8_to_bf16_words(c8.v[i].x, c8.v[i].y);
    chunk_store<DIM>(cs, cr);
}

// Gather K and V^T of positions cs.pos[0..n) into LDS (zeros beyond n).
template <int DIM, typename KV>
__device__ __forceinline__ void gather_chunk(ChunkSmem<DIM> &cs, const KV *__restrict__ kbase,
                                             const KV *__restrict__ vbase, int64_t row_stride, int n)
{
    ChunkRegs<KV> cr;
    chunk_load<DIM>(cr, kbase, vbase, row_stride, n, [&](int i) { return (int64_t)cs.pos[i]; });
    chunk_store<DIM>(cs, cr);
}

// A raw logit where the query attends the position (bit r of its mask word
// set), -inf where it does not: one bit-field extract and one bit-field insert.
__device__ __forceinline__ float masked_logit(float x, uint32_t pmask_word, uint32_t r)
{
    const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int32_t)pmask_word, r, 1u);  // all ones or zero
    return __uint_as_float((__float_as_uint(x) & m) | (0xff800000u & ~m));
}

// One chunk for one wave and its QG groups of 16 queries: S^T, online
// softmax, O += P V.  Every K and V^T operand read from LDS feeds the MFMAs
// of all QG groups.  `rbit[q]` is the mask bit of this lane's query row in
// group q (31, a bit no position carries, when the query slot is unused);
// positions past the chunk's end carry no mask bit.  `scale2` =
// |softmax_scale| * log2(e) > 0: a negative scale is carried by the sign of
// the queries, so the logits' reference max can be taken on raw <q, k> and
// the scale folded into the exponent's FMA.
template <int DIM, int QG>
__device__ __forceinline__ void wave_chunk(const ChunkSmem<DIM> &cs, const bf16x8_t (&qb)[QG][Geo<DIM>::kKs],
                                           const uint32_t (&rbit)[QG], float scale2, WaveState<DIM> (&st)[QG])
{
    using G = Geo<DIM>;
    const int lane = threadIdx.x & 63;
    const int m16 = lane & 15, g = lane >> 4;
    float x[QG][G::kSub][4];  // raw logits, -inf where the query does not attend
    uint4 pm[G::kSub];        // mask words of the lane's positions 4g .. 4g+3 of each sub-tile
    bool any[G::kSub];        // some query of the wave attends the sub-tile
#pragma unroll
    for (int sub = 0; sub < G::kSub; ++sub) {
        pm[sub] = *(const uint4 *)&cs.pmask[sub * 16 + 4 * g];
        const uint32_t pall = pm[sub].x | pm[sub].y | pm[sub].z | pm[sub].w;
        bool some = false;
#pragma unroll
        for (int q = 0; q < QG; ++q) some |= ((pall >> rbit[q]) & 1u) != 0u;
        any[sub] = __ballot(some) != 0ull;
    }
    // S^T of one sub-tile: its K operands are read 4 at a time, then their MFMAs issue
    auto sub_tile = [&](int sub, auto masked) {
        f32x4_t acc[QG];
#pragma unroll
        for (int q = 0; q < QG; ++q) acc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k0 = 0; k0 < G::kKs; k0 += 4) {
            uint4 kv[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kv[ks] = *(const uint4 *)&cs.k[sub * 16 + m16][(DIM / 4) * g + 8 * (k0 + ks)];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int q = 0; q < QG; ++q)
                    acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kv[ks]), qb[q][k0 + ks], acc[q], 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < QG; ++q) {
            if (decltype(masked)::value) {
                x[q][sub][0] = masked_logit(acc[q][0], pm[sub].x, rbit[q]);
                x[q][sub][1] = masked_logit(acc[q][1], pm[sub].y, rbit[q]);
                x[q][sub][2] = masked_logit(acc[q][2], pm[sub].z, rbit[q]);
                x[q][sub][3] = masked_logit(acc[q][3], pm[sub].w, rbit[q]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) x[q][sub][j] = acc[q][j];
            }
        }
    };
    bool all_any = true;
    uint32_t pand = ~0u;  // the mask bits every position of the lane's four per sub-tile carries
#pragma unroll
    for (int sub = 0; sub < G::kSub; ++sub) {
        all_any = all_any && any[sub];
        pand &= pm[sub].x & pm[sub].y & pm[sub].z & pm[sub].w;
    }
    bool lane_full = true;
#pragma unroll
    for (int q = 0; q < QG; ++q) lane_full = lane_full && ((pand >> rbit[q]) & 1u);
    if (__ballot(lane_full) == ~0ull) {  // every query of the wave attends every position: no masks
#pragma unroll
        for (int sub = 0; sub < G::kSub; ++sub) sub_tile(sub, std::false_type{});
    } else if (all_any) {  // every sub-tile has work for the wave (neighbouring rows sharing their blocks)
#pragma unroll
        for (int sub = 0; sub < G::kSub; ++sub) sub_tile(sub, std::true_type{});
    } else {
#pragma unroll
        for (int sub = 0; sub < G::kSub; ++sub) {
            if (any[sub]) {
                sub_tile(sub, std::true_type{});
            } else {
#pragma unroll
                for (int q = 0; q < QG; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[q][sub][j] = -INFINITY;
            }
        }
    }
    // online softmax per query (lane l%16 of group q; the 4 lane groups hold its positions)
    uint4 pa[QG][G::kSub / 2];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        float xmax = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < G::kSub; ++sub)
#pragma unroll
            for (int j = 0; j < 4; ++j) xmax = fmaxf(xmax, x[q][sub][j]);
        const float cmax = max_xor32(max_xor16(xmax)) * scale2;  // scale2 > 0: the max of the scaled logits
        const bool raise = cmax > st[q].m + kLazy;  // also the first logit of a query (st.m = kNoMax)
        const float m_ref = raise ? cmax : st[q].m;
        if (__ballot(raise && st[q].m != kNoMax)) {  // some query's O and l change scale
            const float alpha = raise ? __builtin_amdgcn_exp2f(st[q].m - m_ref) : 1.0f;
            st[q].l *= alpha;
            float a4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) a4[j] = __shfl(alpha, 4 * g + j);
#pragma unroll
            for (int nt = 0; nt < G::kNt; ++nt)
#pragma unroll
                for (int j = 0; j < 4; ++j) st[q].o[nt][j] *= a4[j];
        }
        st[q].m = m_ref;
        float p[G::kSub][4];
        float psum = 0.0f;
#pragma unroll
        for (int sub = 0; sub < G::kSub; ++sub)
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // a masked logit (-inf) gives 0; m_ref is finite
                p[sub][j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[q][sub][j], scale2, -m_ref));
                psum += p[sub][j];
            }
        st[q].l += psum;  // per-lane partial; the 4 groups are summed at the end
#pragma unroll
        for (int i = 0; i < G::kSub / 2; ++i)
            pa[q][i] = make_uint4(pack_bf16x2(p[2 * i][0], p[2 * i][1]), pack_bf16x2(p[2 * i][2], p[2 * i][3]),
                                  pack_bf16x2(p[2 * i + 1][0], p[2 * i + 1][1]),
                                  pack_bf16x2(p[2 * i + 1][2], p[2 * i + 1][3]));
    }
    // O += P V over the chunk's 32-position steps
#pragma unroll
    for (int i = 0; i < G::kSub / 2; ++i) {
        if (!(any[2 * i] || any[2 * i + 1])) continue;
#pragma unroll
        for (int h = 0; h < G::kNt / 4; ++h) {  // V^T operands 4 at a time: one LDS wait per 4 x QG MFMAs
            bf16x8_t Bv[4];
#pragma unroll
            for (int n = 0; n < 4; ++n)
                Bv[n] = as_bf16x8(*(const uint4 *)&cs.vt[16 * (4 * h + n) + m16][32 * i + 8 * g]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int q = 0; q < QG; ++q)
                    st[q].o[4 * h + n] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa[q][i]), Bv[n], st[q].o[4 * h + n], 0, 0, 0);
        }
    }
}

// A lane's query operands, negated when `neg` (exact in bf16).
template <int DIM>
__device__ __forceinline__ void load_query(const bf16_t *__restrict__ qrow, bool valid, bool neg,
                                           bf16x8_t (&qb)[Geo<DIM>::kKs])
{
    const int g = (threadIdx.x & 63) >> 4;
    const uint32_t flip = neg ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < Geo<DIM>::kKs; ++ks) {
        uint4 w = valid ? *(const uint4 *)(qrow + (DIM / 4) * g + 8 * ks) : make_uint4(0, 0, 0, 0);
        w.x ^= flip;
        w.y ^= flip;
        w.z ^= flip;
        w.w ^= flip;
        qb[ks] = as_bf16x8(w);
    }
}

// The exponent scale of the logits, |softmax_scale| * log2(e) (times the
// K scale for FP8 keys), kept positive: a negative scale is carried by the
// sign of the queries, and a zero one becomes the smallest normal float
// (every logit then rounds to 0 in the exponent, as with a zero scale).
__device__ __forceinline__ float logit_scale2(const AttnArgs &a, bool fp8, bool &neg)
{
    const float s2 = (fp8 ? a.scale * a.k_scale : a.scale) * kLog2e;
    neg = s2 < 0.0f;
    return fmaxf(fabsf(s2), __FLT_MIN__);
}

template <int DIM>
__device__ __forceinline__ void init_state(WaveState<DIM> &st)
{
#pragma unroll
    for (int nt = 0; nt < Geo<DIM>::kNt; ++nt) st.o[nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    st.m = kNoMax;
    st.l = 0.0f;
}

// Final per-query sums; returns l_total of the lane's query (l%16).
template <int DIM>
__device__ __forceinline__ float total_l(const WaveState<DIM> &st)
{
    return sum_xor32(sum_xor16(st.l));
}

}  // namespace

static_assert(kSplitBlocks * kBlock == kAttnChunk, "a decode split covers one chunk of attn_decode_splits()");

// ---------------------------------------------------------------------------
// Prefill: grid (row tiles, Hkv).  rows_per_tile * hg <= 64 QG: each wave
// holds QG groups of 16 queries.
// ---------------------------------------------------------------------------
template <int DIM, typename KV, int QG>
__global__ __launch_bounds__(256, 2) void attn_prefill_mfma_kernel(AttnArgs a, int32_t rows_per_tile)
{
    constexpr bool kFp8 = sizeof(KV) == 1;
    using G = Geo<DIM>;
    static_assert(sizeof(UnionBuild) <= sizeof(ChunkSmem<DIM>), "the union build fits the chunk buffer");
    __shared__ union {
        ChunkSmem<DIM> cs;
        UnionBuild ub;
    } sm;
    ChunkSmem<DIM> &cs = sm.cs;
    UnionBuild &ub = sm.ub;
    __shared__ UnionSmem us;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m16 = lane & 15, g = lane >> 4;
    const int hg = a.Hq / a.Hkv;
    const int kvh = blockIdx.y;
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_tile;
    const int nrows = (int)min((int64_t)rows_per_tile, (int64_t)a.n_sel - row0);
    // this lane's query in group q (an S^T column): tile query 16 (QG wave + q) + m16
    bool qneg;
    const float scale2 = logit_scale2(a, kFp8, qneg);
    uint32_t rbit[QG];
    bf16x8_t qb[QG][G::kKs];
    WaveState<DIM> st[QG];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        const int qi = 16 * (QG * wave + q) + m16;
        const int r_local = qi / hg, head = kvh * hg + qi % hg;
        const bool q_valid = r_local < nrows;
        rbit[q] = q_valid ? (uint32_t)r_local : 31u;  // rows of other sequences carry no bit either
        load_query<DIM>((const bf16_t *)a.q + ((row0 + (q_valid ? r_local : 0)) * a.Hq + head) * DIM, q_valid,
                        qneg, qb[q]);
        init_state(st[q]);
    }
    const int64_t row_stride = (int64_t)a.Hkv * DIM;
    // ---- the tile's rows, read once: position, sequence, kept count, last
    // kept block ----
    __shared__ int32_t s_pos[kMaxTileRows], s_seq[kMaxTileRows], s_cnt[kMaxTileRows], s_last[kMaxTileRows];
    if (t < nrows) {
        const int64_t r = row0 + t;
        const int32_t c = max(0, min(a.sel_count[r], a.top_k));
        s_pos[t] = a.row_pos[r];
        s_seq[t] = a.row_seq[r];
        s_cnt[t] = c;
        s_last[t] = c > 0 ? a.sel_blocks[r * a.top_k + c - 1] : -1;
    }
    __syncthreads();
    // the union build's view of the selections: thread t reads row er = t / 16
    // of the tile (ranks below ecnt are kept, 0 for a row not being built)
    static_assert(256 / 16 == kMaxTileRows, "16 threads per tile row");
    constexpr int kEntBatch = 32;  // entries a thread reads per batch (512 ranks per row)
    const int er = t >> 4, ei = t & 15;
    const __amdgpu_buffer_rsrc_t sel_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.sel_blocks + row0 * a.top_k), 0, nrows * a.top_k * 4, 0x00020000);
    uint32_t todo = nrows >= 32 ? 0xffffffffu : ((1u << nrows) - 1u);
    while (todo) {  // rows of one sequence at a time (uniform across the workgroup)
        const int first = __builtin_ctz(todo);
        const int32_t seq = s_seq[first];
        uint32_t active = 0;
        for (int r = first; r < nrows; ++r)
            if (((todo >> r) & 1u) && s_seq[r] == seq) active |= 1u << r;
        todo &= ~active;
        const uint32_t ecnt = er < nrows && ((active >> er) & 1u) ? (uint32_t)s_cnt[er] : 0u;
        const int64_t seq_off = a.page_table ? 0 : (int64_t)seq * a.kv_seq_stride;
        const KV *kbase = (const KV *)a.k_cache + seq_off + (int64_t)kvh * DIM;
        const KV *vbase = (const KV *)a.v_cache + seq_off + (int64_t)kvh * DIM;
        // block range of the active rows' selections
        int32_t hi_blk = 0;
        for (int r = 0; r < nrows; ++r)
            if ((active >> r) & 1u) hi_blk = max(hi_blk, s_last[r] + 1);
        for (int32_t w0 = 0; w0 < hi_blk; w0 += kWin) {
            // ---- union of the active rows' kept blocks in [w0, w0 + kWin).
            // Thread t takes row er = t / 16 of the tile and its ranks
            // i0 + t % 16 + 16 j (j < 32) of each batch of 512 ranks, so all
            // of a thread's entries share one row and one count.  A batch's
            // 32 entries are buffer loads in flight together (past the
            // tile's entries they read 0; a rank at or past the row's count
            // is not kept), and an entry that is not kept updates nothing
            // (an OR of 0, a store to a spare slot): no pass branches. ----
            // pk[j] = (block - w0) | kept << 16
            auto load_batch = [&](int32_t i0, uint32_t(&pk)[kEntBatch]) {
                // computed here, per pass, not hoisted to the kernel's start and held across it
                int32_t vo = (er * a.top_k + i0 + ei) * 4;
                asm volatile("" : "+v"(vo));
                int32_t eb[kEntBatch];
#pragma unroll
                for (int j = 0; j < kEntBatch; ++j)
                    eb[j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(sel_rsrc, vo + 64 * j, 0, 0) - w0;
#pragma unroll
                for (int j = 0; j < kEntBatch; ++j) {
                    const bool ok = (uint32_t)(i0 + ei + 16 * j) < ecnt && (uint32_t)eb[j] < (uint32_t)kWin;
                    pk[j] = ((uint32_t)eb[j] & 0xffffu) | ((uint32_t)ok << 16);
                }
            };
            for (int i = t; i < kWinWords; i += blockDim.x) ub.bitmap[i] = 0u;
            __syncthreads();
            for (int32_t i0 = 0; i0 < a.top_k; i0 += 16 * kEntBatch) {
                uint32_t pk[kEntBatch];
                load_batch(i0, pk);
#pragma unroll
                for (int j = 0; j < kEntBatch; ++j)
                    atomicOr(&ub.bitmap[(pk[j] & 0xffffu) >> 5], ((pk[j] >> 16) & 1u) << (pk[j] & 31u));
            }
            __syncthreads();
            {   // exclusive prefix of popcounts over the words (8 words per thread)
                constexpr int per = kWinWords / 256;
                uint32_t cnt = 0;
#pragma unroll
                for (int i = 0; i < per; ++i) cnt += __popc(ub.bitmap[t * per + i]);
                const uint32_t x = wave_incl_scan(cnt);
                __shared__ uint32_t wsum[4];
                if (lane == 63) wsum[wave] = x;
                __syncthreads();
                uint32_t before = 0, total = 0;
                for (int w = 0; w < 4; ++w) {
                    before += w < wave ? wsum[w] : 0u;
                    total += wsum[w];
                }
                if (t == 0) us.count = total;
                uint32_t run = before + x - cnt;
#pragma unroll
                for (int i = 0; i < per; ++i) {
                    ub.wprefix[t * per + i] = (uint16_t)run;
                    run += __popc(ub.bitmap[t * per + i]);
                }
                for (uint32_t k = t; k < (total + 1) / 2; k += blockDim.x) us.mask2[k] = 0u;
            }
            __syncthreads();
            // each entry's union index: its word's prefix plus the set bits below it;
            // entries of several rows with one block store the same list value
            for (int32_t i0 = 0; i0 < a.top_k; i0 += 16 * kEntBatch) {
                uint32_t pk[kEntBatch];
                load_batch(i0, pk);
                constexpr int kHalf = kEntBatch / 2;  // half the entries' LDS reads in flight at a time
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t wd[kHalf], pf[kHalf];
#pragma unroll
                    for (int j = 0; j < kHalf; ++j) {
                        const uint32_t w = (pk[h * kHalf + j] & 0xffffu) >> 5;
                        wd[j] = ub.bitmap[w];
                        pf[j] = ub.wprefix[w];
                    }
#pragma unroll
                    for (int j = 0; j < kHalf; ++j) {
                        const uint32_t e = pk[h * kHalf + j], b = e & 0xffffu, ok = (e >> 16) & 1u;
                        const uint32_t idx = ok ? pf[j] + __popc(wd[j] & ((1u << (b & 31u)) - 1u)) : kMaxUnionBlocks;
                        us.blk[idx] = (uint16_t)b;
                        atomicOr(&us.mask2[idx >> 1], ok << (er + 16 * (idx & 1u)));
                    }
                }
            }
            __syncthreads();
            const int32_t nu = (int32_t)us.count;
            // ---- the union's blocks, kChB per chunk; chunk c+1's gather is in
            // flight while chunk c is computed ----
            constexpr int kChB = G::kChB;
            const int32_t nch = (nu + kChB - 1) / kChB;
            ChunkRegs<KV> cr;
            if (nch > 0)
                chunk_load_blocks<DIM>(cr, kbase, vbase, (uint32_t)row_stride, us.blk, w0, min(kChB, nu), a, seq);
            for (int32_t c = 0; c < nch; ++c) {
                const int32_t c0 = c * kChB;
                const int nb = min(kChB, nu - c0);
                chunk_store<DIM>(cs, cr);
                if (t < G::kCh) cs.pmask[t] = t / kBlock < nb ? union_mask(us, c0 + t / kBlock) : 0u;
                __syncthreads();
                if (c + 1 < nch) {
                    const int32_t c1 = c0 + kChB;
                    chunk_load_blocks<DIM>(cr, kbase, vbase, (uint32_t)row_stride, us.blk + c1, w0,
                                           min(kChB, nu - c1), a, seq);
                }
                wave_chunk<DIM, QG>(cs, qb, rbit, scale2, st);
                __syncthreads();
            }
        }
        // ---- tails: positions [4*nc(t), t] of every active row (at most 16
        // rows x 3 tokens), a chunk at a time ----
        int ntail = 0;
        for (int r = 0; r < nrows; ++r) {
            if (!((active >> r) & 1u)) continue;
            const int32_t tr = s_pos[r];
            ntail += tr - (int32_t)(kBlock * visible_blocks(tr)) + 1;
        }
        for (int tc = 0; tc < ntail; tc += G::kCh) {
            if (t < G::kCh) {
                const int idx = tc + t;
                int n = 0;
                int32_t pos = 0;
                uint32_t msk = 0;
                for (int r = 0; r < nrows && n <= idx; ++r) {
                    if (!((active >> r) & 1u)) continue;
                    const int32_t tr = s_pos[r];
                    const int32_t ts = (int32_t)(kBlock * visible_blocks(tr));
                    const int len = tr - ts + 1;  // 0..3
                    if (idx < n + len) {
                        pos = ts + (idx - n);
                        msk = 1u << r;
                    }
                    n += len;
                }
                cs.pos[t] = (int32_t)kv_slot(a, seq, pos);
                cs.pmask[t] = msk;
            }
            __syncthreads();
            // positions beyond the tails carry no mask bit, so they stay out
            gather_chunk<DIM>(cs, kbase, vbase, row_stride, min(G::kCh, ntail - tc));
            __syncthreads();
            wave_chunk<DIM, QG>(cs, qb, rbit, scale2, st);
            __syncthreads();
        }
    }
    // ---- output ----
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        const float ltot = total_l(st[q]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qo = 16 * (QG * wave + q) + 4 * g + j;  // query of o[.][j]
            const int ro = qo / hg;
            const float lq = __shfl(ltot, 4 * g + j);
            if (ro >= nrows) continue;
            const int ho = kvh * hg + qo % hg;
            bf16_t *orow = (bf16_t *)a.out + ((row0 + ro) * a.Hq + ho) * DIM;
            const float inv = lq > 0.0f ? (kFp8 ? a.v_scale : 1.0f) / lq : 0.0f;
#pragma unroll
            for (int nt = 0; nt < G::kNt; ++nt) orow[16 * nt + m16] = f32_to_bf16(st[q].o[nt][j] * inv);
        }
        const int qi = 16 * (QG * wave + q) + m16;
        if (a.lse && g == 0 && qi / hg < nrows)
            a.lse[(row0 + qi / hg) * a.Hq + kvh * hg + qi % hg] =
                ltot > 0.0f ? (st[q].m + __log2f(ltot)) * kLn2 : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Decode: grid (splits, batch * Hkv).  q_per_sel * hg <= 64, q_per_sel <= 32.
// Split i < nsplit-1 takes kept blocks [S i, S i + S), S = 16 ceil(n / (nsplit
// - 1)) for the n 16-block groups of top_k (S = 16 with one split per group);
// the last split takes the tails.
// ---------------------------------------------------------------------------
template <int DIM, typename KV>  // D = 256 needs the two-wave register budget to avoid spilling
__global__ __launch_bounds__(256, DIM == 256 ? 2 : 1) void attn_decode_mfma_kernel(AttnArgs a)
{
    constexpr bool kFp8 = sizeof(KV) == 1;
    using G = Geo<DIM>;
    __shared__ ChunkSmem<DIM> cs;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int m16 = lane & 15, g = lane >> 4;
    const int hg = a.Hq / a.Hkv;
    const int64_t s = blockIdx.y / a.Hkv;
    const int kvh = blockIdx.y % a.Hkv;
    const int split = blockIdx.x;
    const int nq = a.q_per_sel * hg;
    const int qi = 16 * wave + m16;
    const int jrow = qi / hg;
    const bool q_valid = qi < nq;
    const int head = kvh * hg + qi % hg;
    const int64_t qrow = (s * a.q_per_sel + (q_valid ? jrow : 0)) * a.Hq + head;
    bool qneg;
    const float scale2 = logit_scale2(a, kFp8, qneg);
    bf16x8_t qb[1][G::kKs];
    load_query<DIM>((const bf16_t *)a.q + qrow * DIM, q_valid, qneg, qb[0]);
    WaveState<DIM> st[1];
    init_state(st[0]);
    const uint32_t rbit[1] = {q_valid ? (uint32_t)jrow : 31u};
    const int64_t row_stride = (int64_t)a.Hkv * DIM;
    const int64_t seq_off = a.page_table ? 0 : s * a.kv_seq_stride;
    const KV *kbase = (const KV *)a.k_cache + seq_off + (int64_t)kvh * DIM;
    const KV *vbase = (const KV *)a.v_cache + seq_off + (int64_t)kvh * DIM;
    const int32_t count = min(a.sel_count[s], a.top_k);
    const uint32_t all_rows = a.q_per_sel >= 32 ? 0xffffffffu : ((1u << a.q_per_sel) - 1u);
    if (split < a.nsplit - 1) {
        // the kept blocks in nsplit - 1 runs of whole 16-block groups: one group
        // per split, or several when the caller gave fewer splits
        const int32_t n16 = (a.top_k + kSplitBlocks - 1) / kSplitBlocks;
        const int32_t sb = kSplitBlocks * ((n16 + a.nsplit - 2) / (a.nsplit - 1));
        const int32_t b0 = split * sb;
        const int nb = max(0, min(sb, count - b0));
        for (int c0 = 0; c0 < nb; c0 += G::kChB) {
            const int cb = min(G::kChB, nb - c0);
            if (t < G::kCh) {
                const int bi = t / kBlock;
                cs.pos[t] = bi < cb ? (int32_t)kv_slot(a, s, (int64_t)a.sel_blocks[s * a.top_k + b0 + c0 + bi] *
                                                                 kBlock + (t % kBlock))
                                    : 0;
                cs.pmask[t] = bi < cb ? all_rows : 0u;
            }
            __syncthreads();
            gather_chunk<DIM>(cs, kbase, vbase, row_stride, cb * kBlock);
            __syncthreads();
            wave_chunk<DIM, 1>(cs, qb, rbit, scale2, st);
            __syncthreads();
        }
    } else {
        // tails: row j attends [ts_j, t_j]; walk [min ts, max t] in chunks
        int32_t lo = INT32_MAX, hi = -1;
        for (int j = 0; j < a.q_per_sel; ++j) {
            const int32_t tj = a.row_pos[s * a.q_per_sel + j];
            const int32_t ts = a.tail_start ? a.tail_start[s] : (int32_t)(kBlock * visible_blocks(tj));
            lo = min(lo, ts);
            hi = max(hi, tj);
        }
        for (int64_t p0 = lo; p0 <= hi; p0 += G::kCh) {
            const int n = (int)min((int64_t)G::kCh, (int64_t)hi - p0 + 1);
            if (t < G::kCh) {
                const int64_t p = p0 + t;
                uint32_t msk = 0;
                if (t < n) {
                    for (int j = 0; j < a.q_per_sel; ++j) {
                        const int32_t tj = a.row_pos[s * a.q_per_sel + j];
                        const int32_t ts = a.tail_start ? a.tail_start[s] : (int32_t)(kBlock * visible_blocks(tj));
                        if (p >= ts && p <= tj) msk |= 1u << j;
                    }
                }
                cs.pos[t] = t < n ? (int32_t)kv_slot(a, s, p) : 0;
                cs.pmask[t] = msk;
            }
            __syncthreads();
            gather_chunk<DIM>(cs, kbase, vbase, row_stride, n);
            __syncthreads();
            wave_chunk<DIM, 1>(cs, qb, rbit, scale2, st);
            __syncthreads();
        }
    }
    // ---- partial softmax state of this split ----
    const float ltot = total_l(st[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int qo = 16 * wave + 4 * g + j;
        if (qo >= nq) continue;
        const int jo = qo / hg, ho = kvh * hg + qo % hg;
        float *pp = a.partial + (((s * a.q_per_sel + jo) * a.Hq + ho) * a.nsplit + split) * (DIM + 2);
        const float vs = kFp8 ? a.v_scale : 1.0f;  // the partial outputs carry the V scale
#pragma unroll
        for (int nt = 0; nt < G::kNt; ++nt) pp[16 * nt + m16] = st[0].o[nt][j] * vs;
    }
    if (q_valid && g == 0) {
        float *pp = a.partial + (qrow * a.nsplit + split) * (DIM + 2);
        pp[DIM] = st[0].m * kLn2;  // natural-log units for the combine
        pp[DIM + 1] = ltot;
    }
}

// Rows of a prefill tile whose waves hold qg groups of 16 queries each.
static int32_t prefill_rows(int32_t hg, int32_t top_k, int32_t qg)
{
    int32_t r = max(1, 64 * qg / hg);
    r = min(r, kMaxTileRows);                  // row masks are 16 bits
    r = min(r, kMaxUnionBlocks / top_k);       // the union of the rows' selections fits LDS
    return max(r, 1);
}

// Two query groups per wave at head dim 128 when the tile then holds more
// than 64 queries (so no wave's second group is always empty).
static int32_t prefill_groups(int32_t hg, int32_t top_k, int32_t D)
{
    return D == 128 && (int64_t)prefill_rows(hg, top_k, 2) * hg > 64 ? 2 : 1;
}

bool attn_mfma_supported(int32_t Hq, int32_t Hkv, int32_t q_per_sel, int32_t D, bool bf16)
{
    if (!bf16 || (D != 128 && D != 256) || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return false;
    const int32_t hg = Hq / Hkv;
    return hg <= 64 && (int64_t)q_per_sel * hg <= 64 &&
           q_per_sel <= 32 &&                            // decode row masks are 32 bits
           (int64_t)Hkv * D * kBlock <= (int64_t)UINT32_MAX;  // a block's K/V span as a 32-bit element count
}

void launch_attn_prefill_mfma(const AttnArgs &a, hipStream_t stream)
{
    const int32_t hg = a.Hq / a.Hkv;
    const int32_t qg = prefill_groups(hg, a.top_k, a.D);
    const int32_t rpt = prefill_rows(hg, a.top_k, qg);
    const dim3 grid((unsigned)((a.n_sel + rpt - 1) / rpt), (unsigned)a.Hkv), block(256);
    if (a.D == 256 && a.kv_fp8)
        QSA_LAUNCH("attn_prefill_mfma_d256_fp8kv", (attn_prefill_mfma_kernel<256, uint8_t, 1>), grid, block, 0,
                   stream, a, rpt);
    else if (a.D == 256)
        QSA_LAUNCH("attn_prefill_mfma_d256", (attn_prefill_mfma_kernel<256, bf16_t, 1>), grid, block, 0, stream, a,
                   rpt);
    else if (a.kv_fp8 && qg == 2)
        QSA_LAUNCH("attn_prefill_mfma_fp8kv", (attn_prefill_mfma_kernel<128, uint8_t, 2>), grid, block, 0, stream,
                   a, rpt);
    else if (a.kv_fp8)
        QSA_LAUNCH("attn_prefill_mfma_fp8kv", (attn_prefill_mfma_kernel<128, uint8_t, 1>), grid, block, 0, stream,
                   a, rpt);
    else if (qg == 2)
        QSA_LAUNCH("attn_prefill_mfma", (attn_prefill_mfma_kernel<128, bf16_t, 2>), grid, block, 0, stream, a, rpt);
    else
        QSA_LAUNCH("attn_prefill_mfma", (attn_prefill_mfma_kernel<128, bf16_t, 1>), grid, block, 0, stream, a, rpt);
}

void launch_attn_decode_mfma(const AttnArgs &a, hipStream_t stream)
{
    const dim3 grid((unsigned)a.nsplit, (unsigned)((int64_t)a.n_sel * a.Hkv)), block(256);
    if (a.D == 256 && a.kv_fp8)
        QSA_LAUNCH("attn_decode_mfma_d256_fp8kv", (attn_decode_mfma_kernel<256, uint8_t>), grid, block, 0, stream,
                   a);
    else if (a.D == 256)
        QSA_LAUNCH("attn_decode_mfma_d256", (attn_decode_mfma_kernel<256, bf16_t>), grid, block, 0, stream, a);
    else if (a.kv_fp8)
        QSA_LAUNCH("attn_decode_mfma_fp8kv", (attn_decode_mfma_kernel<128, uint8_t>), grid, block, 0, stream, a);
    else
        QSA_LAUNCH("attn_decode_mfma", (attn_decode_mfma_kernel<128, bf16_t>), grid, block, 0, stream, a);
}

}  // namespace qsa
