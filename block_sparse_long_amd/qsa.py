"""Thin ctypes binding of libqsa (declared in include/qsa.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the GPU (torch supplies device memory
and the current stream); bf16 tensors are ``torch.bfloat16``, fp32 tensors
``torch.float32``.  A missing library raises ``QsaLibraryMissing``; a
rejected call raises ``QsaError`` carrying the library's status code.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqsa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_DEVICE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
FLAG_NO_ROPE = 1 << 0
FLAG_POOL_RMSNORM = 1 << 1
FLAG_SCORE_ROWS = 1 << 8
FLAG_SCORE_GEMM = 1 << 9
INDEX_DIM, INDEX_HEADS, BLOCK_TOKENS, MAX_TOP_K, MAX_QUERY_GROUP = 128, 4, 4, 4096, 64

# every symbol include/qsa.h declares
EXPORTS = ("qsa_pool_index_keys", "qsa_pool_index_keys_ex", "qsa_score_topk_ex", "qsa_pool_index_keys_fp8", "qsa_pool_append", "qsa_score_topk_workspace_size",
           "qsa_score_topk", "qsa_score_topk_merge_modes_offset", "qsa_score_topk_fp8_workspace_size",
           "qsa_score_topk_fp8", "qsa_score_topk_paged",
           "qsa_pool_index_keys_paged", "qsa_sparse_attn_prefill_paged", "qsa_sparse_attn_decode_paged",
           "qsa_sparse_attn_prefill_fp8kv",
           "qsa_sparse_attn_decode_fp8kv",
           "qsa_sparse_attn_prefill", "qsa_sparse_attn_decode_workspace_size",
           "qsa_sparse_attn_decode", "qsa_sparse_attn_decode_noalloc", "qsa_status_string",
           "qsa_last_device_error", "qsa_profile_enable",
           "qsa_profile_reset", "qsa_profile_kernel_ms")


class QsaLibraryMissing(RuntimeError):
    pass


class QsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


_lib = None


def load():
    """Open libqsa.so (built in-tree by block_sparse_long_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise QsaLibraryMissing(f"{LIB_PATH} is not built; run `python -m block_sparse_long_amd.build`")
    # torch ships its own HIP runtime under the same soname as ROCm's.  Loaded
    # first, it is the one libqsa binds to, so the process has one runtime and
    # torch's device memory and stream handles are valid in libqsa's calls.
    # Opened in the other order, two runtimes coexist and the second finds
    # no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                      ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
    st = ctypes.c_int
    lib.qsa_pool_index_keys.argtypes = [P, i64, P, i64, i32, i32, i32, f64, u32, st, P]
    lib.qsa_pool_index_keys.restype = st
    lib.qsa_pool_index_keys_ex.argtypes = [P, i64, P, i64, i32, i32, i32, P, P, u32, st, P]
    lib.qsa_pool_index_keys_ex.restype = st
    lib.qsa_score_topk_ex.argtypes = [P, P, P, i32, P, i64, i32, i32, P, u32, st, P, P, P, P, sz, P]
    lib.qsa_score_topk_ex.restype = st
    lib.qsa_pool_index_keys_fp8.argtypes = [P, i64, P, P, i64, i32, i32, i32, f64, u32, st, P]
    lib.qsa_pool_index_keys_fp8.restype = st
    lib.qsa_score_topk_fp8_workspace_size.argtypes = [i32, i32, i32, u32]
    lib.qsa_score_topk_fp8_workspace_size.restype = sz
    lib.qsa_score_topk_fp8.argtypes = [P, P, P, i32, P, P, i64, i32, i32, f64, u32, P, P, P, P, sz, P]
    lib.qsa_score_topk_fp8.restype = st
    lib.qsa_score_topk_paged.argtypes = [P, P, P, i32, P, P, P, P, i64, i32, i32, i32, f64, u32, st, P, P, P, P, sz,
                                         P]
    lib.qsa_score_topk_paged.restype = st
    lib.qsa_sparse_attn_prefill_paged.argtypes = [P, P, P, i32, P, P, P, i64, i32, P, P, i32, i32, i32, i32, f32, st,
                                                  P, P, P]
    lib.qsa_sparse_attn_prefill_paged.restype = st
    lib.qsa_sparse_attn_decode_paged.argtypes = [P, P, i32, i32, P, P, P, P, i64, i32, P, P, i32, i32, i32, i32, f32,
                                                 st, P, P, P, sz, P]
    lib.qsa_sparse_attn_decode_paged.restype = st
    lib.qsa_pool_index_keys_paged.argtypes = [P, i64, P, P, P, P, i64, i32, i32, i32, i32, f64, u32, st, P]
    lib.qsa_pool_index_keys_paged.restype = st
    lib.qsa_sparse_attn_prefill_fp8kv.argtypes = [P, P, P, i32, P, P, i64, P, i64, i32, f32, f32, P, P, i32, i32,
                                                  i32, i32, f32, P, P, P]
    lib.qsa_sparse_attn_prefill_fp8kv.restype = st
    lib.qsa_sparse_attn_decode_fp8kv.argtypes = [P, P, i32, i32, P, P, P, i64, P, i64, i32, f32, f32, P, P, i32, i32,
                                                 i32, i32, f32, P, P, P, sz, P]
    lib.qsa_sparse_attn_decode_fp8kv.restype = st
    lib.qsa_pool_append.argtypes = [P, P, P, P, P, i32, f64, u32, st, P]
    lib.qsa_pool_append.restype = st
    lib.qsa_score_topk_workspace_size.argtypes = [i32, i32, i32, st, u32]
    lib.qsa_score_topk_workspace_size.restype = sz
    lib.qsa_score_topk_merge_modes_offset.argtypes = [i32, i32, i32, st, u32]
    lib.qsa_score_topk_merge_modes_offset.restype = sz
    lib.qsa_score_topk.argtypes = [P, P, P, i32, P, i64, i32, i32, f64, u32, st, P, P, P, P, sz, P]
    lib.qsa_score_topk.restype = st
    lib.qsa_sparse_attn_prefill.argtypes = [P, P, P, i32, P, P, i64, P, P, i32, i32, i32, i32, f32, st,
                                            P, P, P]
    lib.qsa_sparse_attn_prefill.restype = st
    lib.qsa_sparse_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.qsa_sparse_attn_decode_workspace_size.restype = sz
    lib.qsa_sparse_attn_decode.argtypes = [P, P, i32, i32, P, P, P, i64, P, P, i32, i32, i32, i32, f32,
                                           st, P, P, P, sz, P]
    lib.qsa_sparse_attn_decode.restype = st
    lib.qsa_sparse_attn_decode_noalloc.argtypes = [P, P, i32, i32, P, P, P, i64, P, P, i32, i32, i32, i32, f32,
                                                   st, P, P, P]
    lib.qsa_sparse_attn_decode_noalloc.restype = st
    lib.qsa_status_string.argtypes = [st]
    lib.qsa_status_string.restype = ctypes.c_char_p
    lib.qsa_last_device_error.argtypes = []
    lib.qsa_last_device_error.restype = ctypes.c_char_p
    lib.qsa_profile_enable.argtypes = [ctypes.c_int]
    lib.qsa_profile_enable.restype = st
    lib.qsa_profile_reset.argtypes = []
    lib.qsa_profile_reset.restype = st
    lib.qsa_profile_kernel_ms.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double)]
    lib.qsa_profile_kernel_ms.restype = i32
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().qsa_status_string(code).decode()


def _check(fn: str, rc: int):
    if rc != OK:
        msg = status_string(rc)
        if rc == ERR_DEVICE:
            msg += ": " + load().qsa_last_device_error().decode()
        raise QsaError(fn, rc, msg)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"libqsa takes bfloat16 or float32 tensors, got {t.dtype}")


def _need_contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("libqsa takes contiguous tensors")


class Rope(ctypes.Structure):
    """qsa_rope_t: RoPE base and YaRN scaling (yarn_factor 1 = plain RoPE)."""
    _fields_ = [("theta", ctypes.c_double), ("yarn_factor", ctypes.c_double),
                ("yarn_original_context", ctypes.c_double), ("yarn_alpha", ctypes.c_double),
                ("yarn_beta", ctypes.c_double)]


def rope(theta: float, yarn_factor: float = 1.0, yarn_original_context: float = 0.0, yarn_alpha: float = 1.0,
         yarn_beta: float = 32.0) -> Rope:
    return Rope(float(theta), float(yarn_factor), float(yarn_original_context), float(yarn_alpha),
                float(yarn_beta))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def pool_index_keys_ex(raw_keys, pooled, block_begin: int, block_end: int, rope_params: Optional[Rope],
                       norm_weight=None, flags: int = 0, stream=None):
    """pool_index_keys with a Rope (YaRN scaling) and an optional learned
    norm weight (fp32 [128] on the device; needs FLAG_POOL_RMSNORM)."""
    _need_contig(raw_keys, pooled, norm_weight)
    B, L, _ = raw_keys.shape
    rp = ctypes.byref(rope_params) if rope_params is not None else None
    rc = load().qsa_pool_index_keys_ex(_ptr(raw_keys), L * INDEX_DIM, _ptr(pooled), pooled.shape[1] * INDEX_DIM, B,
                                       int(block_begin), int(block_end), rp, _ptr(norm_weight), int(flags),
                                       _dtype_code(raw_keys), _stream(stream))
    _check("qsa_pool_index_keys_ex", rc)

def pool_index_keys(raw_keys, pooled, block_begin: int, block_end: int, rope_theta: float,
                    flags: int = 0, stream=None):
    """a1-a3 into `pooled` [B][NB][128] from `raw_keys` [B][L][128]."""
    _need_contig(raw_keys, pooled)
    B, L, _ = raw_keys.shape
    rc = load().qsa_pool_index_keys(_ptr(raw_keys), L * INDEX_DIM, _ptr(pooled),
                                    pooled.shape[1] * INDEX_DIM, B, int(block_begin), int(block_end),
                                    float(rope_theta), int(flags), _dtype_code(raw_keys), _stream(stream))
    _check("qsa_pool_index_keys", rc)


def pool_index_keys_fp8(raw_keys, codes, scales, block_begin: int, block_end: int, rope_theta: float,
                        flags: int = 0, stream=None):
    """a1-a3 with FP8 storage: codes [B][NB][128] uint8 (E4M3) and scales
    [B][NB] float32 from `raw_keys` [B][L][128] (bf16 or float32)."""
    _need_contig(raw_keys, codes, scales)
    B, L, _ = raw_keys.shape
    assert codes.shape[:2] == scales.shape and codes.shape[2] == INDEX_DIM
    rc = load().qsa_pool_index_keys_fp8(_ptr(raw_keys), L * INDEX_DIM, _ptr(codes), _ptr(scales), codes.shape[1], B,
                                        int(block_begin), int(block_end), float(rope_theta), int(flags),
                                        _dtype_code(raw_keys), _stream(stream))
    _check("qsa_pool_index_keys_fp8", rc)


def pool_append(new_keys, positions, full_slots, ring, compressed, rope_theta: float, flags: int = 0,
                stream=None):
    """One decode step of incremental pooling: new_keys [B][128] into the
    4-slot rings [B][4][128]; a completed block's compressed key goes to
    compressed [S][128] at full_slots // 4 (positions int32, full_slots int64)."""
    _need_contig(new_keys, positions, full_slots, ring, compressed)
    rc = load().qsa_pool_append(_ptr(new_keys), _ptr(positions), _ptr(full_slots), _ptr(ring), _ptr(compressed),
                                new_keys.shape[0], float(rope_theta), int(flags), _dtype_code(new_keys),
                                _stream(stream))
    _check("qsa_pool_append", rc)


def score_topk_workspace_size(rows: int, max_visible_blocks: int, top_k: int, dtype_code: int,
                              flags: int = 0) -> int:
    return int(load().qsa_score_topk_workspace_size(int(rows), int(max_visible_blocks), int(top_k),
                                                    int(dtype_code), int(flags)))


MERGE_MODES = {0: "none", 1: "staged", 2: "prefiltered", 3: "list_walk", 4: "recomputed"}


def score_topk_merge_modes_offset(rows: int, max_visible_blocks: int, top_k: int, dtype_code: int,
                                  flags: int = 0) -> Optional[int]:
    """Byte offset of the fused scorer's per-row merge modes in a score_topk
    workspace (int32 [rows], see MERGE_MODES), or None for the per-row path."""
    off = int(load().qsa_score_topk_merge_modes_offset(int(rows), int(max_visible_blocks), int(top_k),
                                                       int(dtype_code), int(flags)))
    return None if off == ctypes.c_size_t(-1).value else off


def score_topk(q_index, row_seq, row_pos, pooled, max_visible_blocks: int, top_k: int,
               rope_theta: float, flags: int = 0, sel_blocks=None, sel_count=None, sel_scores=None,
               workspace=None, want_scores: bool = True, stream=None):
    """a4-a6.  Returns (sel_blocks [R][top_k] int32, sel_count [R] int32,
    sel_scores [R][top_k] float32 or None).  Output tensors and the workspace
    may be passed in (no allocation then)."""
    import torch
    _need_contig(q_index, row_seq, row_pos, pooled)
    R = q_index.shape[0]
    dev = q_index.device
    dt = _dtype_code(q_index)
    if sel_blocks is None:
        sel_blocks = torch.empty((R, top_k), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((R,), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((R, top_k), dtype=torch.float32, device=dev)
    need = score_topk_workspace_size(R, max_visible_blocks, top_k, dt, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    rc = load().qsa_score_topk(_ptr(q_index), _ptr(row_seq), _ptr(row_pos), R, _ptr(pooled),
                               pooled.shape[1] * INDEX_DIM, int(max_visible_blocks), int(top_k),
                               float(rope_theta), int(flags), dt, _ptr(sel_blocks), _ptr(sel_count),
                               _ptr(sel_scores), _ptr(workspace), workspace.numel(), _stream(stream))
    _check("qsa_score_topk", rc)
    return sel_blocks, sel_count, sel_scores


def score_topk_ex(q_index, row_seq, row_pos, pooled, max_visible_blocks: int, top_k: int,
                  rope_params: Optional[Rope], flags: int = 0, sel_blocks=None, sel_count=None, sel_scores=None,
                  workspace=None, want_scores: bool = True, stream=None):
    """score_topk with a Rope (the keys pooled with the same rotation)."""
    import torch
    _need_contig(q_index, row_seq, row_pos, pooled)
    R = q_index.shape[0]
    dev = q_index.device
    dt = _dtype_code(q_index)
    if sel_blocks is None:
        sel_blocks = torch.empty((R, top_k), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((R,), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((R, top_k), dtype=torch.float32, device=dev)
    need = score_topk_workspace_size(R, max_visible_blocks, top_k, dt, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    rp = ctypes.byref(rope_params) if rope_params is not None else None
    rc = load().qsa_score_topk_ex(_ptr(q_index), _ptr(row_seq), _ptr(row_pos), R, _ptr(pooled),
                                  pooled.shape[1] * INDEX_DIM, int(max_visible_blocks), int(top_k), rp,
                                  int(flags), dt, _ptr(sel_blocks), _ptr(sel_count), _ptr(sel_scores),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _check("qsa_score_topk_ex", rc)
    return sel_blocks, sel_count, sel_scores


def score_topk_fp8_workspace_size(rows: int, max_visible_blocks: int, top_k: int, flags: int = 0) -> int:
    return int(load().qsa_score_topk_fp8_workspace_size(int(rows), int(max_visible_blocks), int(top_k), int(flags)))


def score_topk_fp8(q_index, row_seq, row_pos, codes, scales, max_visible_blocks: int, top_k: int,
                   rope_theta: float, flags: int = 0, sel_blocks=None, sel_count=None, sel_scores=None,
                   workspace=None, want_scores: bool = True, stream=None):
    """a4-a6 on FP8 keys (codes [B][NB][128] uint8, scales [B][NB] float32);
    q_index bf16.  Returns as score_topk."""
    import torch
    _need_contig(q_index, row_seq, row_pos, codes, scales)
    R = q_index.shape[0]
    dev = q_index.device
    if sel_blocks is None:
        sel_blocks = torch.empty((R, top_k), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((R,), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((R, top_k), dtype=torch.float32, device=dev)
    need = score_topk_fp8_workspace_size(R, max_visible_blocks, top_k, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    rc = load().qsa_score_topk_fp8(_ptr(q_index), _ptr(row_seq), _ptr(row_pos), R, _ptr(codes), _ptr(scales),
                                   codes.shape[1], int(max_visible_blocks), int(top_k), float(rope_theta), int(flags),
                                   _ptr(sel_blocks), _ptr(sel_count), _ptr(sel_scores), _ptr(workspace),
                                   workspace.numel(), _stream(stream))
    _check("qsa_score_topk_fp8", rc)
    return sel_blocks, sel_count, sel_scores


def sparse_attn_prefill(q, row_seq, row_pos, k_cache, v_cache, sel_blocks, sel_count,
                        softmax_scale: Optional[float] = None, out=None, lse=None, want_lse=True,
                        stream=None):
    """a7+a8.  q [R][Hq][D]; k/v [B][L][Hkv][D].  Returns (out, lse)."""
    import torch
    _need_contig(q, row_seq, row_pos, k_cache, v_cache, sel_blocks, sel_count)
    R, Hq, D = q.shape
    _, L, Hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    rc = load().qsa_sparse_attn_prefill(_ptr(q), _ptr(row_seq), _ptr(row_pos), R, _ptr(k_cache),
                                        _ptr(v_cache), L * Hkv * D, _ptr(sel_blocks), _ptr(sel_count),
                                        sel_blocks.shape[1], Hq, Hkv, D, scale, _dtype_code(q), _ptr(out),
                                        _ptr(lse), _stream(stream))
    _check("qsa_sparse_attn_prefill", rc)
    return out, lse


def sparse_attn_decode_workspace_size(batch: int, q_per_seq: int, Hq: int, D: int, top_k: int) -> int:
    return int(load().qsa_sparse_attn_decode_workspace_size(int(batch), int(q_per_seq), int(Hq),
                                                            int(D), int(top_k)))


def sparse_attn_decode(q, row_pos, k_cache, v_cache, sel_blocks, sel_count, tail_start=None,
                       softmax_scale: Optional[float] = None, out=None, lse=None, want_lse=True,
                       workspace=None, stream=None):
    """a7+a9.  q [B][Qn][Hq][D]; row_pos [B][Qn]; sel [B][top_k].  Returns (out, lse)."""
    import torch
    _need_contig(q, row_pos, k_cache, v_cache, sel_blocks, sel_count, tail_start)
    B, Qn, Hq, D = q.shape
    _, L, Hkv, _ = k_cache.shape
    top_k = sel_blocks.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Qn, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_decode_workspace_size(B, Qn, Hq, D, top_k)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    rc = load().qsa_sparse_attn_decode(_ptr(q), _ptr(row_pos), B, Qn, _ptr(tail_start), _ptr(k_cache),
                                       _ptr(v_cache), L * Hkv * D, _ptr(sel_blocks), _ptr(sel_count), top_k,
                                       Hq, Hkv, D, scale, _dtype_code(q), _ptr(out), _ptr(lse),
                                       _ptr(workspace), workspace.numel(), _stream(stream))
    _check("qsa_sparse_attn_decode", rc)
    return out, lse


NOALLOC_SCRATCH_BYTES = 16 << 20


def sparse_attn_decode_noalloc(q, row_pos, k_cache, v_cache, sel_blocks, sel_count, tail_start=None,
                               softmax_scale: Optional[float] = None, out=None, lse=None, want_lse=True,
                               stream=None):
    """sparse_attn_decode through the allocation-free entry point: the split
    partials live in the library's static per-device scratch, so no workspace
    is passed (the call itself allocates nothing; pass `out` / `lse` to keep
    this wrapper from allocating them).  Returns (out, lse)."""
    import torch
    _need_contig(q, row_pos, k_cache, v_cache, sel_blocks, sel_count, tail_start)
    B, Qn, Hq, D = q.shape
    _, L, Hkv, _ = k_cache.shape
    top_k = sel_blocks.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Qn, Hq), dtype=torch.float32, device=q.device)
    rc = load().qsa_sparse_attn_decode_noalloc(_ptr(q), _ptr(row_pos), B, Qn, _ptr(tail_start), _ptr(k_cache),
                                               _ptr(v_cache), L * Hkv * D, _ptr(sel_blocks), _ptr(sel_count),
                                               top_k, Hq, Hkv, D, scale, _dtype_code(q), _ptr(out), _ptr(lse),
                                               _stream(stream))
    _check("qsa_sparse_attn_decode_noalloc", rc)
    return out, lse


def score_topk_paged(q_index, row_seq, row_pos, page_table, page_tokens: int, max_visible_blocks: int,
                     top_k: int, rope_theta: float, pooled=None, codes=None, scales=None, flags: int = 0,
                     sel_blocks=None, sel_count=None, sel_scores=None, workspace=None, want_scores: bool = True,
                     stream=None):
    """a4-a6 on paged compressed keys: `pooled` [slots/4][128] (dtype of
    q_index), or FP8 `codes` [slots/4][128] uint8 + `scales` [slots/4];
    page_table [n_seq][pages] int32.  Returns as score_topk."""
    import torch
    _need_contig(q_index, row_seq, row_pos, page_table, pooled, codes, scales)
    R = q_index.shape[0]
    dev = q_index.device
    dt = _dtype_code(q_index)
    if sel_blocks is None:
        sel_blocks = torch.empty((R, top_k), dtype=torch.int32, device=dev)
    if sel_count is None:
        sel_count = torch.empty((R,), dtype=torch.int32, device=dev)
    if sel_scores is None and want_scores:
        sel_scores = torch.empty((R, top_k), dtype=torch.float32, device=dev)
    need = score_topk_workspace_size(R, max_visible_blocks, top_k, dt, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    rc = load().qsa_score_topk_paged(_ptr(q_index), _ptr(row_seq), _ptr(row_pos), R, _ptr(pooled), _ptr(codes),
                                     _ptr(scales), _ptr(page_table), page_table.shape[1], int(page_tokens),
                                     int(max_visible_blocks), int(top_k), float(rope_theta), int(flags), dt,
                                     _ptr(sel_blocks), _ptr(sel_count), _ptr(sel_scores), _ptr(workspace),
                                     workspace.numel(), _stream(stream))
    _check("qsa_score_topk_paged", rc)
    return sel_blocks, sel_count, sel_scores


def sparse_attn_prefill_paged(q, row_seq, row_pos, k_cache, v_cache, page_table, page_tokens: int, sel_blocks,
                              sel_count, softmax_scale: Optional[float] = None, out=None, lse=None, want_lse=True,
                              stream=None):
    """a7+a8 on a paged K/V pool: k/v [slots][Hkv][D]; page_table [R_seq][pages]."""
    import torch
    _need_contig(q, row_seq, row_pos, k_cache, v_cache, page_table, sel_blocks, sel_count)
    R, Hq, D = q.shape
    _, Hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    rc = load().qsa_sparse_attn_prefill_paged(_ptr(q), _ptr(row_seq), _ptr(row_pos), R, _ptr(k_cache), _ptr(v_cache),
                                              _ptr(page_table), page_table.shape[1], int(page_tokens),
                                              _ptr(sel_blocks), _ptr(sel_count), sel_blocks.shape[1], Hq, Hkv, D,
                                              scale, _dtype_code(q), _ptr(out), _ptr(lse), _stream(stream))
    _check("qsa_sparse_attn_prefill_paged", rc)
    return out, lse


def sparse_attn_decode_paged(q, row_pos, k_cache, v_cache, page_table, page_tokens: int, sel_blocks, sel_count,
                             tail_start=None, softmax_scale: Optional[float] = None, out=None, lse=None,
                             want_lse=True, workspace=None, stream=None):
    """a7+a9 on a paged K/V pool: k/v [slots][Hkv][D]; page_table [B][pages]."""
    import torch
    _need_contig(q, row_pos, k_cache, v_cache, page_table, sel_blocks, sel_count, tail_start)
    B, Qn, Hq, D = q.shape
    _, Hkv, _ = k_cache.shape
    top_k = sel_blocks.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Qn, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_decode_workspace_size(B, Qn, Hq, D, top_k)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    rc = load().qsa_sparse_attn_decode_paged(_ptr(q), _ptr(row_pos), B, Qn, _ptr(tail_start), _ptr(k_cache),
                                             _ptr(v_cache), _ptr(page_table), page_table.shape[1], int(page_tokens),
                                             _ptr(sel_blocks), _ptr(sel_count), top_k, Hq, Hkv, D, scale,
                                             _dtype_code(q), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                             _stream(stream))
    _check("qsa_sparse_attn_decode_paged", rc)
    return out, lse


def pool_index_keys_paged(raw_keys, page_table, page_tokens: int, block_begin: int, block_end: int,
                          rope_theta: float, pooled=None, codes=None, scales=None, flags: int = 0, stream=None):
    """a1-a3 into a paged compressed-key pool: raw_keys [B][L][128]; `pooled`
    [slots/4][128] (raw dtype), or FP8 `codes` [slots/4][128] uint8 + `scales`
    [slots/4]; block b of sequence s goes to key slot(4b) / 4."""
    _need_contig(raw_keys, page_table, pooled, codes, scales)
    B, L, _ = raw_keys.shape
    rc = load().qsa_pool_index_keys_paged(_ptr(raw_keys), L * INDEX_DIM, _ptr(pooled), _ptr(codes), _ptr(scales),
                                          _ptr(page_table), page_table.shape[1], int(page_tokens), B,
                                          int(block_begin), int(block_end), float(rope_theta), int(flags),
                                          _dtype_code(raw_keys), _stream(stream))
    _check("qsa_pool_index_keys_paged", rc)


def _fp8_codes(t):
    """uint8 codes, or a torch.float8_e4m3fn tensor viewed as its codes."""
    import torch
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def sparse_attn_prefill_fp8kv(q, row_seq, row_pos, k_codes, v_codes, k_scale: float, v_scale: float, sel_blocks,
                              sel_count, page_table=None, page_tokens: int = 0, softmax_scale: Optional[float] = None,
                              out=None, lse=None, want_lse=True, stream=None):
    """a7+a8 on an FP8 K/V cache: E4M3 codes [B][L][Hkv][D] (or [slots][Hkv][D]
    with a page table), values k_scale * E4M3(code) and v_scale * E4M3(code);
    q, out bf16."""
    import torch
    k_codes, v_codes = _fp8_codes(k_codes), _fp8_codes(v_codes)
    _need_contig(q, row_seq, row_pos, k_codes, v_codes, page_table, sel_blocks, sel_count)
    R, Hq, D = q.shape
    Hkv = k_codes.shape[-2]
    stride = 0 if page_table is not None else k_codes.shape[1] * Hkv * D
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((R, Hq), dtype=torch.float32, device=q.device)
    rc = load().qsa_sparse_attn_prefill_fp8kv(
        _ptr(q), _ptr(row_seq), _ptr(row_pos), R, _ptr(k_codes), _ptr(v_codes), stride, _ptr(page_table),
        0 if page_table is None else page_table.shape[1], int(page_tokens), float(k_scale), float(v_scale),
        _ptr(sel_blocks), _ptr(sel_count), sel_blocks.shape[1], Hq, Hkv, D, scale, _ptr(out), _ptr(lse),
        _stream(stream))
    _check("qsa_sparse_attn_prefill_fp8kv", rc)
    return out, lse


def sparse_attn_decode_fp8kv(q, row_pos, k_codes, v_codes, k_scale: float, v_scale: float, sel_blocks, sel_count,
                             tail_start=None, page_table=None, page_tokens: int = 0,
                             softmax_scale: Optional[float] = None, out=None, lse=None, want_lse=True,
                             workspace=None, stream=None):
    """a7+a9 on an FP8 K/V cache (as sparse_attn_prefill_fp8kv)."""
    import torch
    k_codes, v_codes = _fp8_codes(k_codes), _fp8_codes(v_codes)
    _need_contig(q, row_pos, k_codes, v_codes, page_table, sel_blocks, sel_count, tail_start)
    B, Qn, Hq, D = q.shape
    Hkv = k_codes.shape[-2]
    stride = 0 if page_table is not None else k_codes.shape[1] * Hkv * D
    top_k = sel_blocks.shape[1]
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Qn, Hq), dtype=torch.float32, device=q.device)
    need = sparse_attn_decode_workspace_size(B, Qn, Hq, D, top_k)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=q.device)
    rc = load().qsa_sparse_attn_decode_fp8kv(
        _ptr(q), _ptr(row_pos), B, Qn, _ptr(tail_start), _ptr(k_codes), _ptr(v_codes), stride, _ptr(page_table),
        0 if page_table is None else page_table.shape[1], int(page_tokens), float(k_scale), float(v_scale),
        _ptr(sel_blocks), _ptr(sel_count), top_k, Hq, Hkv, D, scale, _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream))
    _check("qsa_sparse_attn_decode_fp8kv", rc)
    return out, lse


# ---------------------------------------------------------------------------
# per-kernel timing (hipEvents on the launch stream)
# ---------------------------------------------------------------------------

def profile_enable(on: bool = True):
    _check("qsa_profile_enable", load().qsa_profile_enable(1 if on else 0))


def profile_reset():
    _check("qsa_profile_reset", load().qsa_profile_reset())


def profile_kernel_ms(name: str):
    """(launches recorded, total ms) of kernel `name` since the last reset."""
    tot = ctypes.c_double(0.0)
    n = load().qsa_profile_kernel_ms(name.encode(), ctypes.byref(tot))
    return int(n), float(tot.value)
