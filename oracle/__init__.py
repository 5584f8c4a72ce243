"""CPU oracle for the QSA hot path (ctypes wrapper over ``qsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library and its Python
binding never import this package.

Every function takes and returns numpy arrays.  bf16 tensors are passed as
``uint16`` bit patterns, fp32 tensors as ``float32``.  The C source cites the
page passage behind each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_oracle.so")

F32 = 0
BF16 = 1
FLAG_NO_ROPE = 1
FLAG_POOL_RMSNORM = 2

DIM = 128
IDX_HEADS = 4
BLOCK = 4

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C99 + OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-D_DEFAULT_SOURCE", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, u32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
    lib.qsa_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.qsa_oracle_bf16_to_double.restype = f64
    lib.qsa_oracle_bf16_from_double.argtypes = [f64]
    lib.qsa_oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.qsa_oracle_rope.argtypes = [P, i64, f64]
    lib.qsa_oracle_rope.restype = None
    lib.qsa_oracle_pool.argtypes = [P, i64, P, i64, i32, i32, i32, f64, u32, i32]
    lib.qsa_oracle_pool.restype = ctypes.c_int
    lib.qsa_oracle_fp8_to_double.argtypes = [ctypes.c_uint8]
    lib.qsa_oracle_fp8_to_double.restype = f64
    lib.qsa_oracle_fp8_from_double.argtypes = [f64]
    lib.qsa_oracle_fp8_from_double.restype = ctypes.c_uint8
    lib.qsa_oracle_fp8_encode.argtypes = [P, P, i64]
    lib.qsa_oracle_fp8_encode.restype = None
    lib.qsa_oracle_pool_fp8.argtypes = [P, i64, P, P, i64, i32, i32, i32, f64, u32, i32]
    lib.qsa_oracle_pool_fp8.restype = ctypes.c_int
    lib.qsa_oracle_score_topk_fp8.argtypes = [P, i32, P, P, i32, P, P, i64, i32, f64, u32, P, P, P, P, i64]
    lib.qsa_oracle_score_topk_fp8.restype = ctypes.c_int
    lib.qsa_oracle_pool_append.argtypes = [P, P, P, P, P, i32, f64, u32, i32]
    lib.qsa_oracle_pool_append.restype = ctypes.c_int
    lib.qsa_oracle_score_topk.argtypes = [P, P, P, i32, P, i64, i32, f64, u32, i32, P, P, P, P, i64]
    lib.qsa_oracle_score_topk.restype = ctypes.c_int
    lib.qsa_oracle_sparse_attn_prefill.argtypes = [P, P, P, i32, P, P, i64, P, P, i32, i32, i32,
                                                   i32, f64, i32, P, P]
    lib.qsa_oracle_sparse_attn_prefill.restype = ctypes.c_int
    lib.qsa_oracle_sparse_attn_decode.argtypes = [P, P, i32, i32, P, P, P, i64, P, P, i32, i32,
                                                  i32, i32, f64, i32, P, P]
    lib.qsa_oracle_sparse_attn_decode.restype = ctypes.c_int
    lib.qsa_oracle_sparse_attn_prefill_fp8kv.argtypes = [P, P, P, i32, P, P, i64, f64, f64, P, P, i32, i32,
                                                         i32, i32, f64, i32, P, P]
    lib.qsa_oracle_sparse_attn_prefill_fp8kv.restype = ctypes.c_int
    lib.qsa_oracle_sparse_attn_decode_fp8kv.argtypes = [P, P, i32, i32, P, P, P, i64, f64, f64, P, P, i32,
                                                        i32, i32, i32, f64, i32, P, P]
    lib.qsa_oracle_sparse_attn_decode_fp8kv.restype = ctypes.c_int
    lib.qsa_oracle_rope_freq.argtypes = [P, i64, P]
    lib.qsa_oracle_rope_freq.restype = None
    lib.qsa_oracle_rope_plain_freq.argtypes = [f64, P]
    lib.qsa_oracle_rope_plain_freq.restype = None
    lib.qsa_oracle_yarn_freq.argtypes = [f64, f64, f64, f64, f64, P]
    lib.qsa_oracle_yarn_freq.restype = ctypes.c_int
    lib.qsa_oracle_pool_ex.argtypes = [P, i64, P, i64, i32, i32, i32, P, P, u32, i32]
    lib.qsa_oracle_pool_ex.restype = ctypes.c_int
    lib.qsa_oracle_score_topk_ex.argtypes = [P, P, P, i32, P, i64, i32, P, u32, i32, P, P, P, P, i64]
    lib.qsa_oracle_score_topk_ex.restype = ctypes.c_int
    lib.qsa_oracle_threads.argtypes = []
    lib.qsa_oracle_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def _dtype_code(arr) -> int:
    if arr.dtype == np.uint16:
        return BF16
    if arr.dtype == np.float32:
        return F32
    raise TypeError(f"oracle takes uint16 (bf16 bits) or float32 arrays, got {arr.dtype}")


def _c(a, dtype=None):
    return np.ascontiguousarray(np.asarray(a) if dtype is None else np.asarray(a, dtype=dtype))


def threads() -> int:
    return int(_load().qsa_oracle_threads())


def bf16_to_float(bits) -> np.ndarray:
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    out = np.array([lib.qsa_oracle_bf16_to_double(int(b)) for b in bits.reshape(-1)], dtype=np.float64)
    return out.reshape(bits.shape)


def bf16_from_float(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    out = np.array([lib.qsa_oracle_bf16_from_double(float(v)) for v in x.reshape(-1)], dtype=np.uint16)
    return out.reshape(x.shape)


def fp8_to_float(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> values (float64, NaN for the NaN codes)."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.qsa_oracle_fp8_to_double(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def fp8_from_float(x) -> np.ndarray:
    """values -> E4M3 codes (uint8), nearest with ties to the even code."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().qsa_oracle_fp8_encode(_ptr(x), _ptr(out), x.size)
    return out


def rope(vec, pos: int, theta: float) -> np.ndarray:
    """Rotate one 128-d vector (float64) at `pos`; returns a new array."""
    v = np.array(vec, dtype=np.float64, copy=True).reshape(DIM)
    _load().qsa_oracle_rope(_ptr(v), int(pos), float(theta))
    return v


def rope_freq(vec, pos: int, inv_freq) -> np.ndarray:
    """Rotate one 128-d vector at `pos` with the 64 pair frequencies given."""
    v = np.array(vec, dtype=np.float64, copy=True).reshape(DIM)
    f = _c(inv_freq, np.float64)
    assert f.shape == (DIM // 2,)
    _load().qsa_oracle_rope_freq(_ptr(v), int(pos), _ptr(f))
    return v


def plain_freq(theta: float) -> np.ndarray:
    """Plain RoPE's pair frequencies theta^(-j/64)."""
    f = np.empty(DIM // 2, np.float64)
    _load().qsa_oracle_rope_plain_freq(float(theta), _ptr(f))
    return f


# YaRN for the 1M-token extension of the 262,144-token native context (see
# qsa_oracle_yarn_freq): scale 4, original context 262,144, ramp 1..32.
YARN_1M = dict(s=4.0, L=262144.0, alpha=1.0, beta=32.0)


def yarn_freq(base: float, s: float, L: float, alpha: float = 1.0, beta: float = 32.0) -> np.ndarray:
    """YaRN's interpolated pair frequencies h(theta_d) (qsa_oracle_yarn_freq)."""
    f = np.empty(DIM // 2, np.float64)
    _check(_load().qsa_oracle_yarn_freq(float(base), float(s), float(L), float(alpha), float(beta), _ptr(f)),
           "yarn_freq")
    return f


def pool_ex(raw, block_begin: int, block_end: int, inv_freq, norm_weight=None, flags: int = 0,
            pooled=None) -> np.ndarray:
    """pool() with the rotation's pair frequencies given and an optional
    learned per-dim weight of the RMS norm (needs FLAG_POOL_RMSNORM)."""
    raw = _c(raw)
    dt = _dtype_code(raw)
    B, L, d = raw.shape
    assert d == DIM and 4 * block_end <= L
    if pooled is None:
        pooled = np.zeros((B, block_end, DIM), dtype=raw.dtype)
    assert pooled.dtype == raw.dtype and pooled.flags.c_contiguous
    f = _c(inv_freq, np.float64)
    w = None if norm_weight is None else _c(norm_weight, np.float32)
    assert f.shape == (DIM // 2,) and (w is None or w.shape == (DIM,))
    rc = _load().qsa_oracle_pool_ex(_ptr(raw), L * DIM, _ptr(pooled), pooled.shape[1] * DIM, B, int(block_begin),
                                    int(block_end), _ptr(f), _ptr(w), int(flags), dt)
    _check(rc, "pool_ex")
    return pooled


def pool(raw, block_begin: int, block_end: int, theta: float, flags: int = 0,
         pooled=None) -> np.ndarray:
    """a1-a3.  raw: [B][L][128] (uint16 bf16 bits or float32).  Returns (or
    fills) pooled [B][NB][128], NB = pooled.shape[1] or block_end."""
    raw = _c(raw)
    dt = _dtype_code(raw)
    B, L, d = raw.shape
    assert d == DIM and 4 * block_end <= L
    if pooled is None:
        pooled = np.zeros((B, block_end, DIM), dtype=raw.dtype)
    assert pooled.dtype == raw.dtype and pooled.flags.c_contiguous
    rc = _load().qsa_oracle_pool(_ptr(raw), L * DIM, _ptr(pooled), pooled.shape[1] * DIM, B,
                                 int(block_begin), int(block_end), float(theta), int(flags), dt)
    _check(rc, "pool")
    return pooled


def pool_fp8(raw, block_begin: int, block_end: int, theta: float, flags: int = 0, codes=None, scales=None):
    """a1-a3 with FP8 storage (see qsa_oracle_pool_fp8).  raw: [B][L][128]
    (uint16 bf16 bits or float32).  Returns (or fills) codes [B][NB][128]
    uint8 and scales [B][NB] float32, NB = codes.shape[1] or block_end."""
    raw = _c(raw)
    dt = _dtype_code(raw)
    B, L, d = raw.shape
    assert d == DIM and 4 * block_end <= L
    if codes is None:
        codes = np.zeros((B, block_end, DIM), dtype=np.uint8)
        scales = np.zeros((B, block_end), dtype=np.float32)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32 and codes.shape[:2] == scales.shape
    assert codes.flags.c_contiguous and scales.flags.c_contiguous
    rc = _load().qsa_oracle_pool_fp8(_ptr(raw), L * DIM, _ptr(codes), _ptr(scales), codes.shape[1], B,
                                     int(block_begin), int(block_end), float(theta), int(flags), dt)
    _check(rc, "pool_fp8")
    return codes, scales


def pool_append(new_keys, positions, full_slots, ring, compressed, theta: float, flags: int = 0):
    """One decode step of incremental pooling (see qsa_oracle_pool_append):
    writes each request's new raw key into its 4-slot ring and, when that
    completes a block, the block's compressed key at full_slot // 4.  `ring`
    [B][4][128] and `compressed` [S][128] are updated in place (contiguous
    numpy arrays of the keys' dtype)."""
    new_keys = _c(new_keys)
    dt = _dtype_code(new_keys)
    for arr in (ring, compressed):
        assert arr.flags["C_CONTIGUOUS"] and arr.dtype == new_keys.dtype
    pos = _c(positions, np.int32)
    slots = _c(full_slots, np.int64)
    B = new_keys.shape[0]
    assert ring.shape == (B, 4, DIM) and pos.shape == (B,) and slots.shape == (B,)
    assert int(slots.max(initial=-1)) // 4 < compressed.shape[0]
    _check(_load().qsa_oracle_pool_append(_ptr(new_keys), _ptr(pos), _ptr(slots), _ptr(ring), _ptr(compressed), B,
                                          float(theta), int(flags), dt), "pool_append")


def score_topk(q_index, row_seq, row_pos, pooled, top_k: int, theta: float, flags: int = 0,
               want_raw: bool = False):
    """a4-a6.  q_index: [R][4][128]; pooled: [B][NB][128].
    Returns (sel [R][top_k] int32, count [R] int32, scores [R][top_k] float32,
    raw [R][NB] float64 or None)."""
    q_index = _c(q_index)
    pooled = _c(pooled)
    dt = _dtype_code(q_index)
    assert _dtype_code(pooled) == dt
    row_seq = _c(row_seq, np.int32)
    row_pos = _c(row_pos, np.int32)
    R = q_index.shape[0]
    NB = pooled.shape[1]
    assert q_index.shape[1:] == (IDX_HEADS, DIM)
    for r in range(R):  # contract: the visible blocks exist
        assert (int(row_pos[r]) + 1) // BLOCK <= NB
    sel = np.empty((R, top_k), np.int32)
    cnt = np.empty((R,), np.int32)
    sc = np.empty((R, top_k), np.float32)
    raw = np.full((R, NB), np.nan, np.float64) if want_raw else None
    rc = _load().qsa_oracle_score_topk(_ptr(q_index), _ptr(row_seq), _ptr(row_pos), R, _ptr(pooled),
                                       NB * DIM, int(top_k), float(theta), int(flags), dt,
                                       _ptr(sel), _ptr(cnt), _ptr(sc), _ptr(raw), NB)
    _check(rc, "score_topk")
    return sel, cnt, sc, raw


def score_topk_ex(q_index, row_seq, row_pos, pooled, top_k: int, inv_freq, flags: int = 0,
                  want_raw: bool = False):
    """score_topk() with the index queries rotated by the given pair
    frequencies (the keys pooled with the same ones)."""
    q_index = _c(q_index)
    pooled = _c(pooled)
    dt = _dtype_code(q_index)
    assert _dtype_code(pooled) == dt
    row_seq = _c(row_seq, np.int32)
    row_pos = _c(row_pos, np.int32)
    R = q_index.shape[0]
    NB = pooled.shape[1]
    assert q_index.shape[1:] == (IDX_HEADS, DIM)
    for r in range(R):
        assert (int(row_pos[r]) + 1) // BLOCK <= NB
    f = _c(inv_freq, np.float64)
    assert f.shape == (DIM // 2,)
    sel = np.empty((R, top_k), np.int32)
    cnt = np.empty((R,), np.int32)
    sc = np.empty((R, top_k), np.float32)
    raw = np.full((R, NB), np.nan, np.float64) if want_raw else None
    rc = _load().qsa_oracle_score_topk_ex(_ptr(q_index), _ptr(row_seq), _ptr(row_pos), R, _ptr(pooled),
                                          NB * DIM, int(top_k), _ptr(f), int(flags), dt,
                                          _ptr(sel), _ptr(cnt), _ptr(sc), _ptr(raw), NB)
    _check(rc, "score_topk_ex")
    return sel, cnt, sc, raw


def score_topk_fp8(q_index, row_seq, row_pos, codes, scales, top_k: int, theta: float, flags: int = 0,
                   want_raw: bool = False):
    """a4-a6 on FP8 keys.  q_index: [R][4][128] (bf16 bits or float32);
    codes: [B][NB][128] uint8; scales: [B][NB] float32.  Returns as
    score_topk."""
    q_index = _c(q_index)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    dt = _dtype_code(q_index)
    row_seq = _c(row_seq, np.int32)
    row_pos = _c(row_pos, np.int32)
    R = q_index.shape[0]
    NB = codes.shape[1]
    assert q_index.shape[1:] == (IDX_HEADS, DIM) and codes.shape[2] == DIM and scales.shape == codes.shape[:2]
    for r in range(R):
        assert (int(row_pos[r]) + 1) // BLOCK <= NB
    sel = np.empty((R, top_k), np.int32)
    cnt = np.empty((R,), np.int32)
    sc = np.empty((R, top_k), np.float32)
    raw = np.full((R, NB), np.nan, np.float64) if want_raw else None
    rc = _load().qsa_oracle_score_topk_fp8(_ptr(q_index), dt, _ptr(row_seq), _ptr(row_pos), R, _ptr(codes),
                                           _ptr(scales), NB, int(top_k), float(theta), int(flags), _ptr(sel),
                                           _ptr(cnt), _ptr(sc), _ptr(raw), NB)
    _check(rc, "score_topk_fp8")
    return sel, cnt, sc, raw


def sparse_attn_prefill(q, row_seq, row_pos, k_cache, v_cache, sel, count, softmax_scale=None):
    """a7+a8.  q: [R][Hq][D]; k/v: [B][L][Hkv][D]; sel: [R][top_k]; count: [R].
    Returns (out [R][Hq][D] same dtype as q, lse [R][Hq] float32)."""
    q = _c(q)
    k_cache = _c(k_cache)
    v_cache = _c(v_cache)
    dt = _dtype_code(q)
    R, Hq, D = q.shape
    B, L, Hkv, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    sel = _c(sel, np.int32)
    count = _c(count, np.int32)
    top_k = sel.shape[1]
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(D)
    out = np.empty_like(q)
    lse = np.empty((R, Hq), np.float32)
    rc = _load().qsa_oracle_sparse_attn_prefill(
        _ptr(q), _ptr(_c(row_seq, np.int32)), _ptr(_c(row_pos, np.int32)), R, _ptr(k_cache),
        _ptr(v_cache), L * Hkv * D, _ptr(sel), _ptr(count), top_k, Hq, Hkv, D, scale, dt, _ptr(out),
        _ptr(lse))
    _check(rc, "sparse_attn_prefill")
    return out, lse


def sparse_attn_decode(q, row_pos, k_cache, v_cache, sel, count, tail_start=None,
                       softmax_scale=None):
    """a7+a9.  q: [B][Qn][Hq][D]; row_pos: [B][Qn]; sel: [B][top_k]; count: [B];
    tail_start: [B] or None.  Returns (out like q, lse [B][Qn][Hq] float32)."""
    q = _c(q)
    k_cache = _c(k_cache)
    v_cache = _c(v_cache)
    dt = _dtype_code(q)
    B, Qn, Hq, D = q.shape
    Bk, L, Hkv, D2 = k_cache.shape
    assert D2 == D and Bk >= B and v_cache.shape == k_cache.shape
    sel = _c(sel, np.int32)
    count = _c(count, np.int32)
    top_k = sel.shape[1]
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(D)
    ts = None if tail_start is None else _c(tail_start, np.int32)
    out = np.empty_like(q)
    lse = np.empty((B, Qn, Hq), np.float32)
    rc = _load().qsa_oracle_sparse_attn_decode(
        _ptr(q), _ptr(_c(row_pos, np.int32)), B, Qn, _ptr(ts), _ptr(k_cache), _ptr(v_cache),
        L * Hkv * D, _ptr(sel), _ptr(count), top_k, Hq, Hkv, D, scale, dt, _ptr(out), _ptr(lse))
    _check(rc, "sparse_attn_decode")
    return out, lse


def sparse_attn_prefill_fp8kv(q, row_seq, row_pos, k_codes, v_codes, k_scale, v_scale, sel, count,
                              softmax_scale=None):
    """a7+a8 on an FP8 K/V cache: k_codes / v_codes [B][L][Hkv][D] uint8 E4M3
    codes whose values are k_scale * E4M3(code) and v_scale * E4M3(code).
    q: [R][Hq][D] (bf16 bits or float32).  Returns (out like q, lse)."""
    q = _c(q)
    k_codes = _c(k_codes, np.uint8)
    v_codes = _c(v_codes, np.uint8)
    dt = _dtype_code(q)
    R, Hq, D = q.shape
    B, L, Hkv, D2 = k_codes.shape
    assert D2 == D and v_codes.shape == k_codes.shape
    sel = _c(sel, np.int32)
    count = _c(count, np.int32)
    top_k = sel.shape[1]
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(D)
    out = np.empty_like(q)
    lse = np.empty((R, Hq), np.float32)
    rc = _load().qsa_oracle_sparse_attn_prefill_fp8kv(
        _ptr(q), _ptr(_c(row_seq, np.int32)), _ptr(_c(row_pos, np.int32)), R, _ptr(k_codes), _ptr(v_codes),
        L * Hkv * D, float(k_scale), float(v_scale), _ptr(sel), _ptr(count), top_k, Hq, Hkv, D, scale, dt,
        _ptr(out), _ptr(lse))
    _check(rc, "sparse_attn_prefill_fp8kv")
    return out, lse


def sparse_attn_decode_fp8kv(q, row_pos, k_codes, v_codes, k_scale, v_scale, sel, count, tail_start=None,
                             softmax_scale=None):
    """a7+a9 on an FP8 K/V cache (as sparse_attn_prefill_fp8kv)."""
    q = _c(q)
    k_codes = _c(k_codes, np.uint8)
    v_codes = _c(v_codes, np.uint8)
    dt = _dtype_code(q)
    B, Qn, Hq, D = q.shape
    Bk, L, Hkv, D2 = k_codes.shape
    assert D2 == D and Bk >= B and v_codes.shape == k_codes.shape
    sel = _c(sel, np.int32)
    count = _c(count, np.int32)
    top_k = sel.shape[1]
    scale = float(softmax_scale) if softmax_scale is not None else 1.0 / np.sqrt(D)
    ts = None if tail_start is None else _c(tail_start, np.int32)
    out = np.empty_like(q)
    lse = np.empty((B, Qn, Hq), np.float32)
    rc = _load().qsa_oracle_sparse_attn_decode_fp8kv(
        _ptr(q), _ptr(_c(row_pos, np.int32)), B, Qn, _ptr(ts), _ptr(k_codes), _ptr(v_codes), L * Hkv * D,
        float(k_scale), float(v_scale), _ptr(sel), _ptr(count), top_k, Hq, Hkv, D, scale, dt, _ptr(out),
        _ptr(lse))
    _check(rc, "sparse_attn_decode_fp8kv")
    return out, lse
