"""The C-ABI boundary without a GPU: the library loads, exports every symbol
include/qsa.h declares, and rejects bad arguments on the host before any HIP
call (so none of these calls touches a device)."""
import ctypes
import os
import re

import pytest

from block_sparse_long_amd import qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "qsa.h")

# fake, 256-byte aligned "device" addresses: validation never dereferences them
A = 0x10000
B_ = 0x20000
C = 0x30000
MIS = 0x10008  # 8-byte aligned only


def declared_functions():
    text = open(HDR).read()
    return sorted(set(re.findall(r"\b(qsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_exports(libqsa):
    decl = declared_functions()
    assert set(decl) == set(qsa.EXPORTS)
    for name in decl:
        assert hasattr(libqsa, name), name


def test_exports_are_c_symbols(libqsa):
    raw = ctypes.CDLL(qsa.LIB_PATH)
    for name in declared_functions():
        assert ctypes.cast(getattr(raw, name), ctypes.c_void_p).value


def test_status_strings(libqsa):
    assert qsa.status_string(qsa.OK) == "ok"
    assert "workspace" in qsa.status_string(qsa.ERR_WORKSPACE)
    assert qsa.status_string(99) == "unknown status"


def test_pool_validation(libqsa):
    f = libqsa.qsa_pool_index_keys
    # empty work -> OK, no launch
    assert f(A, 1024, B_, 256, 0, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.OK
    assert f(A, 1024, B_, 256, 2, 3, 3, 1e7, 0, qsa.BF16, None) == qsa.OK
    assert f(A, 1024, B_, 256, 2, 0, 2, 1e7, 0, 7, None) == qsa.ERR_UNSUPPORTED
    assert f(None, 1024, B_, 256, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(MIS, 1024, B_, 256, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, 1024, B_, 256, 2, 2, 1, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # end < begin
    assert f(A, 1024, B_, 256, -1, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, 1020, B_, 256, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # stride % 8
    assert f(A, 512, B_, 256, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG   # raw stride short
    assert f(A, 1024, B_, 128, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # pooled short
    assert f(A, 1024, B_, 256, 2, 0, 2, 0.5, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # theta
    assert f(A, 1024, B_, 256, 2, 0, 2, 1e7, 1 << 5, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # flag


def test_pool_append_validation(libqsa):
    f = libqsa.qsa_pool_append
    assert f(A, B_, C, A, B_, 0, 1e7, 0, qsa.BF16, None) == qsa.OK            # empty batch
    assert f(A, B_, C, A, B_, 2, 1e7, 0, 7, None) == qsa.ERR_UNSUPPORTED
    assert f(None, B_, C, A, B_, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(MIS, B_, C, A, B_, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # keys not 16-byte aligned
    assert f(A, None, C, A, B_, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, B_, None, A, B_, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, B_, C, A, MIS, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, B_, C, A, B_, -1, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, B_, C, A, B_, 2, 0.5, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG     # theta
    assert f(A, B_, C, A, B_, 2, 1e7, 1 << 8, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # a score flag


def test_score_topk_validation(libqsa):
    f = libqsa.qsa_score_topk
    ws = qsa.score_topk_workspace_size(4, 100, 16, qsa.BF16)
    assert ws > 0 and qsa.score_topk_workspace_size(0, 100, 16, qsa.BF16) == 0
    assert qsa.score_topk_workspace_size(4, 100, 0, qsa.BF16) == 0
    assert qsa.score_topk_workspace_size(4, 100, 16, qsa.BF16, 1 << 12) == 0
    # many rows: the fused scorer keeps no score matrix; the per-row scorer does
    big = qsa.score_topk_workspace_size(8192, 65536, 512, qsa.BF16, qsa.FLAG_SCORE_ROWS)
    fused = qsa.score_topk_workspace_size(8192, 65536, 512, qsa.BF16)
    assert big >= 8192 * 65536 * 4 and fused < big
    good = dict(q=A, seq=B_, pos=C, rows=4, pooled=A, stride=128 * 100, nb=100, k=16, theta=1e7,
                flags=0, dt=qsa.BF16, sel=B_, cnt=C, sc=None, ws=0x100000, wsb=ws)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["q"], a["seq"], a["pos"], a["rows"], a["pooled"], a["stride"], a["nb"], a["k"],
                 a["theta"], a["flags"], a["dt"], a["sel"], a["cnt"], a["sc"], a["ws"], a["wsb"], None)

    assert call(rows=0) == qsa.OK
    assert call(wsb=ws - 1) == qsa.ERR_WORKSPACE
    assert call(ws=0x100010) == qsa.ERR_INVALID_ARG      # workspace not 256-aligned
    assert call(k=0) == qsa.ERR_INVALID_ARG
    assert call(k=qsa.MAX_TOP_K + 1) == qsa.ERR_INVALID_ARG
    assert call(q=None) == qsa.ERR_INVALID_ARG
    assert call(q=MIS) == qsa.ERR_INVALID_ARG
    assert call(sel=None) == qsa.ERR_INVALID_ARG
    assert call(nb=-1) == qsa.ERR_INVALID_ARG
    assert call(dt=5) == qsa.ERR_UNSUPPORTED
    assert call(flags=qsa.FLAG_SCORE_ROWS | qsa.FLAG_SCORE_GEMM) == qsa.ERR_INVALID_ARG
    assert call(flags=qsa.FLAG_SCORE_GEMM, dt=qsa.F32,
                wsb=qsa.score_topk_workspace_size(4, 100, 16, qsa.F32)) == qsa.ERR_UNSUPPORTED
    fws = qsa.score_topk_workspace_size(4, 100, 16, qsa.BF16, qsa.FLAG_SCORE_GEMM)
    assert fws > 0 and fws != ws                              # the flag picks another layout
    assert call(flags=qsa.FLAG_SCORE_GEMM, wsb=fws - 1) == qsa.ERR_WORKSPACE
    assert call(flags=qsa.FLAG_POOL_RMSNORM) == qsa.ERR_INVALID_ARG  # pooling flag, not a score flag
    assert call(theta=float("nan")) == qsa.ERR_INVALID_ARG


def test_ex_validation(libqsa):
    # qsa_pool_index_keys_ex / qsa_score_topk_ex: the rotation and the norm
    # weight are checked before any HIP call
    import ctypes as ct
    f = libqsa.qsa_pool_index_keys_ex
    good = qsa.rope(1e7, 4.0, 262144.0, 1.0, 32.0)
    nf = qsa.FLAG_POOL_RMSNORM

    def pool(rope=good, w=None, flags=0, batch=1, dt=qsa.BF16):
        rp = ct.byref(rope) if rope is not None else None
        return f(A, 4 * 128 * 100, B_, 128 * 100, batch, 0, 100, rp, w, flags, dt, None)

    assert pool(batch=0) == qsa.OK
    assert pool(rope=None) == qsa.ERR_INVALID_ARG                   # rotation without parameters
    assert pool(w=C) == qsa.ERR_INVALID_ARG                         # a weight without the norm
    assert pool(w=C + 2, flags=nf) == qsa.ERR_INVALID_ARG           # misaligned weight
    assert pool(rope=qsa.rope(1.0)) == qsa.ERR_INVALID_ARG          # base must exceed 1
    assert pool(rope=qsa.rope(1e7, 0.5, 262144.0)) == qsa.ERR_INVALID_ARG
    assert pool(rope=qsa.rope(1e7, 4.0, 0.0)) == qsa.ERR_INVALID_ARG
    assert pool(rope=qsa.rope(1e7, 4.0, 262144.0, 32.0, 1.0)) == qsa.ERR_INVALID_ARG
    assert pool(rope=qsa.rope(1e7, float("inf"), 262144.0)) == qsa.ERR_INVALID_ARG
    assert pool(flags=1 << 5) == qsa.ERR_INVALID_ARG
    assert pool(dt=7) == qsa.ERR_UNSUPPORTED
    g = libqsa.qsa_score_topk_ex
    ws = qsa.score_topk_workspace_size(4, 100, 16, qsa.BF16)

    def score(rope=good, flags=0, rows=4, k=16):
        rp = ct.byref(rope) if rope is not None else None
        return g(A, B_, C, rows, A, 128 * 100, 100, k, rp, flags, qsa.BF16, B_, C, None, 0x100000, ws, None)

    assert score(rows=0) == qsa.OK
    assert score(rope=None) == qsa.ERR_INVALID_ARG
    assert score(rope=qsa.rope(1e7, 2.0, -5.0)) == qsa.ERR_INVALID_ARG
    assert score(k=0) == qsa.ERR_INVALID_ARG
    assert score(flags=qsa.FLAG_POOL_RMSNORM) == qsa.ERR_INVALID_ARG


def test_merge_modes_offset(libqsa):
    # the fused scorer's per-row merge record sits inside its workspace; the
    # per-row scorer keeps none
    for rows, nb, k, flags in ((8192, 65536, 512, 0), (100, 5000, 37, qsa.FLAG_SCORE_GEMM)):
        ws = qsa.score_topk_workspace_size(rows, nb, k, qsa.BF16, flags)
        off = qsa.score_topk_merge_modes_offset(rows, nb, k, qsa.BF16, flags)
        assert off is not None and off % 256 == 0 and off + 4 * rows <= ws
    assert qsa.score_topk_merge_modes_offset(4, 100, 16, qsa.BF16) is None          # few rows: per-row path
    assert qsa.score_topk_merge_modes_offset(8192, 65536, 512, qsa.BF16, qsa.FLAG_SCORE_ROWS) is None
    assert qsa.score_topk_merge_modes_offset(0, 100, 16, qsa.BF16) is None
    assert qsa.score_topk_merge_modes_offset(100, 100, 0, qsa.BF16) is None


def test_fp8_validation(libqsa):
    f = libqsa.qsa_pool_index_keys_fp8
    assert f(A, 1024, B_, C, 8, 0, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.OK          # empty batch
    assert f(A, 1024, B_, C, 8, 2, 0, 2, 1e7, 0, 7, None) == qsa.ERR_UNSUPPORTED
    assert f(A, 1024, MIS, C, 8, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # codes misaligned
    assert f(A, 1024, B_, None, 8, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG
    assert f(A, 1024, B_, C + 2, 8, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # scales misaligned
    assert f(A, 1024, B_, C, 1, 2, 0, 2, 1e7, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # stride < blocks
    assert f(A, 1024, B_, C, 8, 2, 0, 2, 0.5, 0, qsa.BF16, None) == qsa.ERR_INVALID_ARG  # theta
    g = libqsa.qsa_score_topk_fp8
    ws = qsa.score_topk_fp8_workspace_size(4, 100, 16)
    assert ws == qsa.score_topk_workspace_size(4, 100, 16, qsa.BF16)
    assert g(A, B_, C, 0, B_, C, 100, 100, 16, 1e7, 0, B_, C, None, 0x100000, ws, None) == qsa.OK
    assert g(A, B_, C, 4, B_, C, 100, 100, 16, 1e7, 0, B_, C, None, 0x100000, ws - 1, None) == qsa.ERR_WORKSPACE
    assert g(A, B_, C, 4, MIS, C, 100, 100, 16, 1e7, 0, B_, C, None, 0x100000, ws, None) == qsa.ERR_INVALID_ARG
    assert g(A, B_, C, 4, B_, None, 100, 100, 16, 1e7, 0, B_, C, None, 0x100000, ws, None) == qsa.ERR_INVALID_ARG
    assert g(A, B_, C, 4, B_, C, 100, 100, 0, 1e7, 0, B_, C, None, 0x100000, ws, None) == qsa.ERR_INVALID_ARG
    assert g(A, B_, C, 4, B_, C, -1, 100, 16, 1e7, 0, B_, C, None, 0x100000, ws, None) == qsa.ERR_INVALID_ARG


def test_paged_validation(libqsa):
    ws = qsa.score_topk_workspace_size(4, 100, 16, qsa.BF16)
    g = libqsa.qsa_score_topk_paged

    def score(**kw):
        a = dict(q=A, seq=B_, pos=C, rows=4, pooled=A, codes=None, scales=None, table=C, pts=100, P=16, nb=100,
                 k=16, th=1e7, flags=0, dt=qsa.BF16, sel=B_, cnt=C, sc=None, ws=0x100000, wsb=ws)
        a.update(kw)
        return g(a["q"], a["seq"], a["pos"], a["rows"], a["pooled"], a["codes"], a["scales"], a["table"], a["pts"],
                 a["P"], a["nb"], a["k"], a["th"], a["flags"], a["dt"], a["sel"], a["cnt"], a["sc"], a["ws"],
                 a["wsb"], None)

    assert score(rows=0) == qsa.OK
    assert score(P=6) == qsa.ERR_INVALID_ARG              # pages must hold whole blocks
    assert score(P=0) == qsa.ERR_INVALID_ARG
    assert score(table=None) == qsa.ERR_INVALID_ARG
    assert score(pts=1) == qsa.ERR_INVALID_ARG            # the table cannot cover 100 blocks
    assert score(pooled=MIS) == qsa.ERR_INVALID_ARG
    assert score(pooled=A, codes=B_, scales=C) == qsa.ERR_INVALID_ARG  # both key formats
    assert score(pooled=None, codes=B_, scales=C, dt=qsa.F32) == qsa.ERR_UNSUPPORTED
    assert score(wsb=ws - 1) == qsa.ERR_WORKSPACE
    f = libqsa.qsa_sparse_attn_prefill_paged
    args = [A, B_, C, 4, A, B_, C, 100, 16, B_, C, 16, 8, 1, 128, 0.1, qsa.BF16, A, None, None]
    assert f(*args[:3], 0, *args[4:]) == qsa.OK
    bad = list(args)
    bad[8] = 10
    assert f(*bad) == qsa.ERR_INVALID_ARG                 # page_tokens % 4
    bad = list(args)
    bad[6] = None
    assert f(*bad) == qsa.ERR_INVALID_ARG                 # no table
    bad = list(args)
    bad[16] = qsa.F32
    assert f(*bad) == qsa.ERR_UNSUPPORTED                 # the paged gather is the bf16 MFMA path's
    d = libqsa.qsa_sparse_attn_decode_paged
    wsa = qsa.sparse_attn_decode_workspace_size(2, 1, 8, 128, 16)
    dargs = [A, B_, 2, 1, None, A, B_, C, 100, 16, B_, C, 16, 8, 1, 128, 0.1, qsa.BF16, A, None, 0x100000, wsa, None]
    assert d(*dargs[:2], 0, *dargs[3:]) == qsa.OK
    bad = list(dargs)
    bad[9] = 2
    assert d(*bad) == qsa.ERR_INVALID_ARG
    bad = list(dargs)
    bad[7] = None
    assert d(*bad) == qsa.ERR_INVALID_ARG


def test_pool_paged_validation(libqsa):
    f = libqsa.qsa_pool_index_keys_paged
    # raw, raw_stride, pooled, codes, scales, table, pt_stride, P, batch, b0, b1, theta, flags, dtype, stream
    args = [A, 1024, B_, None, None, C, 10, 16, 2, 0, 40, 1e7, 0, qsa.BF16, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a8=0) == qsa.OK
    assert call(a10=0) == qsa.OK                                    # empty block range
    assert call(a7=6) == qsa.ERR_INVALID_ARG                        # pages hold whole blocks
    assert call(a5=None) == qsa.ERR_INVALID_ARG
    assert call(a10=41) == qsa.ERR_INVALID_ARG                      # 10 pages x 4 blocks cover 40
    assert call(a3=B_, a4=C) == qsa.ERR_INVALID_ARG                 # both key formats
    assert call(a2=MIS) == qsa.ERR_INVALID_ARG
    assert call(a13=9) == qsa.ERR_UNSUPPORTED
    assert call(a11=0.5) == qsa.ERR_INVALID_ARG


def test_attn_validation(libqsa):
    fp = libqsa.qsa_sparse_attn_prefill
    # rows == 0 -> OK without touching anything
    assert fp(None, None, None, 0, None, None, 0, None, None, 512, 8, 1, 128, 0.1, qsa.BF16, None, None,
              None) == qsa.OK
    args = [A, B_, C, 4, A, B_, 1024, C, A, 512, 8, 1, 128, 0.1, qsa.BF16, B_, None, None]

    def call(i, v):
        a = list(args)
        a[i] = v
        return fp(*a)

    assert fp(*args[:12], 64, *args[13:]) == qsa.ERR_UNSUPPORTED       # D is 128 or 256
    assert fp(*args[:12], 192, *args[13:]) == qsa.ERR_UNSUPPORTED
    assert fp(*args[:12], 256, *args[13:14], qsa.F32, *args[15:]) == qsa.ERR_UNSUPPORTED  # D = 256: bf16 only
    assert call(11, 3) == qsa.ERR_INVALID_ARG                          # Hq % Hkv
    assert call(10, 128) == qsa.ERR_UNSUPPORTED                        # group of 128 heads
    assert call(9, 0) == qsa.ERR_INVALID_ARG                           # top_k
    assert call(0, MIS) == qsa.ERR_INVALID_ARG
    assert call(6, 1001) == qsa.ERR_INVALID_ARG                        # kv stride % 8
    assert call(14, 9) == qsa.ERR_UNSUPPORTED
    assert call(13, float("inf")) == qsa.ERR_INVALID_ARG

    fd = libqsa.qsa_sparse_attn_decode
    ws = qsa.sparse_attn_decode_workspace_size(4, 4, 8, 128, 512)
    assert ws == 4 * 4 * 8 * (4 * 512 // 64 + 1) * 130 * 4
    d = [A, B_, 4, 4, None, A, B_, 1024, C, A, 512, 8, 1, 128, 0.1, qsa.BF16, B_, None, 0x100000, ws, None]

    def dcall(i, v):
        a = list(d)
        a[i] = v
        return fd(*a)

    assert dcall(19, ws - 1) == qsa.ERR_WORKSPACE
    assert dcall(3, 9) == qsa.ERR_UNSUPPORTED                          # 9 rows x 8 heads > 64
    assert dcall(3, 0) == qsa.ERR_INVALID_ARG
    assert dcall(2, 0) == qsa.OK
    ws256 = qsa.sparse_attn_decode_workspace_size(4, 4, 24, 256, 512)
    assert ws256 == 4 * 4 * 24 * (4 * 512 // 64 + 1) * 258 * 4
    assert qsa.sparse_attn_decode_workspace_size(4, 4, 8, 192, 512) == 0
    d256 = list(d)
    d256[11], d256[12], d256[13], d256[19] = 24, 2, 256, ws256
    assert fd(*d256[:15], qsa.F32, *d256[16:]) == qsa.ERR_UNSUPPORTED    # D = 256: bf16 only
    assert fd(*d256[:3], 33, *d256[4:11], 2, 2, *d256[13:]) == qsa.ERR_UNSUPPORTED  # 33 rows > 32 masks
    assert fd(*d256[:19], ws256 - 1, *d256[20:]) == qsa.ERR_WORKSPACE
    assert dcall(18, 0x100004) == qsa.ERR_INVALID_ARG
    assert dcall(1, None) == qsa.ERR_INVALID_ARG


def test_attn_decode_noalloc_validation(libqsa):
    # the allocation-free decode: qsa_sparse_attn_decode's checks, then the
    # static scratch's limit, all before any HIP call
    fn = libqsa.qsa_sparse_attn_decode_noalloc
    d = [A, B_, 4, 4, None, A, B_, 1024, C, A, 512, 8, 1, 128, 0.1, qsa.BF16, B_, None, None]

    def call(i, v):
        a = list(d)
        a[i] = v
        return fn(*a)

    assert call(2, 0) == qsa.OK                                        # nothing to do
    assert call(3, 9) == qsa.ERR_UNSUPPORTED                           # 9 rows x 8 heads > 64
    assert call(0, MIS) == qsa.ERR_INVALID_ARG
    assert call(1, None) == qsa.ERR_INVALID_ARG
    assert call(10, 0) == qsa.ERR_INVALID_ARG
    assert call(13, 64) == qsa.ERR_UNSUPPORTED
    # a call whose partials would not fit the static scratch is refused
    big = 200
    assert qsa.sparse_attn_decode_workspace_size(big, 1, 8, 128, 512) > qsa.NOALLOC_SCRATCH_BYTES
    assert qsa.sparse_attn_decode_workspace_size(100, 1, 8, 128, 512) <= qsa.NOALLOC_SCRATCH_BYTES
    a = list(d)
    a[2], a[3] = big, 1
    assert fn(*a) == qsa.ERR_WORKSPACE
    hdr = open(HDR).read()
    assert f"#define QSA_NOALLOC_SCRATCH_BYTES (16u << 20)" in hdr and qsa.NOALLOC_SCRATCH_BYTES == 16 << 20


def test_profile_api_without_launches(libqsa):
    qsa.profile_enable(True)
    qsa.profile_reset()
    assert qsa.profile_kernel_ms("score_rows_bf16") == (0, 0.0)
    qsa.profile_enable(False)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(qsa, "LIB_PATH", str(tmp_path / "libqsa.so"))
    monkeypatch.setattr(qsa, "_lib", None)
    with pytest.raises(qsa.QsaLibraryMissing):
        qsa.load()


def test_fp8kv_validation(libqsa):
    f = libqsa.qsa_sparse_attn_prefill_fp8kv
    # q, seq, pos, rows, k, v, stride, table, pt_stride, P, ks, vs, sel, cnt, top_k, Hq, Hkv, D, scale, out, lse, st
    args = [A, B_, C, 4, A, B_, 1024, None, 0, 0, 0.02, 0.03, C, A, 512, 8, 1, 128, 0.1, B_, None, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a3=0) == qsa.OK
    assert call(a10=0.0) == qsa.ERR_INVALID_ARG                     # scales must be positive and finite
    assert call(a11=float("nan")) == qsa.ERR_INVALID_ARG
    assert call(a10=-1.0) == qsa.ERR_INVALID_ARG
    assert call(a6=1032) == qsa.ERR_INVALID_ARG                     # stride: 16-byte rows of codes
    assert call(a4=MIS) == qsa.ERR_INVALID_ARG
    assert call(a17=192) == qsa.ERR_UNSUPPORTED
    assert call(a15=256, a16=2) == qsa.ERR_UNSUPPORTED              # a group of 128 heads
    assert call(a7=C, a8=100, a9=6) == qsa.ERR_INVALID_ARG           # pages hold whole blocks
    d = libqsa.qsa_sparse_attn_decode_fp8kv
    ws = qsa.sparse_attn_decode_workspace_size(4, 4, 24, 256, 512)
    dargs = [A, B_, 4, 4, None, A, B_, 1024, None, 0, 0, 0.02, 0.03, C, A, 512, 24, 2, 256, 0.1, B_, None, 0x100000,
             ws, None]

    def dcall(**kw):
        a = list(dargs)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return d(*a)

    assert dcall(a2=0) == qsa.OK
    assert dcall(a23=ws - 1) == qsa.ERR_WORKSPACE
    assert dcall(a12=0.0) == qsa.ERR_INVALID_ARG
    assert dcall(a3=6) == qsa.ERR_UNSUPPORTED                       # 6 rows x 12 heads > 64
    assert dcall(a8=C, a9=100, a10=2) == qsa.ERR_INVALID_ARG
