"""Parity at the extremes of the selection budget: top_k = 1 (the degenerate
selection of a single block) and top_k = QSA_MAX_TOP_K = 4096 (the largest
budget the C-ABI accepts), through both scorers, both attention entry points
and both dtypes, against the CPU oracle.

At 4096 the fused scorer's sampled threshold rests on more candidates than
its lanes keep, so every visible block is listed and the rows overflow the
merge's stage; the prefill attention fits only two rows' selections per tile,
and decode runs 257 splits.  Rows whose visible blocks number fewer than
top_k keep them all.  Also the largest query group (QSA_MAX_QUERY_GROUP = 64
queries on one KV head and one selection) in prefill and decode, at head dims
128 and 256.  Tolerances are those of the other parity tests.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128
THETA = 1.0e7
MAX_K = 4096
PATHS = {"rows": qsa.FLAG_SCORE_ROWS, "gemm": qsa.FLAG_SCORE_GEMM}


def _store(x, dtype):
    return synth.bf16_bits(np.asarray(x, np.float32)) if dtype == "bf16" else np.asarray(x, np.float32)


def _selection(rng, anchor, k):
    """min(k, nc) distinct visible blocks per row, ascending, -1 padded."""
    sel = np.full((len(anchor), k), -1, np.int32)
    cnt = np.zeros(len(anchor), np.int32)
    for r, t in enumerate(anchor):
        nc = (int(t) + 1) // 4
        n = min(k, nc)
        if n:
            sel[r, :n] = np.sort(rng.choice(nc, size=n, replace=False))
        cnt[r] = n
    return sel, cnt


@pytest.mark.parametrize("k,path,dtype,R", [(1, "rows", "bf16", 40), (1, "gemm", "bf16", 90), (1, "rows", "f32", 40),
                                            (MAX_K, "rows", "bf16", 40), (MAX_K, "gemm", "bf16", 90),
                                            (MAX_K, "rows", "f32", 24)])
def test_score_topk_extreme_k(gpu, k, path, dtype, R):
    rng = np.random.default_rng(50 + k + R)
    B, NB = 2, 12000
    pooled = _store(rng.standard_normal((B, NB, DIM)), dtype)
    iq = _store(rng.standard_normal((R, 4, DIM)), dtype)
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    pos[:4] = [0, 4 * k - 2, 4 * k + 3, 4 * NB - 1]   # no block, one short of k, k + 1, every block
    o_sel, o_cnt, _, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, want_raw=True)
    sel, cnt, sc = qsa.score_topk(dev(iq, dtype), dev(seq, "i"), dev(pos, "i"), dev(pooled, dtype), NB, k, THETA,
                                  flags=PATHS[path])
    g_sel, g_cnt, g_sc = host(sel), host(cnt), host(sc)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, o_raw, exact=False)
    for r in range(R):
        n = g_cnt[r]
        np.testing.assert_allclose(g_sc[r, :n], o_raw[r, g_sel[r, :n]] / np.sqrt(128.0), rtol=1e-3, atol=1e-3)
        assert np.all(g_sc[r, n:] == 0)


@pytest.mark.parametrize("path", ["rows", "gemm"])
def test_score_topk_max_k_integer_ties_bit_exact(gpu, path):
    # few distinct integer keys: thousands of blocks share each score, and the
    # 4096-th best is cut among them by block id, exactly
    rng = np.random.default_rng(57)
    B, NB, R, k = 1, 12000, 40 if path == "rows" else 70, MAX_K
    base = rng.integers(-4, 5, size=(7, DIM)).astype(np.float32)
    pooled = _store(base[rng.integers(0, 7, size=(B, NB))], "bf16")
    iq = _store(rng.integers(-3, 4, size=(R, 4, DIM)), "bf16")
    seq = np.zeros(R, np.int32)
    pos = rng.integers(4 * k, 4 * NB, R).astype(np.int32)
    o_sel, o_cnt, _, _ = oracle.score_topk(iq, seq, pos, pooled, k, THETA, qsa.FLAG_NO_ROPE, want_raw=True)
    sel, cnt, _ = qsa.score_topk(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(pooled, "bf16"), NB, k, THETA,
                                 flags=qsa.FLAG_NO_ROPE | PATHS[path])
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)


@pytest.mark.parametrize("k", [1, MAX_K])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attn_prefill_extreme_k(gpu, k, dtype):
    rng = np.random.default_rng(60 + k)
    Hq, Hkv = 8, 1
    L, R = 4 * 9000 + 2, 21
    pos = np.sort(rng.choice(L, R, replace=False)).astype(np.int32)
    pos[:3] = [2, 4 * k - 1, 4 * k + 6]        # a tail alone; exactly k blocks; k + 1 blocks and a tail
    pos = np.sort(pos)
    seq = np.zeros(R, np.int32)
    sel, cnt = _selection(rng, pos, k)
    q = _store(rng.standard_normal((R, Hq, DIM)), dtype)
    kc = _store(rng.standard_normal((1, L, Hkv, DIM)), dtype)
    vc = _store(rng.standard_normal((1, L, Hkv, DIM)), dtype)
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, dtype), dev(seq, "i"), dev(pos, "i"), dev(kc, dtype), dev(vc, dtype),
                                       dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, dtype)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("k", [1, MAX_K])
@pytest.mark.parametrize("dtype,Qn,draft", [("bf16", 1, False), ("bf16", 4, True), ("f32", 4, True)])
def test_attn_decode_extreme_k(gpu, k, dtype, Qn, draft):
    rng = np.random.default_rng(70 + k + Qn)
    B, ctx, Hq, Hkv = 2, 4 * 6000 + 1, 8, 1
    L = ctx + (Qn if draft else 0)
    if draft:
        rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
        ts = np.full(B, 4 * (ctx // 4), np.int32)
        anchor = np.full(B, ctx - 1, np.int32)
    else:
        rp = rng.integers(4 * k, ctx, size=(B, Qn)).astype(np.int32)
        ts = None
        anchor = rp.min(1)
    sel, cnt = _selection(rng, anchor, k)
    q = _store(rng.standard_normal((B, Qn, Hq, DIM)), dtype)
    kc = _store(rng.standard_normal((B, L, Hkv, DIM)), dtype)
    vc = _store(rng.standard_normal((B, L, Hkv, DIM)), dtype)
    want, want_lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode(dev(q, dtype), dev(rp, "i"), dev(kc, dtype), dev(vc, dtype), dev(sel, "i"),
                                      dev(cnt, "i"), None if ts is None else dev(ts, "i"))
    assert_close_out(host(out), want, dtype)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


# ---------------------------------------------------------------------------
# the largest query group the C-ABI accepts: QSA_MAX_QUERY_GROUP = 64 queries
# share one KV head and one selection (64 query heads per KV head, or decode
# rows x heads = 64)
# ---------------------------------------------------------------------------

MAX_GROUP = 64


@pytest.mark.parametrize("D,Hq,Hkv,dtype", [(128, 64, 1, "bf16"), (128, 128, 2, "bf16"), (128, 64, 1, "f32"),
                                            (256, 64, 1, "bf16")])
def test_attn_prefill_max_query_group(gpu, D, Hq, Hkv, dtype):
    assert Hq // Hkv == MAX_GROUP
    rng = np.random.default_rng(80 + D + Hq)
    L, R, k = 4 * 500 + 3, 19, 48
    pos = np.sort(rng.choice(L, R, replace=False)).astype(np.int32)
    pos[:3] = [1, 4 * k - 1, L - 1]
    pos = np.sort(pos)
    seq = np.zeros(R, np.int32)
    sel, cnt = _selection(rng, pos, k)
    q = _store(rng.standard_normal((R, Hq, D)), dtype)
    kc = _store(rng.standard_normal((1, L, Hkv, D)), dtype)
    vc = _store(rng.standard_normal((1, L, Hkv, D)), dtype)
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, dtype), dev(seq, "i"), dev(pos, "i"), dev(kc, dtype), dev(vc, dtype),
                                       dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, dtype)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("D,Qn,Hq,Hkv,dtype,draft", [(128, 1, 64, 1, "bf16", False), (128, 4, 16, 1, "bf16", True),
                                                     (128, 1, 128, 2, "f32", False), (256, 2, 32, 1, "bf16", True)])
def test_attn_decode_max_query_group(gpu, D, Qn, Hq, Hkv, dtype, draft):
    assert Qn * (Hq // Hkv) == MAX_GROUP
    rng = np.random.default_rng(90 + D + Qn * Hq)
    B, ctx, k = 3, 4 * 700 + 2, 96
    L = ctx + (Qn if draft else 0)
    if draft:
        rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
        ts = np.full(B, 4 * (ctx // 4), np.int32)
        anchor = np.full(B, ctx - 1, np.int32)
    else:
        rp = rng.integers(4 * k, ctx, size=(B, Qn)).astype(np.int32)
        ts = None
        anchor = rp.min(1)
    sel, cnt = _selection(rng, anchor, k)
    q = _store(rng.standard_normal((B, Qn, Hq, D)), dtype)
    kc = _store(rng.standard_normal((B, L, Hkv, D)), dtype)
    vc = _store(rng.standard_normal((B, L, Hkv, D)), dtype)
    want, want_lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode(dev(q, dtype), dev(rp, "i"), dev(kc, dtype), dev(vc, dtype), dev(sel, "i"),
                                      dev(cnt, "i"), None if ts is None else dev(ts, "i"))
    assert_close_out(host(out), want, dtype)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


# ---------------------------------------------------------------------------
# decode launches of two to four rounds of workgroups: each workgroup takes
# several 16-block groups of the selection (here 3: 48-block splits)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,Qn,Hq,Hkv,D,draft", [(40, 1, 8, 1, 128, False), (16, 2, 24, 2, 256, True),
                                                 (24, 4, 8, 1, 128, True)])
def test_attn_decode_merged_splits(gpu, B, Qn, Hq, Hkv, D, draft):
    rng = np.random.default_rng(100 + B + D)
    ctx, k = 4 * 700 + 1, 512
    L = ctx + (Qn if draft else 0)
    if draft:
        rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
        ts = np.full(B, 4 * (ctx // 4), np.int32)
        anchor = np.full(B, ctx - 1, np.int32)
    else:
        rp = rng.integers(4 * k, ctx, size=(B, Qn)).astype(np.int32)
        ts = None
        anchor = rp.min(1)
    sel, cnt = _selection(rng, anchor, k)
    for s_, c in zip(range(1, 8), [5, 47, 48, 49, 96, 145, 511]):  # selections ending inside and on split edges
        cnt[s_] = c
        sel[s_, c:] = -1
    q = _store(rng.standard_normal((B, Qn, Hq, D)), "bf16")
    kc = _store(rng.standard_normal((B, L, Hkv, D)), "bf16")
    vc = _store(rng.standard_normal((B, L, Hkv, D)), "bf16")
    want, want_lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode(dev(q, "bf16"), dev(rp, "i"), dev(kc, "bf16"), dev(vc, "bf16"), dev(sel, "i"),
                                      dev(cnt, "i"), None if ts is None else dev(ts, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)
