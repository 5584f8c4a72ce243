"""Parity of the HIP path (through the C-ABI) with the CPU oracle, element by
element, on seeded inputs that span several tiles and end in ragged tails.

Tolerances: pooled keys within 1 bf16 ulp (bit-exact on integer inputs with
RoPE off); selections identical except near-ties within 1e-3 relative of the
k-th score, and identical with no exception on integer inputs; attention
output within 2e-2 abs + 1e-2 rel in bf16 and 1e-4 in fp32.
"""
import math

import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import as_float, assert_close_out, check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128
THETA = 1.0e7


def _store(x, dtype):
    return synth.bf16_bits(x.astype(np.float32)) if dtype == "bf16" else x.astype(np.float32)


def _code(dtype):
    return qsa.BF16 if dtype == "bf16" else qsa.F32


def _random_selection(rng, pos, k):
    """A valid selection per row: min(k, nc) distinct blocks < nc, ascending."""
    R = len(pos)
    sel = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        n = min(k, nc)
        if n:
            sel[r, :n] = np.sort(rng.choice(nc, size=n, replace=False))
        cnt[r] = n
    return sel, cnt


# ---------------------------------------------------------------------------
# a1-a3 pooling
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, qsa.FLAG_NO_ROPE, qsa.FLAG_POOL_RMSNORM])
def test_pool_matches_oracle(gpu, dtype, flags):
    rng = np.random.default_rng(100 + flags)
    B, NB = 2, 517
    L = 4 * NB + 3                                  # a ragged, incomplete last block
    raw = _store(rng.standard_normal((B, L, DIM)) * 2.0, dtype)
    want = oracle.pool(raw, 0, NB, THETA, flags)
    pooled = dev(np.zeros((B, NB, DIM), raw.dtype), dtype)
    qsa.pool_index_keys(dev(raw, dtype), pooled, 0, NB, THETA, flags)
    got = host(pooled)
    if dtype == "bf16":
        diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
        assert diff.max() <= 1 and (diff == 0).mean() > 0.999
    else:
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pool_block_range_only(gpu, dtype):
    rng = np.random.default_rng(7)
    B, NB = 3, 300
    raw = _store(rng.standard_normal((B, 4 * NB, DIM)), dtype)
    sentinel = _store(np.full((B, NB, DIM), 3.25), dtype)
    pooled = dev(sentinel, dtype)
    qsa.pool_index_keys(dev(raw, dtype), pooled, 97, 211, THETA)
    got = host(pooled)
    want = oracle.pool(raw, 97, 211, THETA, pooled=sentinel.copy())
    np.testing.assert_array_equal(got[:, :97], sentinel[:, :97])
    np.testing.assert_array_equal(got[:, 211:], sentinel[:, 211:])
    if dtype == "bf16":
        assert np.abs(got.astype(np.int32) - want.astype(np.int32)).max() <= 1
    else:
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pool_integer_inputs_bit_exact(gpu, dtype):
    rng = np.random.default_rng(8)
    raw = _store(rng.integers(-8, 9, size=(2, 4 * 333, DIM)).astype(np.float32), dtype)
    want = oracle.pool(raw, 0, 333, THETA, qsa.FLAG_NO_ROPE)
    pooled = dev(np.zeros((2, 333, DIM), raw.dtype), dtype)
    qsa.pool_index_keys(dev(raw, dtype), pooled, 0, 333, THETA, qsa.FLAG_NO_ROPE)
    np.testing.assert_array_equal(host(pooled), want)


# ---------------------------------------------------------------------------
# a4-a6 scoring and selection
# ---------------------------------------------------------------------------

PATHS = {"rows": qsa.FLAG_SCORE_ROWS, "gemm": qsa.FLAG_SCORE_GEMM}


def _score_case(seed, dtype, B, NB, R, k, integer=False):
    rng = np.random.default_rng(seed)
    if integer:
        base = rng.integers(-4, 5, size=(7, DIM)).astype(np.float32)
        pooled = base[rng.integers(0, 7, size=(B, NB))]          # few distinct keys -> exact ties
        iq = rng.integers(-3, 4, size=(R, 4, DIM)).astype(np.float32)
    else:
        pooled = rng.standard_normal((B, NB, DIM)).astype(np.float32)
        iq = rng.standard_normal((R, 4, DIM)).astype(np.float32)
    pooled, iq = _store(pooled, dtype), _store(iq, dtype)
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    pos[:3] = [0, 4 * k - 2, 4 * NB - 1]          # no block, just below k blocks, every block
    return pooled, iq, seq, pos


@pytest.mark.parametrize("dtype,path,R,NB", [("bf16", "rows", 90, 2600), ("bf16", "gemm", 90, 2600),
                                             ("f32", "rows", 90, 2600), ("bf16", "rows", 40, 9001),
                                             ("f32", "rows", 13, 9001), ("bf16", "gemm", 40, 9001)])
@pytest.mark.parametrize("k", [512, 37])
def test_score_topk_matches_oracle(gpu, dtype, path, R, NB, k):
    # 90 rows: per-row select; <= 64 rows: the split select (several chunks at 9001 blocks)
    B = 2
    pooled, iq, seq, pos = _score_case(11 + k, dtype, B, NB, R, k)
    o_sel, o_cnt, o_sc, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, want_raw=True)
    sel, cnt, sc = qsa.score_topk(dev(iq, dtype), dev(seq, "i"), dev(pos, "i"), dev(pooled, dtype), NB, k,
                                  THETA, flags=PATHS[path])
    g_sel, g_cnt, g_sc = host(sel), host(cnt), host(sc)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, o_raw, exact=False)
    for r in range(R):
        n = g_cnt[r]
        want = o_raw[r, g_sel[r, :n]] / math.sqrt(128)
        np.testing.assert_allclose(g_sc[r, :n], want, rtol=1e-3, atol=1e-3)
        assert np.all(g_sc[r, n:] == 0)


def test_score_topk_fused_crowded_bin_bit_exact(gpu):
    # integer inputs, 40,000 blocks, k = 512 on the fused scorer: ~5,700 blocks
    # tie at the top score, so no pair list overflows but the k-th key's bin
    # holds more pairs than the merge stages, and the merge walks the lists
    B, R, NB, k = 1, 8, 40000, 512
    pooled, iq, seq, pos = _score_case(9, "bf16", B, NB, R, k, integer=True)
    o_sel, o_cnt, _, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, qsa.FLAG_NO_ROPE, want_raw=True)
    sel, cnt, sc = qsa.score_topk(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(pooled, "bf16"), NB, k,
                                  THETA, flags=qsa.FLAG_NO_ROPE | qsa.FLAG_SCORE_GEMM)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)       # ties resolved to the lower block, exactly
    g_sel, g_cnt, g_sc = host(sel), host(cnt), host(sc)
    for r in range(R):
        n = g_cnt[r]
        np.testing.assert_allclose(g_sc[r, :n], o_raw[r, g_sel[r, :n]] / math.sqrt(128), rtol=1e-6, atol=1e-6)


# (8 rows, 40,000 blocks: ~5,700 blocks share each score value, more tied
# candidates than the split selection stages in LDS)
@pytest.mark.parametrize("dtype,path,R,NB", [("bf16", "rows", 80, 1500), ("bf16", "gemm", 80, 1500),
                                             ("f32", "rows", 80, 1500), ("bf16", "rows", 30, 9001),
                                             ("f32", "rows", 30, 9001), ("bf16", "rows", 8, 40000)])
def test_score_topk_integer_inputs_bit_exact(gpu, dtype, path, R, NB):
    B, k = 2, 64
    pooled, iq, seq, pos = _score_case(5, dtype, B, NB, R, k, integer=True)
    o_sel, o_cnt, o_sc, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, qsa.FLAG_NO_ROPE,
                                                  want_raw=True)
    sel, cnt, sc = qsa.score_topk(dev(iq, dtype), dev(seq, "i"), dev(pos, "i"), dev(pooled, dtype), NB, k,
                                  THETA, flags=qsa.FLAG_NO_ROPE | PATHS[path])
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)       # ties resolved to the lower block, exactly
    np.testing.assert_array_equal(host(sc), o_sc)


def test_score_topk_all_ties_lowest_blocks_win(gpu):
    # every pooled key identical: every visible block scores the same, so the
    # kept set is blocks 0..k-1 (ties go to the lower block).  With 4,100 rows
    # the fused scorer's per-split pair buffers overflow and the merge redoes
    # the rows from recomputed scores.
    rng = np.random.default_rng(17)
    NB, R, k = 40000, 4100, 512
    key = rng.integers(-4, 5, size=DIM).astype(np.float32)
    pooled = synth.bf16_bits(np.broadcast_to(key, (1, NB, DIM)).copy())
    iq = rng.integers(-3, 4, size=(R, 4, DIM)).astype(np.float32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    pos[:2] = [4 * NB - 1, 4 * k + 1]
    sel, cnt, sc = qsa.score_topk(dev(synth.bf16_bits(iq), "bf16"), dev(np.zeros(R, np.int32), "i"),
                                  dev(pos, "i"), dev(pooled, "bf16"), NB, k, THETA, flags=qsa.FLAG_NO_ROPE)
    sel, cnt, sc = host(sel), host(cnt), host(sc)
    raw = np.maximum(iq.astype(np.float64) @ key.astype(np.float64), 0).sum(1)
    for r in range(R):
        n = min(k, (int(pos[r]) + 1) // 4)
        assert cnt[r] == n
        np.testing.assert_array_equal(sel[r, :n], np.arange(n))
        assert np.all(sel[r, n:] == -1)
        np.testing.assert_array_equal(sc[r, :n], np.float32(raw[r] / math.sqrt(128)))


@pytest.mark.parametrize("n_high,n_tied", [(600, 1600), (300, 1900)])
def test_score_topk_long_pair_lists_exact(gpu, n_high, n_tied):
    # Rows whose filter keeps more pairs than the merge stages at once.
    # Block scores are exact integers: n_high distinct values >= 1024, n_tied
    # blocks at 100, the rest at 1.  The sampled threshold lands on 100, so
    # every row keeps n_high + n_tied = 2,200 pairs.  With 600 distinct high
    # values the k-th best key's bin is narrow and only its pairs are staged;
    # with 300 the k-th best is one of the ties and its bin alone exceeds the
    # stage (the list-walking path).  Either way: exact, lowest tied blocks.
    rng = np.random.default_rng(31 + n_high)
    NB, R, k = 8192, 64, 512
    exps = np.arange(10, 16)
    mant = np.arange(128)
    pool_vals = ((128 + mant[None, :]) * 2.0 ** (exps[:, None] - 7)).ravel().astype(np.float32)
    vals = np.ones(NB, np.float32)
    blocks = rng.permutation(NB)
    vals[blocks[:n_high]] = rng.choice(pool_vals, size=n_high, replace=False)
    vals[blocks[n_high:n_high + n_tied]] = 100.0
    pooled = np.zeros((1, NB, DIM), np.float32)
    pooled[0, :, 0] = vals
    iq = np.zeros((R, 4, DIM), np.float32)
    iq[:, 0, 0] = rng.integers(1, 5, R)            # head 0 reads dim 0; raw = q * value, exact
    pooled, iq = synth.bf16_bits(pooled), synth.bf16_bits(iq)
    seq = np.zeros(R, np.int32)
    pos = np.full(R, 4 * NB - 1, np.int32)
    o_sel, o_cnt, o_sc, _ = oracle.score_topk(iq, seq, pos, pooled, k, THETA, qsa.FLAG_NO_ROPE)
    sel, cnt, sc = qsa.score_topk(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(pooled, "bf16"), NB, k,
                                  THETA, flags=qsa.FLAG_NO_ROPE | qsa.FLAG_SCORE_GEMM)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)
    np.testing.assert_array_equal(host(sc), o_sc)


def test_score_topk_default_paths_agree(gpu):
    # few rows take the streaming scorer, many rows the GEMM: same answer
    B, NB, R, k = 1, 3000, 130, 100
    pooled, iq, seq, pos = _score_case(21, "bf16", B, NB, R, k)
    args = (dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(pooled, "bf16"), NB, k, THETA)
    a = [host(x) for x in qsa.score_topk(*args)]
    b = [host(x) for x in qsa.score_topk(*args, flags=qsa.FLAG_SCORE_ROWS)]
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# a7-a9 attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (16, 2), (4, 4), (6, 2), (32, 1)])
def test_attn_prefill_matches_oracle(gpu, dtype, Hq, Hkv):
    rng = np.random.default_rng(30 + Hq + Hkv)
    L, R, k = 4 * 700 + 2, 70, 64
    pos = np.sort(rng.choice(L, R, replace=False)).astype(np.int32)
    pos[:4] = [0, 1, 2, 3]                        # tails of 1..3 tokens, one complete block
    seq = np.zeros(R, np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q = _store(rng.standard_normal((R, Hq, DIM)), dtype)
    kc = _store(rng.standard_normal((1, L, Hkv, DIM)), dtype)
    vc = _store(rng.standard_normal((1, L, Hkv, DIM)), dtype)
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, dtype), dev(seq, "i"), dev(pos, "i"), dev(kc, dtype),
                                       dev(vc, dtype), dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, dtype)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


def test_attn_prefill_overlapping_and_mixed_sequences(gpu):
    # consecutive rows whose selections overlap (a shared core plus own blocks),
    # rows of two sequences interleaved, and runs of identical rows
    rng = np.random.default_rng(33)
    B, L, R, k, Hq, Hkv = 2, 4 * 900 + 3, 77, 96, 8, 1
    seq = rng.integers(0, 2, R).astype(np.int32)
    seq[20:40] = 1
    pos = rng.integers(4 * k, L, R).astype(np.int32)
    pos[50:60] = pos[50]
    core = np.sort(rng.choice(4 * k // 4, 60, replace=False))
    sel = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        own = rng.choice(np.setdiff1d(np.arange(nc), core), k - len(core), replace=False)
        s_ = np.sort(np.concatenate([core, own]))
        sel[r] = s_
        cnt[r] = k
    sel[55] = sel[50]
    q = synth.bf16_bits(rng.standard_normal((R, Hq, DIM)).astype(np.float32))
    kc = synth.bf16_bits(rng.standard_normal((B, L, Hkv, DIM)).astype(np.float32))
    vc = synth.bf16_bits(rng.standard_normal((B, L, Hkv, DIM)).astype(np.float32))
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"),
                                       dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5, 1e-3])
@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (4, 4)])
def test_attn_softmax_scale_sign_and_zero(gpu, scale, Hq, Hkv):
    # the kernels keep the exponent scale positive: a negative softmax_scale
    # is carried by the queries' sign, a zero one gives every attended
    # position the same weight
    rng = np.random.default_rng(36)
    L, R, k = 4 * 300 + 1, 37, 32
    pos = np.sort(rng.choice(L, R, replace=False)).astype(np.int32)
    pos[:3] = [0, 5, 6]
    seq = np.zeros(R, np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q = synth.bf16_bits(rng.standard_normal((R, Hq, DIM)).astype(np.float32))
    kc = synth.bf16_bits(rng.standard_normal((1, L, Hkv, DIM)).astype(np.float32))
    vc = synth.bf16_bits(rng.standard_normal((1, L, Hkv, DIM)).astype(np.float32))
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt, softmax_scale=scale)
    out, lse = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"),
                                       dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"), softmax_scale=scale)
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)
    # decode: the last row of each of two sequences, sharing the prefill's cache
    B = 2
    qd = synth.bf16_bits(rng.standard_normal((B, 1, Hq, DIM)).astype(np.float32))
    kd = np.concatenate([kc, kc[:, ::-1]], axis=0)
    vd = np.concatenate([vc, vc[:, ::-1]], axis=0)
    pd = np.array([[L - 1], [L - 3]], np.int32)
    seld, cntd = _random_selection(rng, pd[:, 0], k)
    want, want_lse = oracle.sparse_attn_decode(qd, pd, kd, vd, seld, cntd, softmax_scale=scale)
    out, lse = qsa.sparse_attn_decode(dev(qd, "bf16"), dev(pd, "i"), dev(kd, "bf16"), dev(vd, "bf16"),
                                      dev(seld, "i"), dev(cntd, "i"), softmax_scale=scale)
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


def test_attn_prefill_union_across_windows(gpu):
    # the prefill kernel builds a tile's union of kept blocks one window of
    # 65,536 blocks at a time: kept blocks on both sides of each window edge,
    # a ragged third window, rows keeping fewer blocks, and tiles of 16 rows
    # (8 query heads per KV head) with a ragged last tile
    rng = np.random.default_rng(35)
    W = 65536
    NB = 2 * W + 5001
    L, R, k, Hq, Hkv = 4 * NB + 2, 40, 128, 8, 1
    pos = np.sort(rng.integers(4 * (W + 16), L, R)).astype(np.int32)
    pos[-1] = L - 1
    edges = np.array([0, 1, W - 2, W - 1, W, W + 1, 2 * W - 1, 2 * W, 2 * W + 1, NB - 1], np.int64)
    sel = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        base = edges[edges < nc]
        n = k if r % 7 else k // 3
        extra = rng.choice(nc, size=3 * k, replace=False)
        extra = extra[~np.isin(extra, base)][: n - len(base)]
        sel[r, :n] = np.sort(np.concatenate([base, extra]))
        cnt[r] = n
    print(f"[windows] attention prefill L={L} rows={R} k={k}", flush=True)
    q = synth.bf16_bits(rng.standard_normal((R, Hq, DIM)).astype(np.float32))
    kc = synth.bf16_bits(rng.standard_normal((1, L, Hkv, DIM)).astype(np.float32))
    vc = synth.bf16_bits(rng.standard_normal((1, L, Hkv, DIM)).astype(np.float32))
    seq = np.zeros(R, np.int32)
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"),
                                       dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (4, 4)])
def test_attn_prefill_tails_share_blocks_and_skip_unwritten(gpu, Hq, Hkv):
    # runs of consecutive rows (a row's tail block is a kept, fully visible
    # block of the rows 4 positions later), rows at the first positions (a
    # tail and nothing else), two sequences; every cache position past a
    # sequence's last row holds NaN, as memory never written may: no row
    # attends those tokens, and none of them may reach the result
    rng = np.random.default_rng(37)
    B, L, k = 2, 4 * 600 + 3, 64
    runs = [(0, np.arange(0, 7)), (0, np.arange(1500, 1540)), (1, np.arange(900, 925)),
            (1, np.arange(2, 4)), (0, np.array([2001]))]
    seq = np.concatenate([np.full(len(p_), s_, np.int32) for s_, p_ in runs])
    pos = np.concatenate([p_ for _, p_ in runs]).astype(np.int32)
    R = len(pos)
    sel = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        n = min(k, nc)
        if n:
            recent = np.arange(max(0, nc - 6), nc)          # the blocks holding earlier rows' tails
            rest = rng.permutation(np.setdiff1d(np.arange(nc), recent))[: max(0, n - len(recent))]
            sel[r, :n] = np.sort(np.concatenate([recent, rest]))[:n]
        cnt[r] = n
    q = synth.bf16_bits(rng.standard_normal((R, Hq, DIM)).astype(np.float32))
    kf = rng.standard_normal((B, L, Hkv, DIM)).astype(np.float32)
    vf = rng.standard_normal((B, L, Hkv, DIM)).astype(np.float32)
    for b in range(B):
        last = pos[seq == b].max()
        kf[b, last + 1:] = np.nan
        vf[b, last + 1:] = np.nan
    kc, vc = synth.bf16_bits(kf), synth.bf16_bits(vf)
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    assert np.isfinite(synth.bf16_to_f32(want)).all()
    out, lse = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"),
                                       dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Qn,Hq,Hkv,draft", [(1, 8, 1, False), (4, 8, 1, True), (2, 16, 2, True),
                                             (3, 4, 2, False), (2, 6, 2, True), (8, 8, 1, True)])
def test_attn_decode_matches_oracle(gpu, dtype, Qn, Hq, Hkv, draft):
    rng = np.random.default_rng(40 + Qn * Hq)
    B, ctx, k = 3, 4 * 900 + 1, 128
    L = ctx + (Qn if draft else 0)
    if draft:  # IndexShare rows after the anchor at ctx - 1
        rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
        ts = np.full(B, 4 * (ctx // 4), np.int32)
        anchor = np.full(B, ctx - 1, np.int32)
    else:      # independent rows at (possibly) different positions, own tails
        rp = rng.integers(4 * k, ctx, size=(B, Qn)).astype(np.int32)
        ts = None
        anchor = rp.min(1)
    sel, cnt = _random_selection(rng, anchor, k)
    cnt[1] = 5                                     # a short selection
    sel[1, 5:] = -1
    q = _store(rng.standard_normal((B, Qn, Hq, DIM)), dtype)
    kc = _store(rng.standard_normal((B, L, Hkv, DIM)), dtype)
    vc = _store(rng.standard_normal((B, L, Hkv, DIM)), dtype)
    want, want_lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode(dev(q, dtype), dev(rp, "i"), dev(kc, dtype), dev(vc, dtype),
                                      dev(sel, "i"), dev(cnt, "i"),
                                      None if ts is None else dev(ts, "i"))
    assert_close_out(host(out), want, dtype)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


# ---------------------------------------------------------------------------
# the whole path on scaled-down copies of the five workloads
# ---------------------------------------------------------------------------

SCALED = {
    "decode-8k-f32": dict(ctx=4 * 1200 + 2),
    "prefill-32k": dict(ctx=4 * 700, chunk=4 * 700),
    "decode-128k": dict(batch=5, ctx=4 * 2500 + 3),
    "chunk-256k": dict(ctx=4 * 3000, chunk=150, n_plant=60),
    "decode-1m-draft": dict(ctx=4 * 3000),
}


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_whole_path_scaled(gpu, name):
    spec = synth.scaled(name, **SCALED[name])
    w = synth.make(spec)
    dt = spec.dtype
    B, nb, k = spec.batch, spec.n_blocks, spec.top_k
    # a1-a3
    pooled_d = dev(np.zeros((B, nb, DIM), w["raw_keys"].dtype), dt)
    qsa.pool_index_keys(dev(w["raw_keys"], dt), pooled_d, 0, nb, spec.theta)
    pooled = host(pooled_d)
    o_pooled = oracle.pool(w["raw_keys"], 0, nb, spec.theta)
    if dt == "bf16":
        assert np.abs(pooled.astype(np.int32) - o_pooled.astype(np.int32)).max() <= 1
    else:
        np.testing.assert_allclose(pooled, o_pooled, rtol=2e-6, atol=1e-6)
    # a4-a6 (the oracle scores the GPU's pooled keys, so pooling rounding does not cascade)
    max_nb = int((w["row_pos"].max() + 1) // 4)
    sel, cnt, _ = qsa.score_topk(dev(w["idx_q"], dt), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"),
                                 pooled_d, max_nb, k, spec.theta)
    o_sel, o_cnt, _, o_raw = oracle.score_topk(w["idx_q"], w["row_seq"], w["row_pos"], pooled, k,
                                               spec.theta, want_raw=True)
    g_sel, g_cnt = host(sel), host(cnt)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, o_raw, exact=False)
    # planted blocks are found
    if spec.kind == "decode":
        for s in range(B):
            planted = set(w["planted"][s].tolist())
            got = set(g_sel[s, :g_cnt[s]].tolist())
            assert planted <= got if len(planted) <= k else got <= planted
    # a7-a9 on the GPU's own selection
    if spec.kind == "decode":
        ts = None if w["tail_start"] is None else dev(w["tail_start"], "i")
        out, lse = qsa.sparse_attn_decode(dev(w["q"], dt), dev(w["attn_pos"], "i"), dev(w["k_cache"], dt),
                                          dev(w["v_cache"], dt), sel, cnt, ts)
        want, want_lse = oracle.sparse_attn_decode(w["q"], w["attn_pos"], w["k_cache"], w["v_cache"], g_sel,
                                                   g_cnt, w["tail_start"])
    else:
        out, lse = qsa.sparse_attn_prefill(dev(w["q"], dt), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"),
                                           dev(w["k_cache"], dt), dev(w["v_cache"], dt), sel, cnt)
        want, want_lse = oracle.sparse_attn_prefill(w["q"], w["row_seq"], w["row_pos"], w["k_cache"],
                                                    w["v_cache"], g_sel, g_cnt)
    assert_close_out(host(out), want, dt)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


def test_empty_calls_launch_nothing(gpu):
    import torch
    e = torch.empty((0, 4, DIM), dtype=torch.bfloat16, device="cuda")
    i = torch.empty((0,), dtype=torch.int32, device="cuda")
    pooled = torch.zeros((1, 8, DIM), dtype=torch.bfloat16, device="cuda")
    sel, cnt, sc = qsa.score_topk(e, i, i, pooled, 8, 16, THETA)
    assert sel.shape == (0, 16)
    torch.cuda.synchronize()
