"""Paged KV pool on the GPU ([SGL] "Qwen Sparse Attention": the compressed
keys and K/V live in a paged pool; one compressed key per four token slots at
full_slot / 4).  Every paged path is checked against the oracle on the
logical (unpaged) data, with the tolerances of the contiguous parity tests:
pooled keys within 1 bf16 ulp (codes within one E4M3 step), selections
identical except near-ties within 1e-3 relative of the k-th score, attention
within 2e-2 abs + 1e-2 rel.  Paging only moves data, so each paged call is
also required to equal the contiguous call on the same logical data bit for
bit.  A decode loop writes its compressed keys with qsa_pool_append straight
into the paged pool that the paged scorer reads.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128
THETA = 1.0e7


def _scatter_tokens(x, table, P, n_pages):
    """[B][L][...] contiguous -> [n_pages * P][...] paged by `table`."""
    B, L = x.shape[:2]
    out = np.zeros((n_pages * P,) + x.shape[2:], x.dtype)
    t = np.arange(L)
    for b in range(B):
        out[table[b, t // P].astype(np.int64) * P + t % P] = x[b]
    return out


def _scatter_keys(k, table, P, n_pages):
    """pooled [B][NB][...] -> [n_pages * P / 4][...]: block b of request s at slot(4b) / 4."""
    B, NB = k.shape[:2]
    out = np.zeros((n_pages * P // 4,) + k.shape[2:], k.dtype)
    b = np.arange(NB)
    for s in range(B):
        out[table[s, (4 * b) // P].astype(np.int64) * (P // 4) + b % (P // 4)] = k[s]
    return out


def _layout(rng, B, L, P, spare=7):
    table = synth.page_table(rng, B, L, P, spare)
    return table, table.shape[1] * B + spare


@pytest.mark.parametrize("fmt", ["bf16", "f32", "fp8"])
@pytest.mark.parametrize("P", [4, 64])
def test_pool_paged_equals_contiguous(gpu, fmt, P):
    # a chunk's blocks pooled straight into the paged pool: exactly the
    # contiguous pooling, scattered by the table; pages outside the range keep
    # their contents
    import torch
    rng = np.random.default_rng(91 + P)
    B, NB, b0 = 2, 1500, 300
    raw = rng.standard_normal((B, 4 * NB + 3, DIM)).astype(np.float32)
    dt = "f32" if fmt == "f32" else "bf16"
    raw = synth.bf16_bits(raw) if dt == "bf16" else raw
    table, n_pages = _layout(rng, B, 4 * NB + 3, P)
    nkeys = n_pages * P // 4
    if fmt == "fp8":
        codes = torch.zeros((B, NB, DIM), dtype=torch.uint8, device="cuda")
        scales = torch.zeros((B, NB), dtype=torch.float32, device="cuda")
        qsa.pool_index_keys_fp8(dev(raw, dt), codes, scales, b0, NB, THETA)
        pc = torch.full((nkeys, DIM), 7, dtype=torch.uint8, device="cuda")
        ps = torch.full((nkeys,), -1.0, dtype=torch.float32, device="cuda")
        qsa.pool_index_keys_paged(dev(raw, dt), dev(table, "i"), P, b0, NB, THETA, codes=pc, scales=ps)
        want_c = _scatter_keys(host(codes), table, P, n_pages)
        want_s = _scatter_keys(host(scales), table, P, n_pages)
        got_c, got_s = host(pc), host(ps)
    else:
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        pooled = torch.zeros((B, NB, DIM), dtype=tdt, device="cuda")
        qsa.pool_index_keys(dev(raw, dt), pooled, b0, NB, THETA)
        pp = torch.full((nkeys, DIM), 3.0, dtype=tdt, device="cuda")
        qsa.pool_index_keys_paged(dev(raw, dt), dev(table, "i"), P, b0, NB, THETA, pooled=pp)
        want_c = _scatter_keys(host(pooled), table, P, n_pages)
        got_c = host(pp)
    # keys of blocks [b0, NB) of every sequence
    slots = np.concatenate([table[s, (4 * np.arange(b0, NB)) // P].astype(np.int64) * (P // 4) +
                            np.arange(b0, NB) % (P // 4) for s in range(B)])
    np.testing.assert_array_equal(got_c[slots], want_c[slots])
    if fmt == "fp8":
        np.testing.assert_array_equal(got_s[slots], want_s[slots])
    # the oracle on the logical keys: the paged pool gathered back to [B][NB]
    logical = got_c[slots].reshape(B, NB - b0, DIM)
    if fmt == "fp8":
        o_codes, o_scales = oracle.pool_fp8(raw, b0, NB, THETA)
        np.testing.assert_allclose(got_s[slots].reshape(B, NB - b0), o_scales[:, b0:], rtol=4e-7, atol=0)
        gv, ov = oracle.fp8_to_float(logical), oracle.fp8_to_float(o_codes[:, b0:])
        step = np.where(np.abs(ov) < 2.0 ** -6, 2.0 ** -9,
                        2.0 ** (np.floor(np.log2(np.maximum(np.abs(ov), 2.0 ** -6))) - 3))
        assert np.all(np.abs(gv - ov) <= step * (1 + 1e-9)), "a code is more than one step from the oracle's"
        assert np.mean(logical == o_codes[:, b0:]) > 0.999
    else:
        o_pooled = oracle.pool(raw, b0, NB, THETA)[:, b0:]
        if fmt == "bf16":
            diff = np.abs(logical.astype(np.int32) - o_pooled.astype(np.int32))
            assert diff.max() <= 1 and (diff == 0).mean() > 0.999
        else:
            np.testing.assert_allclose(logical, o_pooled, rtol=2e-6, atol=1e-6)
    untouched = np.setdiff1d(np.arange(nkeys), slots)
    fill = {"fp8": 7, "bf16": synth.bf16_bits(np.float32(3.0)), "f32": 3.0}[fmt]
    assert np.all(got_c[untouched] == fill)
    if fmt == "fp8":
        assert np.all(got_s[untouched] == -1.0)


@pytest.mark.parametrize("P", [16, 256])
@pytest.mark.parametrize("path,R", [("rows", 40), ("gemm", 130)])
def test_score_topk_paged_equals_contiguous(gpu, P, path, R):
    import torch
    rng = np.random.default_rng(81 + P)
    B, NB, k = 3, 5000, 512
    L = 4 * NB
    pooled = synth.bf16_bits(rng.standard_normal((B, NB, DIM)).astype(np.float32))
    iq = synth.bf16_bits(rng.standard_normal((R, 4, DIM)).astype(np.float32))
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, L, R).astype(np.int32)
    pos[:2] = [L - 1, 4 * k + 5]
    table, n_pages = _layout(rng, B, L, P)
    paged = _scatter_keys(pooled, table, P, n_pages)
    flags = qsa.FLAG_SCORE_ROWS if path == "rows" else qsa.FLAG_SCORE_GEMM
    args = (dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"))
    a = [host(x) for x in qsa.score_topk(*args, dev(pooled, "bf16"), NB, k, THETA, flags=flags)]
    b = [host(x) for x in qsa.score_topk_paged(*args, dev(table, "i"), P, NB, k, THETA, pooled=dev(paged, "bf16"),
                                               flags=flags)]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    o_sel, o_cnt, o_sc, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, want_raw=True)
    check_selection(b[0], b[1], o_sel, o_cnt, o_raw, exact=False)
    same = np.array([np.array_equal(b[0][r], o_sel[r]) for r in range(R)])
    np.testing.assert_allclose(b[2][same], o_sc[same], rtol=2e-5, atol=1e-5)   # scaled scores of kept blocks


@pytest.mark.parametrize("path,R", [("rows", 12), ("gemm", 100)])
def test_score_topk_paged_integer_inputs_exact(gpu, path, R):
    # integer keys and queries with RoPE off: every score is exact on both
    # sides, so the paged selection equals the oracle's with no exception
    rng = np.random.default_rng(83)
    B, NB, k, P = 2, 2600, 256, 16
    L = 4 * NB
    pooled = synth.bf16_bits(rng.integers(-3, 4, size=(B, NB, DIM)).astype(np.float32))
    iq = synth.bf16_bits(rng.integers(-2, 3, size=(R, 4, DIM)).astype(np.float32))
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, L, R).astype(np.int32)
    pos[:2] = [L - 1, 4 * k + 1]
    table, n_pages = _layout(rng, B, L, P)
    paged = _scatter_keys(pooled, table, P, n_pages)
    flags = (qsa.FLAG_SCORE_ROWS if path == "rows" else qsa.FLAG_SCORE_GEMM) | qsa.FLAG_NO_ROPE
    got = [host(x) for x in qsa.score_topk_paged(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(table, "i"),
                                                 P, NB, k, THETA, pooled=dev(paged, "bf16"), flags=flags)]
    o_sel, o_cnt, _, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, flags=oracle.FLAG_NO_ROPE,
                                               want_raw=True)
    check_selection(got[0], got[1], o_sel, o_cnt, o_raw, exact=True)


@pytest.mark.parametrize("path,R", [("rows", 8), ("gemm", 100)])
def test_score_topk_paged_fp8_equals_contiguous(gpu, path, R):
    import torch
    rng = np.random.default_rng(85)
    B, NB, k, P = 2, 3000, 256, 32
    L = 4 * NB
    raw = synth.bf16_bits(rng.standard_normal((B, L, DIM)).astype(np.float32))
    codes = torch.zeros((B, NB, DIM), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((B, NB), dtype=torch.float32, device="cuda")
    qsa.pool_index_keys_fp8(dev(raw, "bf16"), codes, scales, 0, NB, THETA)
    iq = synth.bf16_bits(rng.standard_normal((R, 4, DIM)).astype(np.float32))
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, L, R).astype(np.int32)
    table, n_pages = _layout(rng, B, L, P)
    pc = _scatter_keys(host(codes), table, P, n_pages)
    ps = _scatter_keys(host(scales), table, P, n_pages)
    flags = qsa.FLAG_SCORE_ROWS if path == "rows" else qsa.FLAG_SCORE_GEMM
    args = (dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"))
    a = [host(x) for x in qsa.score_topk_fp8(*args, codes, scales, NB, k, THETA, flags=flags)]
    b = [host(x) for x in qsa.score_topk_paged(*args, dev(table, "i"), P, NB, k, THETA,
                                               codes=torch.from_numpy(pc).cuda(), scales=torch.from_numpy(ps).cuda(),
                                               flags=flags)]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # the oracle scores the logical FP8 keys (the GPU's codes and scales)
    o_sel, o_cnt, _, o_raw = oracle.score_topk_fp8(iq, seq, pos, host(codes), host(scales), k, THETA,
                                                   want_raw=True)
    check_selection(b[0], b[1], o_sel, o_cnt, o_raw, exact=False)


@pytest.mark.parametrize("P", [4, 64])
@pytest.mark.parametrize("Hq,Hkv", [(8, 1), (16, 2)])
def test_attn_prefill_paged_equals_contiguous(gpu, P, Hq, Hkv):
    rng = np.random.default_rng(91 + P + Hq)
    B, L, R, k = 2, 6000, 70, 64
    q = synth.bf16_bits(rng.standard_normal((R, Hq, DIM)).astype(np.float32))
    kc = synth.bf16_bits(rng.standard_normal((B, L, Hkv, DIM)).astype(np.float32))
    vc = synth.bf16_bits(rng.standard_normal((B, L, Hkv, DIM)).astype(np.float32))
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, L, R).astype(np.int32)
    pos[:4] = [0, 1, 2, L - 1]
    sel = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        n = min(k, nc)
        if n:
            sel[r, :n] = np.sort(rng.choice(nc, size=n, replace=False))
        cnt[r] = n
    table, n_pages = _layout(rng, B, L, P)
    pk, pv = _scatter_tokens(kc, table, P, n_pages), _scatter_tokens(vc, table, P, n_pages)
    args = (dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"))
    o1, l1 = qsa.sparse_attn_prefill(*args, dev(kc, "bf16"), dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"))
    o2, l2 = qsa.sparse_attn_prefill_paged(*args, dev(pk, "bf16"), dev(pv, "bf16"), dev(table, "i"), P,
                                           dev(sel, "i"), dev(cnt, "i"))
    np.testing.assert_array_equal(host(o1), host(o2))
    np.testing.assert_array_equal(host(l1), host(l2))
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    assert_close_out(host(o2), want, "bf16")
    np.testing.assert_allclose(host(l2), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("P", [8, 128])
def test_attn_decode_paged_equals_contiguous(gpu, P):
    rng = np.random.default_rng(95 + P)
    B, Qn, Hq, Hkv, k = 3, 4, 8, 1, 512
    L = 3000
    q = synth.bf16_bits(rng.standard_normal((B, Qn, Hq, DIM)).astype(np.float32))
    kc = synth.bf16_bits(rng.standard_normal((B, L + Qn, Hkv, DIM)).astype(np.float32))
    vc = synth.bf16_bits(rng.standard_normal((B, L + Qn, Hkv, DIM)).astype(np.float32))
    rpos = (L + np.arange(Qn))[None, :].repeat(B, 0).astype(np.int32)
    ts = np.full(B, L, np.int32)
    nc = L // 4
    sel = np.stack([np.sort(rng.choice(nc, size=k, replace=False)) for _ in range(B)]).astype(np.int32)
    cnt = np.full(B, k, np.int32)
    table, n_pages = _layout(rng, B, L + Qn, P)
    pk, pv = _scatter_tokens(kc, table, P, n_pages), _scatter_tokens(vc, table, P, n_pages)
    o1, l1 = qsa.sparse_attn_decode(dev(q, "bf16"), dev(rpos, "i"), dev(kc, "bf16"), dev(vc, "bf16"),
                                    dev(sel, "i"), dev(cnt, "i"), dev(ts, "i"))
    o2, l2 = qsa.sparse_attn_decode_paged(dev(q, "bf16"), dev(rpos, "i"), dev(pk, "bf16"), dev(pv, "bf16"),
                                          dev(table, "i"), P, dev(sel, "i"), dev(cnt, "i"), dev(ts, "i"))
    np.testing.assert_array_equal(host(o1), host(o2))
    np.testing.assert_array_equal(host(l1), host(l2))
    want, _ = oracle.sparse_attn_decode(q, rpos, kc, vc, sel, cnt, ts)
    assert_close_out(host(o2), want, "bf16")


def test_decode_loop_pool_append_into_paged_pool(gpu):
    # a decode loop: every step appends each request's new raw key through its
    # ring into the paged compressed pool (full_slot from the page table), and
    # the paged scorer then selects from that pool; the selection equals the
    # contiguous pipeline's (whole-sequence pooling, contiguous scorer)
    import torch
    rng = np.random.default_rng(97)
    B, T0, steps, P, k = 3, 4096, 9, 16, 256
    L = T0 + steps
    raw = synth.bf16_bits(rng.standard_normal((B, L, DIM)).astype(np.float32))
    table, n_pages = _layout(rng, B, L, P)
    comp = torch.zeros((n_pages * P // 4, DIM), dtype=torch.bfloat16, device="cuda")
    ring = torch.zeros((B, 4, DIM), dtype=torch.bfloat16, device="cuda")
    raw_d = dev(raw, "bf16")
    slots = table[:, np.arange(L) // P].astype(np.int64) * P + (np.arange(L) % P)[None, :]
    iq = synth.bf16_bits(rng.standard_normal((B, 4, DIM)).astype(np.float32))
    seqs = dev(np.arange(B, dtype=np.int32), "i")
    for t in range(L):   # the whole stream through the ring (prefix then decode steps)
        qsa.pool_append(raw_d[:, t].contiguous(), dev(np.full(B, t, np.int32), "i"),
                        torch.from_numpy(slots[:, t].copy()).cuda(), ring, comp, THETA)
        if t >= T0:
            pos = np.full(B, t, np.int32)
            nb = (t + 1) // 4
            got = [host(x) for x in qsa.score_topk_paged(dev(iq, "bf16"), seqs, dev(pos, "i"), dev(table, "i"), P,
                                                         nb, k, THETA, pooled=comp)]
            pooled = torch.zeros((B, nb, DIM), dtype=torch.bfloat16, device="cuda")
            qsa.pool_index_keys(raw_d, pooled, 0, nb, THETA)
            want = [host(x) for x in qsa.score_topk(dev(iq, "bf16"), seqs, dev(pos, "i"), pooled, nb, k, THETA)]
            for x, y in zip(got, want):
                np.testing.assert_array_equal(x, y)
            # the oracle: the appended keys, gathered to logical order, are the
            # oracle's pooled keys, and the selection is the oracle's on them
            comp_h = host(comp)
            blocks = np.arange(nb)
            logical = np.stack([comp_h[slots[s, 4 * blocks] // 4] for s in range(B)])
            o_pooled = oracle.pool(raw, 0, nb, THETA)
            diff = np.abs(logical.astype(np.int32) - o_pooled.astype(np.int32))
            assert diff.max() <= 1 and (diff == 0).mean() > 0.999
            o_sel, o_cnt, _, o_raw = oracle.score_topk(iq, np.arange(B, dtype=np.int32), pos, logical, k, THETA,
                                                       want_raw=True)
            check_selection(got[0], got[1], o_sel, o_cnt, o_raw, exact=False)
