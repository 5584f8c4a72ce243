"""Attention at the pages' serving shape on the GPU, through the C-ABI: head
dim D = 256 with 24 query heads over 2 KV heads (12 query heads per KV head),
and other query groups that are not powers of two ("Qwen3.8-Flash-Next, Layer
by Layer": the full-attention layers' head layout).  The index side is
unchanged (4 x 128 queries against one 128-d pooled key), so these cases
exercise steps a7-a9.  Output within 2e-2 abs / 1e-2 rel of the oracle (bf16),
lse within 1e-5 rel / 1e-4 abs; paged calls equal contiguous ones bit for bit.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, dev, host

pytestmark = pytest.mark.gpu

WIDE = 256


def _bf16(rng, shape):
    return synth.bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _random_selection(rng, pos, k):
    """A valid selection per row: min(k, nc) distinct blocks < nc, ascending."""
    sel = np.full((len(pos), k), -1, np.int32)
    cnt = np.zeros(len(pos), np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        n = min(k, nc)
        if n:
            sel[r, :n] = np.sort(rng.choice(nc, size=n, replace=False))
        cnt[r] = n
    return sel, cnt


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 24, 2), (256, 8, 1), (256, 4, 4), (256, 48, 2), (128, 24, 2),
                                      (128, 12, 4)])
def test_attn_prefill_wide_matches_oracle(gpu, D, Hq, Hkv):
    # several row tiles, a ragged last tile, rows at t = 0..3 (tails of 1-3
    # tokens, one complete block), and with one query head per KV head 16-row
    # tiles whose 48 tail tokens span two 32-position chunks at D = 256
    rng = np.random.default_rng(300 + D + Hq + Hkv)
    L, R, k = 4 * 700 + 2, 70, 64
    pos = np.sort(rng.choice(L, R, replace=False)).astype(np.int32)
    pos[:4] = [0, 1, 2, 3]
    pos[40:56] = 4 * np.arange(200, 216) + 2          # 16 consecutive rows with 3-token tails
    pos = np.sort(pos)
    seq = np.zeros(R, np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q, kc, vc = _bf16(rng, (R, Hq, D)), _bf16(rng, (1, L, Hkv, D)), _bf16(rng, (1, L, Hkv, D))
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"),
                                       dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


def test_attn_prefill_wide_mixed_sequences(gpu):
    # rows of two sequences interleaved in one tile; overlapping selections
    rng = np.random.default_rng(310)
    B, L, R, k, Hq, Hkv = 2, 4 * 900 + 3, 45, 96, 24, 2
    seq = rng.integers(0, 2, R).astype(np.int32)
    pos = rng.integers(4 * k, L, R).astype(np.int32)
    core = np.sort(rng.choice(k, 40, replace=False))
    sel = np.full((R, k), -1, np.int32)
    cnt = np.full(R, k, np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        own = rng.choice(np.setdiff1d(np.arange(nc), core), k - len(core), replace=False)
        sel[r] = np.sort(np.concatenate([core, own]))
    cnt[7] = 3
    sel[7, 3:] = -1
    q, kc, vc = _bf16(rng, (R, Hq, WIDE)), _bf16(rng, (B, L, Hkv, WIDE)), _bf16(rng, (B, L, Hkv, WIDE))
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt)
    out, lse = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"),
                                       dev(vc, "bf16"), dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("Qn,Hq,Hkv,draft", [(1, 24, 2, False), (4, 24, 2, True), (5, 24, 2, True),
                                             (2, 8, 1, True), (3, 64, 4, False)])
def test_attn_decode_wide_matches_oracle(gpu, Qn, Hq, Hkv, draft):
    # splits of 16 kept blocks are two 32-position chunks at D = 256; a short
    # selection ends inside a split's first chunk
    rng = np.random.default_rng(320 + Qn * Hq)
    B, ctx, k = 3, 4 * 900 + 1, 128
    L = ctx + (Qn if draft else 0)
    if draft:  # IndexShare rows after the anchor at ctx - 1
        rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
        ts = np.full(B, 4 * (ctx // 4), np.int32)
        anchor = np.full(B, ctx - 1, np.int32)
    else:
        rp = rng.integers(4 * k, ctx, size=(B, Qn)).astype(np.int32)
        ts = None
        anchor = rp.min(1)
    sel, cnt = _random_selection(rng, anchor, k)
    cnt[1] = 5
    sel[1, 5:] = -1
    q, kc, vc = _bf16(rng, (B, Qn, Hq, WIDE)), _bf16(rng, (B, L, Hkv, WIDE)), _bf16(rng, (B, L, Hkv, WIDE))
    want, want_lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode(dev(q, "bf16"), dev(rp, "i"), dev(kc, "bf16"), dev(vc, "bf16"),
                                      dev(sel, "i"), dev(cnt, "i"), None if ts is None else dev(ts, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


def _paged(x, table, P, n_pages):
    B, L = x.shape[:2]
    out = np.zeros((n_pages * P,) + x.shape[2:], x.dtype)
    t = np.arange(L)
    for b in range(B):
        out[table[b, t // P].astype(np.int64) * P + t % P] = x[b]
    return out


def test_attn_wide_paged_equals_contiguous(gpu):
    rng = np.random.default_rng(330)
    B, L, R, k, Hq, Hkv, P = 2, 4 * 600 + 3, 30, 64, 24, 2, 32
    table = synth.page_table(rng, B, L, page_tokens=P, spare_pages=5)
    n_pages = int(table.max()) + 1
    kc, vc = _bf16(rng, (B, L, Hkv, WIDE)), _bf16(rng, (B, L, Hkv, WIDE))
    kp, vp = dev(_paged(kc, table, P, n_pages), "bf16"), dev(_paged(vc, table, P, n_pages), "bf16")
    # prefill
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, L, R).astype(np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q = _bf16(rng, (R, Hq, WIDE))
    a = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kc, "bf16"), dev(vc, "bf16"),
                                dev(sel, "i"), dev(cnt, "i"))
    b = qsa.sparse_attn_prefill_paged(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), kp, vp, dev(table, "i"), P,
                                      dev(sel, "i"), dev(cnt, "i"))
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))
    # decode, IndexShare rows
    Qn = 4
    ctx = L - Qn
    rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
    ts = np.full(B, 4 * (ctx // 4), np.int32)
    dsel, dcnt = _random_selection(rng, np.full(B, ctx - 1), k)
    dq = _bf16(rng, (B, Qn, Hq, WIDE))
    a = qsa.sparse_attn_decode(dev(dq, "bf16"), dev(rp, "i"), dev(kc, "bf16"), dev(vc, "bf16"), dev(dsel, "i"),
                               dev(dcnt, "i"), dev(ts, "i"))
    b = qsa.sparse_attn_decode_paged(dev(dq, "bf16"), dev(rp, "i"), kp, vp, dev(table, "i"), P, dev(dsel, "i"),
                                     dev(dcnt, "i"), dev(ts, "i"))
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))


@pytest.mark.parametrize("name,overrides", [
    ("chunk-256k", dict(ctx=65536, chunk=2048)),
    ("decode-1m-draft", dict(ctx=131072)),
])
def test_wide_heads_whole_path_sampled(gpu, name, overrides):
    # the whole path (pool, score, select, attend) on a scaled copy of a
    # workload at the serving head layout; attention of sampled rows (decode:
    # every row) against the oracle on the GPU's selection (the index side
    # does not depend on the head layout and is checked elsewhere)
    spec = synth.scaled(name, Hq=24, Hkv=2, D=WIDE, **overrides)
    w = synth.make(spec)
    raw = dev(w["raw_keys"], "bf16")
    B, nb = raw.shape[0], spec.n_blocks
    import torch
    pooled = torch.zeros((B, nb, 128), dtype=torch.bfloat16, device="cuda")
    qsa.pool_index_keys(raw, pooled, 0, nb, spec.theta)
    max_nb = int((w["row_pos"].max() + 1) // 4)
    sel, cnt, _ = qsa.score_topk(dev(w["idx_q"], "bf16"), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"), pooled,
                                 max_nb, spec.top_k, spec.theta, want_scores=False)
    g_sel, g_cnt = host(sel), host(cnt)
    rng = np.random.default_rng(7)
    kc, vc = dev(w["k_cache"], "bf16"), dev(w["v_cache"], "bf16")
    if spec.kind == "prefill":
        out, lse = qsa.sparse_attn_prefill(dev(w["q"], "bf16"), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"),
                                           kc, vc, sel, cnt)
        rows = np.unique(np.concatenate([[0, spec.chunk - 1], rng.choice(spec.chunk, 14, replace=False)]))
        print(f"[wide] {name}: rows {rows.tolist()}", flush=True)
        want, want_lse = oracle.sparse_attn_prefill(w["q"][rows], w["row_seq"][rows], w["row_pos"][rows],
                                                    w["k_cache"], w["v_cache"], g_sel[rows], g_cnt[rows])
        assert_close_out(host(out)[rows], want, "bf16")
        np.testing.assert_allclose(host(lse)[rows], want_lse, rtol=1e-5, atol=1e-4)
    else:
        ts = None if w["tail_start"] is None else dev(w["tail_start"], "i")
        out, lse = qsa.sparse_attn_decode(dev(w["q"], "bf16"), dev(w["attn_pos"], "i"), kc, vc, sel, cnt, ts)
        want, want_lse = oracle.sparse_attn_decode(w["q"], w["attn_pos"], w["k_cache"], w["v_cache"], g_sel, g_cnt,
                                                   w["tail_start"])
        assert_close_out(host(out), want, "bf16")
        np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("Qn,Hq,Hkv", [(32, 2, 1), (40, 1, 1)])
def test_attn_decode_row_mask_limits(gpu, Qn, Hq, Hkv):
    # 32 rows sharing a selection fill the MFMA path's 32-bit row masks (all
    # bits set for the kept blocks); 40 rows go to the VALU path
    rng = np.random.default_rng(340 + Qn)
    B, ctx, k, D = 2, 4 * 600 + 2, 64, 128
    L = ctx + Qn
    rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
    ts = np.full(B, 4 * (ctx // 4), np.int32)
    sel, cnt = _random_selection(rng, np.full(B, ctx - 1), k)
    q, kc, vc = _bf16(rng, (B, Qn, Hq, D)), _bf16(rng, (B, L, Hkv, D)), _bf16(rng, (B, L, Hkv, D))
    want, want_lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode(dev(q, "bf16"), dev(rp, "i"), dev(kc, "bf16"), dev(vc, "bf16"),
                                      dev(sel, "i"), dev(cnt, "i"), dev(ts, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)
