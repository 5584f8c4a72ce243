"""FP8 K/V cache for attention on the GPU, through the C-ABI ("Qwen3.8-Flash-
Next, Layer by Layer", section "Serving it": the KV cache kept in FP8).  The
caches hold E4M3 codes; values are k_scale * E4M3(code) and v_scale *
E4M3(code).  Output within 2e-2 abs / 1e-2 rel of the oracle (bf16 q and out),
lse within 1e-5 rel / 1e-4 abs.  With power-of-two scales the FP8 path must
equal the bf16 path on the decoded values bit for bit (the codes widen to
bf16 exactly and the scales move by exact powers of two), and paged calls
equal contiguous ones bit for bit.
"""
import math

import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, dev, host

pytestmark = pytest.mark.gpu


def _bf16(rng, shape):
    return synth.bf16_bits(rng.standard_normal(shape).astype(np.float32))


def _codes(rng, shape):
    """Random finite E4M3 codes, values spread like N(0,1) * 448 / 4.5."""
    x = rng.standard_normal(shape).astype(np.float32) * (448.0 / 4.5)
    return oracle.fp8_from_float(np.clip(x, -448.0, 448.0))


def _random_selection(rng, pos, k):
    sel = np.full((len(pos), k), -1, np.int32)
    cnt = np.zeros(len(pos), np.int32)
    for r, t in enumerate(pos):
        nc = (int(t) + 1) // 4
        n = min(k, nc)
        if n:
            sel[r, :n] = np.sort(rng.choice(nc, size=n, replace=False))
        cnt[r] = n
    return sel, cnt


def _u8(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 1), (128, 16, 2), (256, 24, 2), (256, 8, 1)])
def test_fp8kv_prefill_matches_oracle(gpu, D, Hq, Hkv):
    rng = np.random.default_rng(500 + D + Hq)
    L, R, k = 4 * 700 + 2, 70, 64
    pos = np.sort(rng.choice(L, R, replace=False)).astype(np.int32)
    pos[:4] = [0, 1, 2, 3]
    seq = np.zeros(R, np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q = _bf16(rng, (R, Hq, D))
    kc, vc = _codes(rng, (1, L, Hkv, D)), _codes(rng, (1, L, Hkv, D))
    ks, vs = 0.0173, 0.0291
    want, want_lse = oracle.sparse_attn_prefill_fp8kv(q, seq, pos, kc, vc, ks, vs, sel, cnt)
    out, lse = qsa.sparse_attn_prefill_fp8kv(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), _u8(kc), _u8(vc), ks, vs,
                                             dev(sel, "i"), dev(cnt, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("D,Qn,Hq,Hkv,draft", [(128, 1, 8, 1, False), (128, 4, 8, 1, True), (256, 4, 24, 2, True),
                                               (256, 2, 16, 2, False)])
def test_fp8kv_decode_matches_oracle(gpu, D, Qn, Hq, Hkv, draft):
    rng = np.random.default_rng(520 + D + Qn * Hq)
    B, ctx, k = 3, 4 * 900 + 1, 128
    L = ctx + (Qn if draft else 0)
    if draft:
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
    q = _bf16(rng, (B, Qn, Hq, D))
    kc, vc = _codes(rng, (B, L, Hkv, D)), _codes(rng, (B, L, Hkv, D))
    ks, vs = 0.0211, 0.0157
    want, want_lse = oracle.sparse_attn_decode_fp8kv(q, rp, kc, vc, ks, vs, sel, cnt, ts)
    out, lse = qsa.sparse_attn_decode_fp8kv(dev(q, "bf16"), dev(rp, "i"), _u8(kc), _u8(vc), ks, vs, dev(sel, "i"),
                                            dev(cnt, "i"), None if ts is None else dev(ts, "i"))
    assert_close_out(host(out), want, "bf16")
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 1), (256, 24, 2)])
def test_fp8kv_equals_bf16_path_on_exact_values(gpu, D, Hq, Hkv):
    # integer codes (|v| <= 16) times power-of-two scales are bf16 values:
    # the FP8 cache and the bf16 cache of the same values agree bit for bit
    rng = np.random.default_rng(540 + D)
    L, R, k = 4 * 400 + 1, 40, 48
    pos = rng.integers(0, L, R).astype(np.int32)
    seq = np.zeros(R, np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q = _bf16(rng, (R, Hq, D))
    kint = rng.integers(-16, 17, size=(1, L, Hkv, D)).astype(np.float32)
    vint = rng.integers(-16, 17, size=(1, L, Hkv, D)).astype(np.float32)
    kc, vc = oracle.fp8_from_float(kint), oracle.fp8_from_float(vint)
    ks, vs = 0.125, 2.0 ** -5
    kb, vb = synth.bf16_bits(kint * ks), synth.bf16_bits(vint * vs)
    a = qsa.sparse_attn_prefill_fp8kv(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), _u8(kc), _u8(vc), ks, vs,
                                      dev(sel, "i"), dev(cnt, "i"))
    b = qsa.sparse_attn_prefill(dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(kb, "bf16"), dev(vb, "bf16"),
                                dev(sel, "i"), dev(cnt, "i"))
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))
    # decode: 2 sequences x 3 draft rows
    B, Qn = 2, 3
    kc2, vc2 = np.repeat(kc, B, 0), np.repeat(vc, B, 0)
    kb2, vb2 = np.repeat(kb, B, 0), np.repeat(vb, B, 0)
    ctx = L - Qn
    rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
    ts = np.full(B, 4 * (ctx // 4), np.int32)
    dsel, dcnt = _random_selection(rng, np.full(B, ctx - 1), k)
    dq = _bf16(rng, (B, Qn, Hq, D))
    a = qsa.sparse_attn_decode_fp8kv(dev(dq, "bf16"), dev(rp, "i"), _u8(kc2), _u8(vc2), ks, vs, dev(dsel, "i"),
                                     dev(dcnt, "i"), dev(ts, "i"))
    b = qsa.sparse_attn_decode(dev(dq, "bf16"), dev(rp, "i"), dev(kb2, "bf16"), dev(vb2, "bf16"), dev(dsel, "i"),
                               dev(dcnt, "i"), dev(ts, "i"))
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))


def test_fp8kv_paged_equals_contiguous(gpu):
    rng = np.random.default_rng(560)
    B, L, R, k, Hq, Hkv, D, P = 2, 4 * 500 + 3, 30, 64, 24, 2, 256, 16
    table = synth.page_table(rng, B, L, page_tokens=P, spare_pages=3)
    n_pages = int(table.max()) + 1
    kc, vc = _codes(rng, (B, L, Hkv, D)), _codes(rng, (B, L, Hkv, D))

    def paged(x):
        out = np.zeros((n_pages * P,) + x.shape[2:], x.dtype)
        t = np.arange(L)
        for b in range(B):
            out[table[b, t // P].astype(np.int64) * P + t % P] = x[b]
        return out

    kp, vp, tb = _u8(paged(kc)), _u8(paged(vc)), dev(table, "i")
    ks, vs = 0.031, 0.012
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, L, R).astype(np.int32)
    sel, cnt = _random_selection(rng, pos, k)
    q = _bf16(rng, (R, Hq, D))
    args = (dev(q, "bf16"), dev(seq, "i"), dev(pos, "i"))
    a = qsa.sparse_attn_prefill_fp8kv(*args, _u8(kc), _u8(vc), ks, vs, dev(sel, "i"), dev(cnt, "i"))
    b = qsa.sparse_attn_prefill_fp8kv(*args, kp, vp, ks, vs, dev(sel, "i"), dev(cnt, "i"), page_table=tb,
                                      page_tokens=P)
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))
    Qn = 4
    ctx = L - Qn
    rp = (ctx + np.tile(np.arange(Qn), (B, 1))).astype(np.int32)
    ts = np.full(B, 4 * (ctx // 4), np.int32)
    dsel, dcnt = _random_selection(rng, np.full(B, ctx - 1), k)
    dq = _bf16(rng, (B, Qn, Hq, D))
    a = qsa.sparse_attn_decode_fp8kv(dev(dq, "bf16"), dev(rp, "i"), _u8(kc), _u8(vc), ks, vs, dev(dsel, "i"),
                                     dev(dcnt, "i"), dev(ts, "i"))
    b = qsa.sparse_attn_decode_fp8kv(dev(dq, "bf16"), dev(rp, "i"), kp, vp, ks, vs, dev(dsel, "i"), dev(dcnt, "i"),
                                     dev(ts, "i"), page_table=tb, page_tokens=P)
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))


def _quantize(x_bits):
    """bf16 bits -> (E4M3 codes, per-tensor scale = amax / 448), on the host
    with the oracle's (pinned) rounding."""
    x = synth.bf16_to_f32(x_bits)
    amax = float(np.abs(x).max())
    scale = np.float32(amax / 448.0)
    return oracle.fp8_from_float(x.astype(np.float64) / float(scale)), float(scale)


@pytest.mark.parametrize("name", ["chunk-256k", "decode-1m-draft"])
def test_fp8kv_full_size_sampled(gpu, name):
    # the bench workloads' own K/V quantized to FP8 (one scale per tensor),
    # attention on the GPU's selection; sampled rows (decode: every row)
    import torch
    spec = synth.SPECS[name]
    w = synth.make(spec)
    kc, ks = _quantize(w["k_cache"])
    vc, vs = _quantize(w["v_cache"])
    raw = dev(w["raw_keys"], "bf16")
    B, nb = raw.shape[0], spec.n_blocks
    pooled = torch.zeros((B, nb, 128), dtype=torch.bfloat16, device="cuda")
    qsa.pool_index_keys(raw, pooled, 0, nb, spec.theta)
    del raw
    max_nb = int((w["row_pos"].max() + 1) // 4)
    sel, cnt, _ = qsa.score_topk(dev(w["idx_q"], "bf16"), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"), pooled,
                                 max_nb, spec.top_k, spec.theta, want_scores=False)
    g_sel, g_cnt = host(sel), host(cnt)
    if spec.kind == "prefill":
        out, lse = qsa.sparse_attn_prefill_fp8kv(dev(w["q"], "bf16"), dev(w["row_seq"], "i"),
                                                 dev(w["row_pos"], "i"), _u8(kc), _u8(vc), ks, vs, sel, cnt)
        rng = np.random.default_rng(9)
        rows = np.unique(np.concatenate([[0, spec.chunk - 1], rng.choice(spec.chunk, 14, replace=False)]))
        print(f"[fp8kv full-size] {name}: rows {rows.tolist()}", flush=True)
        want, want_lse = oracle.sparse_attn_prefill_fp8kv(w["q"][rows], w["row_seq"][rows], w["row_pos"][rows], kc,
                                                          vc, ks, vs, g_sel[rows], g_cnt[rows])
        assert_close_out(host(out)[rows], want, "bf16")
        np.testing.assert_allclose(host(lse)[rows], want_lse, rtol=1e-5, atol=1e-4)
    else:
        ts = None if w["tail_start"] is None else dev(w["tail_start"], "i")
        out, lse = qsa.sparse_attn_decode_fp8kv(dev(w["q"], "bf16"), dev(w["attn_pos"], "i"), _u8(kc), _u8(vc), ks,
                                                vs, sel, cnt, ts)
        print(f"[fp8kv full-size] {name}: all rows", flush=True)
        want, want_lse = oracle.sparse_attn_decode_fp8kv(w["q"], w["attn_pos"], kc, vc, ks, vs, g_sel, g_cnt,
                                                         w["tail_start"])
        assert_close_out(host(out), want, "bf16")
        np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)
    assert math.isfinite(ks) and math.isfinite(vs)
