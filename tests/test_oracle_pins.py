"""Pins of the CPU oracle against what the pages and the mathematics fix.

No test here compares the oracle with itself.  Each pins one step against a
closed form, an invariant, a textbook/library routine (numpy sort, einsum,
torch SDPA), brute force on tiny inputs, or the constants the pages print
(tests/golden/qsa_page_constants.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "qsa_page_constants.json")))
K4 = GOLD["block_tokens"]["value"]
DIM = GOLD["index_dim"]["value"]
IH = GOLD["index_query_heads"]["value"]


def f32(x):
    return np.asarray(x, np.float32)


# --------------------------------------------------------------------------
# bf16 rounding (storage format of the compressed key and bf16 operands)
# --------------------------------------------------------------------------

def test_bf16_known_values():
    cases = [
        (1.0, 0x3F80),
        (-2.0, 0xC000),
        (1.0 + 2.0 ** -8, 0x3F80),                 # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),    # just above the tie
        (2.0 ** -133, 0x0001),                     # smallest subnormal
        (2.0 ** -134, 0x0000),                     # tie between 0 and 2^-133 -> even (0)
        (1.5 * 2.0 ** -133, 0x0002),               # tie between 1 and 2 steps -> even
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),    # largest finite
        (2.0 ** 128, 0x7F80),                      # overflow -> inf
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    for x, bits in cases:
        assert int(oracle.bf16_from_float([x])[0]) == bits, (x, hex(bits))


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),  # subnormals
                        (rng.standard_normal(1000) * 1e30).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_float(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)
    back = oracle.bf16_to_float(got)
    np.testing.assert_array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16)
                                  .to(torch.float64).numpy())


# --------------------------------------------------------------------------
# RoPE (post-pool key rotation, query rotation)
# --------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal(DIM)
    np.testing.assert_array_equal(oracle.rope(x, 0, 1e7), x)


def test_rope_theta_one_turns_every_pair_by_pos_radians():
    # theta = 1 -> every frequency is 1: pair (j, j+64) turns by exactly `pos`.
    for j in (0, 17, 63):
        for pos in (1, 5, 1000):
            e = np.zeros(DIM)
            e[j] = 1.0
            out = oracle.rope(e, pos, 1.0)
            want = np.zeros(DIM)
            want[j], want[j + 64] = math.cos(pos), math.sin(pos)
            np.testing.assert_allclose(out, want, atol=1e-12)
            e = np.zeros(DIM)
            e[j + 64] = 1.0
            out = oracle.rope(e, pos, 1.0)
            want = np.zeros(DIM)
            want[j], want[j + 64] = -math.sin(pos), math.cos(pos)
            np.testing.assert_allclose(out, want, atol=1e-12)


def test_rope_frequency_schedule():
    # theta = 2^64 -> theta^(-j/64) = 2^-j: at pos 1 pair j turns by 2^-j rad.
    for j in range(0, 64, 7):
        e = np.zeros(DIM)
        e[j] = 1.0
        out = oracle.rope(e, 1, 2.0 ** 64)
        assert math.isclose(math.atan2(out[j + 64], out[j]), 2.0 ** -j, rel_tol=1e-12)
    # theta = 1e8, pair 32 -> frequency theta^-1/2 = 1e-4: pos 10,000 turns by 1 rad.
    e = np.zeros(DIM)
    e[32] = 1.0
    out = oracle.rope(e, 10_000, 1e8)
    assert math.isclose(math.atan2(out[96], out[32]), 1.0, rel_tol=1e-12)


def test_rope_norm_composition_relative_shift():
    rng = np.random.default_rng(2)
    x, y = rng.standard_normal(DIM), rng.standard_normal(DIM)
    th = 1e7
    for p in (3, 4096, 1_048_575):
        assert math.isclose(np.linalg.norm(oracle.rope(x, p, th)), np.linalg.norm(x), rel_tol=1e-13)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, 1234, th), 777, th),
                               oracle.rope(x, 2011, th), atol=1e-11)
    # <R(p)x, R(p')y> depends only on p - p'
    a = oracle.rope(x, 1000, th) @ oracle.rope(y, 200, th)
    b = oracle.rope(x, 1000 + 4 * 12345, th) @ oracle.rope(y, 200 + 4 * 12345, th)
    assert math.isclose(a, b, rel_tol=1e-9, abs_tol=1e-9)


# --------------------------------------------------------------------------
# a1-a3: block mean in FP32, then RoPE at the block's first position
# --------------------------------------------------------------------------

def _raw(L, fill=None, B=1):
    r = np.zeros((B, L, DIM), np.float32)
    if fill is not None:
        r[:] = fill
    return r


def test_pool_hand_example():
    # Block 1 = tokens 4..7.  dim 0 holds 2,4,6,8 (mean 5), dim 1 holds 1 (mean 1).
    raw = _raw(8)
    raw[0, 4:8, 0] = [2, 4, 6, 8]
    raw[0, 4:8, 1] = 1
    th = 1e7
    out = oracle.pool(raw, 0, 2, th)[0, 1].astype(np.float64)
    want = np.zeros(DIM)
    want[0], want[64] = 5 * math.cos(4.0), 5 * math.sin(4.0)      # pair 0: frequency 1
    w1 = 4.0 * 10.0 ** (-7.0 / 64.0)                               # pair 1: 4 * theta^(-1/64)
    want[1], want[65] = math.cos(w1), math.sin(w1)
    np.testing.assert_allclose(out, want, rtol=1e-6, atol=1e-7)
    # block 0 is all zero
    np.testing.assert_array_equal(oracle.pool(raw, 0, 2, th)[0, 0], 0)


def test_pool_mean_is_fp32_in_token_order():
    # ((1 + 2^-24) + 2^-24) + 0 = 1 in FP32, so the mean is exactly 0.25;
    # an exact (fp64) mean would be 0.25 + 2^-25, which FP32 can hold.
    raw = _raw(4)
    raw[0, :, 0] = [1.0, 2.0 ** -24, 2.0 ** -24, 0.0]
    out = oracle.pool(raw, 0, 1, 1e7, flags=oracle.FLAG_NO_ROPE)
    assert out[0, 0, 0] == np.float32(0.25)


def test_pool_integer_means_exact_and_linear():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, size=(2, 64, DIM)).astype(np.float32)
    y = rng.integers(-8, 9, size=(2, 64, DIM)).astype(np.float32)
    flags = oracle.FLAG_NO_ROPE
    px, py = oracle.pool(x, 0, 16, 1e7, flags), oracle.pool(y, 0, 16, 1e7, flags)
    np.testing.assert_array_equal(px, x.reshape(2, 16, 4, DIM).sum(2) / 4)  # exact small integers
    np.testing.assert_array_equal(oracle.pool(2 * x - 0.5 * y, 0, 16, 1e7, flags), 2 * px - 0.5 * py)
    # with RoPE the map is still linear (a rotation), up to FP32 rounding
    pr = oracle.pool(2 * x - 0.5 * y, 0, 16, 1e7)
    lin = 2 * oracle.pool(x, 0, 16, 1e7) - 0.5 * oracle.pool(y, 0, 16, 1e7)
    np.testing.assert_allclose(pr, lin, rtol=1e-5, atol=1e-4)


def test_pool_constant_block_is_rotated_key():
    rng = np.random.default_rng(4)
    k = rng.standard_normal(DIM).astype(np.float32)
    raw = _raw(40)
    raw[0, 4 * 7:4 * 8] = k
    out = oracle.pool(raw, 7, 8, 1e7)[0, 7]
    np.testing.assert_allclose(out, oracle.rope(k.astype(np.float64), 28, 1e7), rtol=1e-6, atol=1e-6)


def test_pool_rotates_after_pooling_at_first_token():
    # Four different keys with energy in the fast pairs: rotating each token at
    # its own position before averaging, or rotating the mean at 4b+3, gives a
    # clearly different compressed key ([ARCH] item 2 says after pooling).
    rng = np.random.default_rng(5)
    b = 11
    keys = rng.standard_normal((4, DIM))
    raw = _raw(4 * (b + 1))
    raw[0, 4 * b:4 * b + 4] = keys.astype(np.float32)
    got = oracle.pool(raw, b, b + 1, 1e7)[0, b].astype(np.float64)
    mean = raw[0, 4 * b:4 * b + 4].astype(np.float64).mean(0)
    post = oracle.rope(mean, 4 * b, 1e7)
    pre = np.mean([oracle.rope(raw[0, 4 * b + i].astype(np.float64), 4 * b + i, 1e7)
                   for i in range(4)], axis=0)
    late = oracle.rope(mean, 4 * b + 3, 1e7)
    np.testing.assert_allclose(got, post, rtol=1e-5, atol=1e-5)
    assert np.abs(got - pre).max() > 1e-2
    assert np.abs(got - late).max() > 1e-2


def _stream_append(raw, slots, theta, flags=0, starts=None):
    """Feed each request's tokens one decode step at a time through the ring."""
    B, L, _ = raw.shape
    ring = np.zeros((B, 4, DIM), raw.dtype)
    sentinel = synth.bf16_bits(np.float32(-7.0)) if raw.dtype == np.uint16 else np.float32(-7.0)
    comp = np.full((int(slots.max()) // 4 + 1, DIM), sentinel, raw.dtype)
    starts = np.zeros(B, np.int64) if starts is None else starts
    for step in range(L):
        t = np.minimum(starts + step, L - 1)  # requests that finished repeat their last token harmlessly
        live = starts + step < L
        if not live.any():
            break
        r = np.nonzero(live)[0]
        oracle.pool_append(raw[r, t[r]], t[r].astype(np.int32), slots[r, t[r]], ring_sub := ring[r].copy(), comp,
                           theta, flags)
        ring[r] = ring_sub
    return ring, comp, sentinel


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, oracle.FLAG_POOL_RMSNORM])
def test_pool_append_stream_equals_whole_sequence_pool(dtype, flags):
    # [SGL]: raw keys of the unfinished block live in a 4-slot ring; the
    # compressed key of a finished block sits at page-aligned full_slot / 4.
    # Streaming the tokens through the ring must give, slot for slot, the
    # (separately pinned) pooling of the whole sequence.
    rng = np.random.default_rng(21)
    B, L = 3, 47                                   # 11 complete blocks + 3 tokens
    x = rng.standard_normal((B, L, DIM)).astype(np.float32)
    raw = synth.bf16_bits(x) if dtype == "bf16" else x
    slots = synth.paged_slots(rng, B, L, page_tokens=16)
    ring, comp, sentinel = _stream_append(raw, slots, 1e7, flags)
    whole = oracle.pool(raw, 0, L // 4, 1e7, flags=flags)
    for r in range(B):
        for b in range(L // 4):
            np.testing.assert_array_equal(comp[slots[r, 4 * b] // 4], whole[r, b])
        # the unfinished block has no compressed key yet; the ring holds its tokens
        assert (comp[slots[r, 4 * (L // 4)] // 4] == sentinel).all()
        for t in range(4 * (L // 4), L):
            np.testing.assert_array_equal(ring[r, t % 4], raw[r, t])


def test_pool_append_constant_keys_give_rotated_key():
    # every token of a request carries the same key k: each finished block is
    # R(4b) k (closed form), whichever page it landed in
    rng = np.random.default_rng(22)
    k = rng.standard_normal(DIM).astype(np.float32)
    raw = np.broadcast_to(k, (2, 24, DIM)).copy()
    slots = synth.paged_slots(rng, 2, 24, page_tokens=8)
    _, comp, _ = _stream_append(raw, slots, 1e7, starts=np.array([0, 0]))
    for r in range(2):
        for b in range(6):
            np.testing.assert_allclose(comp[slots[r, 4 * b] // 4], oracle.rope(k.astype(np.float64), 4 * b, 1e7),
                                       rtol=1e-6, atol=1e-6)


def test_pool_bf16_storage_is_rounded_fp32_result():
    rng = np.random.default_rng(6)
    raw32 = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((1, 256, DIM)).astype(np.float32)))
    p32 = oracle.pool(raw32, 0, 64, 1e7)
    pbf = oracle.pool(synth.bf16_bits(raw32), 0, 64, 1e7)
    want = torch.from_numpy(p32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    diff = np.abs(pbf.astype(np.int32) - want.astype(np.int32))
    assert diff.max() <= 1                      # double rounding via fp32 may move one ulp
    assert (diff == 0).mean() > 0.999


def test_pool_rmsnorm_flag_gives_unit_rms():
    rng = np.random.default_rng(8)
    raw = rng.standard_normal((1, 64, DIM)).astype(np.float32) * 3
    out = oracle.pool(raw, 0, 16, 1e7, flags=oracle.FLAG_NO_ROPE | oracle.FLAG_POOL_RMSNORM)
    rms = np.sqrt((out.astype(np.float64) ** 2).mean(-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-5)


# --------------------------------------------------------------------------
# a4-a6: block score and top-k selection
# --------------------------------------------------------------------------

def _rotated_queries(q, pos, theta, flags, dtype):
    out = np.zeros(q.shape, np.float64)
    for r in range(q.shape[0]):
        for h in range(IH):
            v = q[r, h].astype(np.float64) if dtype == "f32" else synth.bf16_to_f32(q[r, h]).astype(np.float64)
            if not flags & oracle.FLAG_NO_ROPE:
                v = oracle.rope(v, int(pos[r]), theta)
            out[r, h] = v.astype(np.float32) if dtype == "f32" else oracle.bf16_to_float(oracle.bf16_from_float(v))
    return out


@pytest.mark.parametrize("dtype,flags", [("f32", 0), ("bf16", 0), ("bf16", oracle.FLAG_NO_ROPE)])
def test_score_equals_einsum_brute_force(dtype, flags):
    rng = np.random.default_rng(9)
    B, NB, R, th = 2, 24, 7, 1e7
    pooled = rng.standard_normal((B, NB, DIM)).astype(np.float32)
    q = rng.standard_normal((R, IH, DIM)).astype(np.float32)
    if dtype == "bf16":
        pooled, q = synth.bf16_bits(pooled), synth.bf16_bits(q)
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    sel, cnt, sc, raw = oracle.score_topk(q, seq, pos, pooled, 64, th, flags, want_raw=True)
    qr = _rotated_queries(q, pos, th, flags, dtype)
    kv = pooled.astype(np.float64) if dtype == "f32" else synth.bf16_to_f32(pooled).astype(np.float64)
    dots = np.einsum("rhd,rbd->rhb", qr, kv[seq])
    want = np.maximum(dots, 0).sum(1)
    for r in range(R):
        nc = (int(pos[r]) + 1) // 4
        np.testing.assert_allclose(raw[r, :nc], want[r, :nc], rtol=1e-12, atol=1e-12)
        assert np.isnan(raw[r, nc:]).all()  # invisible blocks are never scored
        assert cnt[r] == nc and list(sel[r, :nc]) == list(range(nc))
        np.testing.assert_allclose(sc[r, :nc], want[r, :nc] / math.sqrt(128), rtol=1e-6)


def test_score_relu_per_head():
    # integer vectors, no rotation: head 0 points against the key, heads 1..3 along it
    k = np.zeros(DIM, np.float32)
    k[:5] = [1, 2, 3, 0, -1]
    pooled = np.stack([k, 2 * k])[None]          # [1][2][128]
    q = np.stack([-k, k, k, k])[None]            # [1][4][128]
    sel, cnt, sc, raw = oracle.score_topk(q, [0], [7], pooled, 4, 1e7, oracle.FLAG_NO_ROPE, want_raw=True)
    assert list(raw[0]) == [3 * 15.0, 6 * 15.0]    # |k|^2 = 15; the negative head adds 0
    assert sc[0, 1] == np.float32(90 / math.sqrt(128))


def test_visibility_only_complete_blocks():
    # block b is visible to the row at t iff 4b+3 <= t; a huge invisible block is ignored
    pooled = np.ones((1, 8, DIM), np.float32)
    pooled[0, 2] = 100.0
    q = np.ones((1, IH, DIM), np.float32)
    for t, want in [(0, 0), (2, 0), (3, 1), (6, 1), (7, 2), (10, 2), (11, 3)]:
        sel, cnt, _, _ = oracle.score_topk(q, [0], [t], pooled, 1 if want else 4, 1e7, oracle.FLAG_NO_ROPE)
        assert cnt[0] == min(want, sel.shape[1])
        if t < 11:
            assert 2 not in sel[0]


def _lexsort_topk(raw_row, k):
    order = np.lexsort((np.arange(raw_row.size), -raw_row))  # score desc, then index asc
    return np.sort(order[:k])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_selection_equals_full_sort(seed):
    rng = np.random.default_rng(seed)
    NB, R, k = 80, 9, 13
    pooled = rng.standard_normal((1, NB, DIM)).astype(np.float32)
    q = rng.standard_normal((R, IH, DIM)).astype(np.float32)
    pos = rng.integers(4 * k, 4 * NB, R).astype(np.int32)
    sel, cnt, _, raw = oracle.score_topk(q, np.zeros(R, np.int32), pos, pooled, k, 1e7, 0, want_raw=True)
    qr = _rotated_queries(q, pos, 1e7, 0, "f32")
    want_raw = np.maximum(np.einsum("rhd,bd->rhb", qr, pooled[0].astype(np.float64)), 0).sum(1)
    for r in range(R):
        nc = (int(pos[r]) + 1) // 4
        assert cnt[r] == k
        np.testing.assert_array_equal(sel[r], _lexsort_topk(want_raw[r, :nc], k))


def test_selection_ties_go_to_lower_block_index():
    # integer keys with many exact repeats; no rotation -> exact integer scores
    rng = np.random.default_rng(11)
    NB, k = 60, 10
    base = rng.integers(-2, 3, size=(6, DIM)).astype(np.float32)
    pooled = base[rng.integers(0, 6, NB)][None]          # only 6 distinct keys
    q = rng.integers(-2, 3, size=(3, IH, DIM)).astype(np.float32)
    pos = np.array([4 * NB - 1, 4 * 40 + 2, 4 * 25], np.int32)
    sel, cnt, _, raw = oracle.score_topk(q, np.zeros(3, np.int32), pos, pooled, k, 1e7,
                                         oracle.FLAG_NO_ROPE, want_raw=True)
    for r in range(3):
        nc = (int(pos[r]) + 1) // 4
        exact = np.array([sum(max(0, int(np.dot(q[r, h].astype(np.int64), pooled[0, b].astype(np.int64))))
                              for h in range(IH)) for b in range(nc)])
        np.testing.assert_array_equal(raw[r, :nc], exact)
        np.testing.assert_array_equal(sel[r], _lexsort_topk(exact.astype(np.float64), k))
        chosen = set(sel[r].tolist())
        worst = min((exact[b], -b) for b in chosen)
        best_out = max(((exact[b], -b) for b in range(nc) if b not in chosen), default=None)
        assert best_out is None or worst > best_out


def test_fewer_visible_than_k_keeps_all_and_pads():
    pooled = np.random.default_rng(12).standard_normal((1, 50, DIM)).astype(np.float32)
    q = np.random.default_rng(13).standard_normal((2, IH, DIM)).astype(np.float32)
    sel, cnt, sc, _ = oracle.score_topk(q, [0, 0], [4 * 7 + 1, 4 * 50 - 1], pooled, 64, 1e7)
    assert cnt.tolist() == [7, 50]
    assert sel[0, :7].tolist() == list(range(7)) and (sel[0, 7:] == -1).all()
    assert sel[1, :50].tolist() == list(range(50)) and (sel[1, 50:] == -1).all()


def test_planted_needles_recovered_decode():
    spec = synth.scaled("decode-128k", batch=2, ctx=16384)
    w = synth.make(spec)
    pooled = oracle.pool(w["raw_keys"], 0, spec.n_blocks, spec.theta)
    sel, cnt, _, _ = oracle.score_topk(w["idx_q"], w["row_seq"], w["row_pos"], pooled, spec.top_k,
                                       spec.theta)
    for s in range(spec.batch):
        assert cnt[s] == spec.top_k
        assert set(w["planted"][s].tolist()) <= set(sel[s].tolist())


def test_planted_set_is_the_selection_draft():
    spec = synth.scaled("decode-1m-draft", batch=2, ctx=16384)
    w = synth.make(spec)
    pooled = oracle.pool(w["raw_keys"], 0, spec.n_blocks, spec.theta)
    sel, cnt, _, raw = oracle.score_topk(w["idx_q"], w["row_seq"], w["row_pos"], pooled, spec.top_k,
                                         spec.theta, want_raw=True)
    for s in range(spec.batch):
        np.testing.assert_array_equal(sel[s], w["planted"][s])
        others = np.setdiff1d(np.arange(spec.n_blocks), w["planted"][s])
        assert raw[s, w["planted"][s]].min() > 1.25 * raw[s, others].max()


def test_planted_runs_fill_the_selection_chunk():
    spec = synth.scaled("chunk-256k", ctx=8192, chunk=64)
    w = synth.make(spec)
    pooled = oracle.pool(w["raw_keys"], 0, spec.n_blocks, spec.theta)
    rows = np.arange(0, 64, 9)
    sel, cnt, _, _ = oracle.score_topk(w["idx_q"][rows], w["row_seq"][rows], w["row_pos"][rows], pooled,
                                       spec.top_k, spec.theta)
    planted = set(w["planted"][0].tolist())
    for r in range(len(rows)):
        assert cnt[r] == 512 and set(sel[r].tolist()) <= planted


# --------------------------------------------------------------------------
# a7-a9: expansion, tail, sparse GQA attention
# --------------------------------------------------------------------------

def _sdpa_dense_causal(q, k, v, scale):
    """torch SDPA (is_causal) in fp64 on the CPU; q [L][Hq][D], k/v [L][Hkv][D]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], is_causal=True,
                                                         scale=scale)[0]
    logits = (qt @ kt.transpose(1, 2)) * scale
    mask = torch.triu(torch.ones(q.shape[0], q.shape[0], dtype=torch.bool), 1)
    lse = torch.logsumexp(logits.masked_fill(mask, -math.inf), -1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 1, 32), (4, 2, 32), (6, 3, 32), (24, 2, 256)])
def test_topk_at_least_visible_equals_dense_causal(Hq, Hkv, D):
    # every row keeps all its visible blocks (top_k >= nc) -> QSA == dense causal attention
    rng = np.random.default_rng(20 + Hq + Hkv)
    L, k = 70, 32
    pooled = rng.standard_normal((1, L // 4, DIM)).astype(np.float32)
    iq = rng.standard_normal((L, IH, DIM)).astype(np.float32)
    pos = np.arange(L, dtype=np.int32)
    seq = np.zeros(L, np.int32)
    sel, cnt, _, _ = oracle.score_topk(iq, seq, pos, pooled, k, 1e7)
    q = rng.standard_normal((L, Hq, D)).astype(np.float32)
    kc = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    out, lse = oracle.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt, 1 / math.sqrt(D))
    want, want_lse = _sdpa_dense_causal(q, kc[0], vc[0], 1 / math.sqrt(D))
    np.testing.assert_allclose(out, want, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(lse, want_lse, rtol=1e-6, atol=1e-6)


def test_attention_constant_v_single_position_permutation():
    rng = np.random.default_rng(30)
    L, D, Hq, Hkv = 64, 16, 2, 1
    q = rng.standard_normal((3, Hq, D)).astype(np.float32)
    kc = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    vc = np.broadcast_to(rng.standard_normal(D).astype(np.float32), (1, L, Hkv, D)).copy()
    sel = np.array([[1, 4, 9, 2], [3, 0, -1, -1], [-1, -1, -1, -1]], np.int32)
    cnt = np.array([4, 2, 0], np.int32)
    pos = np.array([63, 13, 0], np.int32)
    out, _ = oracle.sparse_attn_prefill(q, np.zeros(3, np.int32), pos, kc, vc, sel, cnt)
    np.testing.assert_allclose(out, np.broadcast_to(vc[0, 0, 0], out.shape), rtol=1e-6)
    # a row at t = 0 with no complete block attends only position 0
    vc2 = rng.standard_normal((1, L, Hkv, D)).astype(np.float32)
    out2, lse2 = oracle.sparse_attn_prefill(q, np.zeros(3, np.int32), pos, kc, vc2, sel, cnt)
    np.testing.assert_array_equal(out2[2], np.broadcast_to(vc2[0, 0, 0], (Hq, D)))
    np.testing.assert_allclose(lse2[2], (q[2] @ kc[0, 0, 0]) / math.sqrt(D), rtol=1e-6)
    # the order of the kept blocks does not matter
    perm = sel.copy()
    perm[0, :4] = [9, 2, 1, 4]
    out3, _ = oracle.sparse_attn_prefill(q, np.zeros(3, np.int32), pos, kc, vc2, perm, cnt)
    np.testing.assert_allclose(out3, out2, rtol=1e-6, atol=1e-7)


def _indicator_counts(n_blocks_ctx, t, top_k, sel=None, cnt=None, tail_start=None, decode=False):
    """Uniform attention (q = 0) over V = [1, is_tail, is_selected_block_token]:
    out = [1, n_tail/n, n_sel/n] reveals how many positions were attended."""
    L = max(t + 1, 4 * n_blocks_ctx)
    D = 8
    kc = np.zeros((1, L, 1, D), np.float32)
    vc = np.zeros((1, L, 1, D), np.float32)
    vc[0, :, 0, 0] = 1
    ts = tail_start if tail_start is not None else 4 * ((t + 1) // 4)
    vc[0, ts:t + 1, 0, 1] = 1
    if sel is None:
        sel = np.arange(top_k, dtype=np.int32)[None]
        cnt = np.array([top_k], np.int32)
    for b in sel[0, :cnt[0]]:
        vc[0, 4 * b:4 * b + 4, 0, 2] = 1
    if decode:
        q = np.zeros((1, 1, 1, D), np.float32)
        out, _ = oracle.sparse_attn_decode(q, np.array([[t]], np.int32), kc, vc, sel, cnt,
                                           None if tail_start is None else np.array([tail_start], np.int32))
        out = out[0, 0, 0]
    else:
        q = np.zeros((1, 1, D), np.float32)
        out, _ = oracle.sparse_attn_prefill(q, [0], [t], kc, vc, sel, cnt)
        out = out[0, 0]
    n = 1.0 / out[1] * (t + 1 - ts) if t + 1 > ts else None
    return out, n


def test_position_budget_from_the_pages():
    top = GOLD["top_blocks"]["value"]
    sel_tok = GOLD["selected_tokens"]["value"]
    mx = GOLD["max_positions"]["value"]
    assert top * K4 == sel_tok
    for tail in range(GOLD["tail_tokens_min"]["value"], GOLD["tail_tokens_max"]["value"] + 1):
        t = 4 * 600 + tail - 1                       # nc = 600 > 512 complete blocks; tail tokens
        out, _ = _indicator_counts(600, t, top)
        assert out[0] == pytest.approx(1.0, rel=1e-6)
        n_total = sel_tok + tail
        assert out[1] == pytest.approx(tail / n_total, rel=1e-6, abs=1e-9)   # tail always attended
        assert out[2] == pytest.approx(sel_tok / n_total, rel=1e-6)          # 512 blocks -> 2048 tokens
        assert n_total <= mx
    assert sel_tok + GOLD["tail_tokens_max"]["value"] == mx


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_index_cache_cut_from_the_pages(dtype):
    # "Day-0 Support in SGLang", section "Qwen Sparse Attention": one compressed
    # index key per four tokens plus a four-slot per-request ring of raw keys,
    # instead of retaining the raw index keys of the whole context, cuts the
    # index cache by 80%.  Reading: the cache it replaces held every token's
    # raw key next to the compressed keys (raw + raw/4 per token); the cut of
    # keeping only compressed keys and the ring is then 1 - (L/4 + 4)/(5L/4),
    # which tends to 80% from below.  The per-token bytes come from running
    # the incremental pooling over a stream: it writes one compressed key per
    # four token slots and touches only the ring besides.
    rng = np.random.default_rng(12)
    B, L = 2, 64
    keys = rng.standard_normal((B, L, DIM)).astype(np.float32)
    keys = synth.bf16_bits(keys) if dtype == "bf16" else keys
    esz = keys.dtype.itemsize
    ring = np.zeros((B, 4, DIM), keys.dtype)
    comp = np.zeros((B * L // 4, DIM), keys.dtype)
    sentinel = comp.copy()
    for t in range(L):
        slots = np.arange(B, dtype=np.int64) * L + t   # contiguous pages: full_slot = s*L + t
        oracle.pool_append(keys[:, t].copy(), np.full(B, t, np.int32), slots, ring, comp, 1.0e7)
    written = np.any(comp != sentinel, axis=1).sum()
    assert written == B * L // 4                           # one compressed key per 4 tokens
    comp_bytes_per_token = written * DIM * esz / (B * L)
    raw_bytes_per_token = DIM * esz
    ring_bytes_per_request = ring[0].nbytes
    want = GOLD["index_cache_cut_percent"]["value"] / 100.0
    for ctx in (262_144, 1_048_576):
        before = ctx * (raw_bytes_per_token + comp_bytes_per_token)
        after = ctx * comp_bytes_per_token + ring_bytes_per_request
        cut = 1.0 - after / before
        assert cut <= want and want - cut < 2e-5, (ctx, cut)


def test_decode_shared_selection_with_drafted_positions():
    # IndexShare: rows after the anchor reuse its selection and add [tail_start, t]
    rng = np.random.default_rng(40)
    L, D, Hq, Hkv, k = 4 * 40, 16, 4, 2, 8
    Qn = 3
    kc = rng.standard_normal((2, L + Qn, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((2, L + Qn, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((2, Qn, Hq, D)).astype(np.float32)
    sel = np.sort(rng.choice(40, size=(2, k), replace=True), axis=1).astype(np.int32)
    sel = np.stack([np.sort(rng.choice(40, k, replace=False)) for _ in range(2)]).astype(np.int32)
    cnt = np.array([k, k - 2], np.int32)
    sel[1, k - 2:] = -1
    rp = (L + np.tile(np.arange(Qn), (2, 1))).astype(np.int32)
    ts = np.array([L, L], np.int32)
    out, lse = oracle.sparse_attn_decode(q, rp, kc, vc, sel, cnt, ts)
    for s in range(2):
        for j in range(Qn):
            P = [4 * b + i for b in sel[s, :cnt[s]] for i in range(4)] + list(range(L, L + j + 1))
            for h in range(Hq):
                g = h // (Hq // Hkv)
                qt = torch.from_numpy(q[s, j, h].astype(np.float64))[None, None, None]
                kt = torch.from_numpy(kc[s, P, g].astype(np.float64))[None, None]
                vt = torch.from_numpy(vc[s, P, g].astype(np.float64))[None, None]
                o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1 / math.sqrt(D))
                np.testing.assert_allclose(out[s, j, h], o[0, 0, 0].numpy(), rtol=1e-5, atol=1e-6)
                want_lse = torch.logsumexp((kt[0, 0] @ qt[0, 0, 0]) / math.sqrt(D), 0).item()
                assert lse[s, j, h] == pytest.approx(want_lse, rel=1e-6)


def test_attention_bf16_output_is_rounded():
    rng = np.random.default_rng(50)
    L, D = 32, 16
    q = rng.standard_normal((4, 2, D)).astype(np.float32)
    kc = rng.standard_normal((1, L, 1, D)).astype(np.float32)
    vc = rng.standard_normal((1, L, 1, D)).astype(np.float32)
    qb, kb, vb = synth.bf16_bits(q), synth.bf16_bits(kc), synth.bf16_bits(vc)
    sel = np.tile(np.arange(4, dtype=np.int32), (4, 1))
    cnt = np.array([0, 1, 2, 4], np.int32)
    pos = np.array([2, 5, 10, 19], np.int32)
    out32, _ = oracle.sparse_attn_prefill(synth.bf16_to_f32(qb), [0] * 4, pos, synth.bf16_to_f32(kb),
                                          synth.bf16_to_f32(vb), sel, cnt)
    outb, _ = oracle.sparse_attn_prefill(qb, [0] * 4, pos, kb, vb, sel, cnt)
    want = torch.from_numpy(out32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.abs(outb.astype(np.int32) - want.astype(np.int32)).max() <= 1


# --------------------------------------------------------------------------
# FP8 E4M3 index keys ("Qwen3.8-Flash-Next, Layer by Layer", "Serving it":
# the indexer's keys stored in FP8)
# --------------------------------------------------------------------------

def _e4m3_table():
    """Every finite E4M3 value, decoded from the bit fields of the OCP format
    (sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal; 0x7f / 0xff are NaN) -- written from the format, not from the
    oracle's rounding."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_fp8_known_values():
    t = oracle.fp8_to_float(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x40, 0xB8, 0x00, 0x80], np.uint8))
    assert list(t) == [448.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 2.0, -1.0, 0.0, -0.0]
    assert np.isnan(oracle.fp8_to_float(np.array([0x7F, 0xFF], np.uint8))).all()
    table = _e4m3_table()
    assert len(table) == 254 and max(table.values()) == 448.0


def test_fp8_every_code_round_trips():
    table = _e4m3_table()
    codes = np.array(sorted(table), np.uint8)
    np.testing.assert_array_equal(oracle.fp8_to_float(codes), np.array([table[c] for c in codes]))
    np.testing.assert_array_equal(oracle.fp8_from_float(oracle.fp8_to_float(codes)), codes)


def test_fp8_rounding_is_nearest_even_by_brute_force():
    # against a scan of the whole value table: nearest value, ties to the
    # code with an even mantissa (lsb 0)
    table = _e4m3_table()
    pos = sorted((v, c) for c, v in table.items() if c < 0x80)
    rng = np.random.default_rng(41)
    mags = 2.0 ** rng.uniform(-12, np.log2(464.0), 3000)
    mids = [0.5 * (pos[i][0] + pos[i + 1][0]) for i in range(len(pos) - 1)]
    xs = np.concatenate([mags, -mags[:500], np.array(mids), -np.array(mids[:40])])
    want = []
    for x in xs:
        best = min(pos, key=lambda vc: (abs(abs(x) - vc[0]), vc[1] & 1))
        want.append(best[1] | (0x80 if x < 0 and best[0] != 0.0 else 0) if best[0] != 0.0 else (0x80 if x < 0 else 0))
    np.testing.assert_array_equal(oracle.fp8_from_float(xs), np.array(want, np.uint8))
    # beyond 464 there is no finite neighbour: NaN
    assert list(oracle.fp8_from_float([470.0, -1e6])) == [0x7F, 0xFF]


def test_pool_fp8_max_maps_to_448_and_error_within_half_step():
    rng = np.random.default_rng(43)
    raw = synth.bf16_bits(rng.standard_normal((2, 64, DIM)).astype(np.float32) * 3)
    codes, scales = oracle.pool_fp8(raw, 0, 16, 1e7)
    ref = oracle.pool(synth.bf16_to_f32(raw).astype(np.float32), 0, 16, 1e7)   # the FP32-rounded rotated keys
    table = _e4m3_table()
    vals = oracle.fp8_to_float(codes)
    amax = np.abs(ref).max(-1)
    np.testing.assert_array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    # the largest magnitude of each key is the largest code
    arg = np.abs(ref).argmax(-1)
    got = np.take_along_axis(np.abs(vals), arg[..., None], -1)[..., 0]
    assert (got == 448.0).all()
    # every element within half an E4M3 step of the scaled value (step at the
    # scaled magnitude: 2^-9 below 2^-6, else 2^(floor(log2 |x|) - 3))
    x = ref.astype(np.float64) * (448.0 / amax[..., None].astype(np.float64))
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6)))
    step = np.where(np.abs(x) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
    assert (np.abs(vals - x) <= 0.5 * step * (1 + 1e-6)).all()
    assert set(np.unique(codes)) <= set(table)


def test_pool_fp8_power_of_two_scaling_moves_only_the_scale():
    rng = np.random.default_rng(44)
    raw = rng.standard_normal((1, 32, DIM)).astype(np.float32)
    c1, s1 = oracle.pool_fp8(raw, 0, 8, 1e7, oracle.FLAG_NO_ROPE)
    c2, s2 = oracle.pool_fp8(raw * np.float32(8), 0, 8, 1e7, oracle.FLAG_NO_ROPE)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s2, s1 * np.float32(8))


def test_score_fp8_equals_exact_keys_of_the_other_path():
    # keys whose values are exact E4M3 codes with scale 1 (and then 1/8): the
    # FP8 score is the score of the same keys stored exactly (the bf16 path,
    # pinned above against einsum), and the selection does not change
    rng = np.random.default_rng(45)
    B, NB, R, k = 2, 300, 9, 40
    kv = rng.integers(-4, 5, size=(B, NB, DIM)).astype(np.float32)
    kv[..., 0] = 448.0                                  # every key's amax: scale exactly 1
    codes = oracle.fp8_from_float(kv)
    scales = np.ones((B, NB), np.float32)
    q = synth.bf16_bits(rng.integers(-3, 4, size=(R, IH, DIM)).astype(np.float32) / 64)
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    a = oracle.score_topk_fp8(q, seq, pos, codes, scales, k, 1e7, oracle.FLAG_NO_ROPE, want_raw=True)
    b = oracle.score_topk(q, seq, pos, synth.bf16_bits(kv), k, 1e7, oracle.FLAG_NO_ROPE, want_raw=True)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)
    np.testing.assert_array_equal(a[3], b[3])
    c = oracle.score_topk_fp8(q, seq, pos, codes, scales / np.float32(8), k, 1e7, oracle.FLAG_NO_ROPE, want_raw=True)
    np.testing.assert_array_equal(c[0], a[0])
    np.testing.assert_array_equal(c[3], a[3] / 8)


# ---------------------------------------------------------------------------
# FP8 K/V cache ("Qwen3.8-Flash-Next, Layer by Layer", "Serving it"): E4M3
# codes with one scale for K and one for V; value = scale * E4M3(code)
# ---------------------------------------------------------------------------

def _fp8kv_case(seed, L=4 * 60 + 2, R=9, Hq=6, Hkv=2, D=32, k=16):
    rng = np.random.default_rng(seed)
    pos = np.sort(rng.choice(np.arange(4 * k, L), R, replace=False)).astype(np.int32)
    pos[0] = 2                                                   # no complete block: the tail alone
    sel = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r, t in enumerate(pos):
        n = min(k, (int(t) + 1) // 4)
        sel[r, :n] = np.sort(rng.choice((int(t) + 1) // 4, n, replace=False))
        cnt[r] = n
    q = rng.standard_normal((R, Hq, D)).astype(np.float32)
    kint = rng.integers(-8, 9, size=(1, L, Hkv, D)).astype(np.float32)   # exact E4M3 values
    vint = rng.integers(-8, 9, size=(1, L, Hkv, D)).astype(np.float32)
    return q, np.zeros(R, np.int32), pos, kint, vint, sel, cnt


def test_fp8kv_attention_equals_plain_attention_on_exact_values():
    # integer codes times a power-of-two scale are exact fp32 values: the FP8
    # cache and the fp32 cache of the same values give the same result
    q, seq, pos, kint, vint, sel, cnt = _fp8kv_case(90)
    kc, vc = oracle.fp8_from_float(kint), oracle.fp8_from_float(vint)
    np.testing.assert_array_equal(oracle.fp8_to_float(kc), kint)
    out, lse = oracle.sparse_attn_prefill_fp8kv(q, seq, pos, kc, vc, 0.25, 0.5, sel, cnt)
    want, want_lse = oracle.sparse_attn_prefill(q, seq, pos, kint * 0.25, vint * 0.5, sel, cnt)
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(lse, want_lse)
    qd = q.reshape(3, 3, 6, 32)
    rp = np.array([[200, 201, 202]] * 3, np.int32)
    ts = np.array([200, 200, 200], np.int32)
    out, lse = oracle.sparse_attn_decode_fp8kv(qd, rp, np.repeat(kc, 3, 0), np.repeat(vc, 3, 0), 0.25, 0.5,
                                               sel[:3], cnt[:3], ts)
    want, want_lse = oracle.sparse_attn_decode(qd, rp, np.repeat(kint, 3, 0) * 0.25, np.repeat(vint, 3, 0) * 0.5,
                                               sel[:3], cnt[:3], ts)
    np.testing.assert_array_equal(out, want)
    np.testing.assert_array_equal(lse, want_lse)


def test_fp8kv_scales_act_as_logit_and_output_factors():
    rng = np.random.default_rng(91)
    q, seq, pos, _, _, sel, cnt = _fp8kv_case(91)
    L, Hkv, D = 4 * 60 + 2, 2, 32
    kc = rng.integers(0, 256, size=(1, L, Hkv, D)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(1, L, Hkv, D)).astype(np.uint8)
    kc[(kc & 0x7f) == 0x7f] = 0x38                               # no NaN codes
    vc[(vc & 0x7f) == 0x7f] = 0x38
    ks, vs, sm = 0.0137, 0.0211, 1 / math.sqrt(D)
    out, lse = oracle.sparse_attn_prefill_fp8kv(q, seq, pos, kc, vc, ks, vs, sel, cnt, sm)
    # k_scale multiplies every logit: the same as scaling the softmax scale
    out2, lse2 = oracle.sparse_attn_prefill_fp8kv(q, seq, pos, kc, vc, ks * 3.0, vs, sel, cnt, sm / 3.0)
    np.testing.assert_allclose(out2, out, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(lse2, lse, rtol=1e-6, atol=1e-7)
    # v_scale multiplies the output and leaves lse alone
    out3, lse3 = oracle.sparse_attn_prefill_fp8kv(q, seq, pos, kc, vc, ks, vs * 5.0, sel, cnt, sm)
    np.testing.assert_allclose(out3, out * 5.0, rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(lse3, lse)


def test_fp8kv_zero_query_averages_the_decoded_values():
    # q = 0: uniform weights over the attended positions, whose values are
    # v_scale * E4M3(code); lse = log(number of positions)
    q, seq, pos, kint, vint, sel, cnt = _fp8kv_case(92)
    rng = np.random.default_rng(93)
    vc = rng.integers(0, 256, size=vint.shape).astype(np.uint8)
    vc[(vc & 0x7f) == 0x7f] = 0x40
    vs = 0.037
    out, lse = oracle.sparse_attn_prefill_fp8kv(np.zeros_like(q), seq, pos, oracle.fp8_from_float(kint), vc, 0.5,
                                                vs, sel, cnt)
    vals = oracle.fp8_to_float(vc).astype(np.float64) * vs
    for r, t in enumerate(pos):
        P = [4 * b + i for b in sel[r, :cnt[r]] for i in range(4)] + list(range(4 * ((t + 1) // 4), t + 1))
        for h in range(q.shape[1]):
            g = h // (q.shape[1] // vint.shape[2])
            np.testing.assert_allclose(out[r, h], vals[0, P, g].mean(0), rtol=1e-6, atol=1e-7)
            assert lse[r, h] == pytest.approx(math.log(len(P)), rel=1e-6)


def test_fp8_codes_match_torch_float8_e4m3fn():
    # the FP8 K/V entry points take torch.float8_e4m3fn tensors as codes: its
    # conversion (a library routine) and the oracle's rounding give the same
    # codes on every finite value, the midpoints between them and random values
    table = oracle.fp8_to_float(np.arange(256, dtype=np.uint8))
    fin = np.sort(np.unique(table[np.isfinite(table)]))
    mids = (fin[1:] + fin[:-1]) / 2
    rng = np.random.default_rng(95)
    x = np.concatenate([fin, mids, rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01])
    x32 = x.astype(np.float32)
    n = len(fin) + len(mids)
    np.testing.assert_array_equal(x32[:n], x[:n])        # the values and midpoints are exact in fp32
    mine = oracle.fp8_from_float(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, theirs)


# --------------------------------------------------------------------------
# Learned-weight normalization of the pooled key, and YaRN-scaled RoPE
# ("normalized" in the SGLang post's QSA section; YaRN to 1M tokens in the
# flozi.net guide and the aicontrolled journal)
# --------------------------------------------------------------------------

def test_yarn_worked_example_by_regime():
    # base 2^64 makes pair d's frequency 2^-d, and L = 2*pi*2^10 makes it
    # turn r(d) = 2^(10-d) times over the original context: d = 5 sits on
    # the ramp's top (r = 32 -> unchanged), d = 10 on its foot (r = 1 -> 1/s),
    # d = 6 in between (r = 16: gamma = 15/31, h = (16/31)/4 + 15/31 = 19/31
    # of the frequency, at s = 4), d = 2 above it and d = 20 below it.
    L = 2 * math.pi * 2 ** 10
    f = oracle.yarn_freq(2.0 ** 64, s=4.0, L=L, alpha=1.0, beta=32.0)
    for d, factor in ((2, 1.0), (5, 1.0), (6, 19 / 31), (8, (1 - 3 / 31) / 4 + 3 / 31), (10, 0.25),
                      (20, 0.25)):
        assert math.isclose(f[d], factor * 2.0 ** -d, rel_tol=1e-12), (d, f[d] / 2.0 ** -d)
    # frequencies fall with d and stay within [theta/s, theta]
    plain = oracle.plain_freq(2.0 ** 64)
    assert np.all(np.diff(f) < 0)
    assert np.all(f <= plain * (1 + 1e-15)) and np.all(f >= plain / 4 * (1 - 1e-15))
    with pytest.raises(RuntimeError):
        oracle.yarn_freq(1e7, s=0.5, L=L)
    with pytest.raises(RuntimeError):
        oracle.yarn_freq(1e7, s=4.0, L=L, alpha=32.0, beta=1.0)


def test_yarn_keeps_fast_pairs_and_interpolates_slow_ones():
    # At the 1M setting, a pair that turns more than beta times over the
    # native context rotates exactly as plain RoPE; a pair that turns less
    # than alpha times rotates at position p as plain RoPE does at p/4
    # (position interpolation); scale 1 is plain RoPE.
    th = 1e7
    f = oracle.yarn_freq(th, **oracle.YARN_1M)
    plain = oracle.plain_freq(th)
    turns = 262144 * plain / (2 * math.pi)
    fast, slow = np.where(turns > 32)[0], np.where(turns < 1)[0]
    assert len(fast) > 20 and len(slow) > 15 and len(fast) + len(slow) < 64   # all three regimes at 1e7
    rng = np.random.default_rng(31)
    x = rng.standard_normal(DIM)
    for p in (4, 1000, 262_144, 1_048_572):
        y, yp, yq = oracle.rope_freq(x, p, f), oracle.rope(x, p, th), oracle.rope(x, p // 4, th)
        np.testing.assert_allclose(y[fast], yp[fast], rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[fast + 64], yp[fast + 64], rtol=0, atol=1e-12)
        np.testing.assert_allclose(y[slow], yq[slow], rtol=0, atol=1e-9)
        np.testing.assert_allclose(y[slow + 64], yq[slow + 64], rtol=0, atol=1e-9)
    one = oracle.yarn_freq(th, s=1.0, L=262144.0)
    np.testing.assert_allclose(one, plain, rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_freq(x, 123457, one), oracle.rope(x, 123457, th), atol=1e-9)


def test_pool_ex_yarn_is_rotation_after_pooling():
    # a constant block pools to its key rotated at 4b with YaRN's frequencies
    rng = np.random.default_rng(32)
    k = rng.standard_normal(DIM).astype(np.float32)
    raw = _raw(4 * 300)
    raw[0, 4 * 257:4 * 258] = k
    f = oracle.yarn_freq(1e7, **oracle.YARN_1M)
    out = oracle.pool_ex(raw, 257, 258, f)[0, 257]
    np.testing.assert_allclose(out, oracle.rope_freq(k.astype(np.float64), 4 * 257, f), rtol=1e-6, atol=1e-6)
    # with plain frequencies it is qsa pooling itself
    np.testing.assert_array_equal(oracle.pool_ex(raw, 0, 300, oracle.plain_freq(1e7)), oracle.pool(raw, 0, 300, 1e7))


def test_pool_ex_norm_weight():
    rng = np.random.default_rng(33)
    raw = rng.standard_normal((2, 4 * 50, DIM)).astype(np.float32)
    f = oracle.plain_freq(1e7)
    nf = oracle.FLAG_POOL_RMSNORM
    # unit weight is the unweighted norm
    np.testing.assert_array_equal(oracle.pool_ex(raw, 0, 50, f, np.ones(DIM, np.float32), nf),
                                  oracle.pool(raw, 0, 50, 1e7, nf))
    # one-hot weight c*e_j (no rotation): only dim j survives, as c * m_j / rms(m)
    j, c = 37, 1.5
    w = np.zeros(DIM, np.float32)
    w[j] = c
    out = oracle.pool_ex(raw, 0, 50, f, w, nf | oracle.FLAG_NO_ROPE)
    m = raw.reshape(2, 50, 4, DIM).astype(np.float32)
    m = ((((m[:, :, 0] + m[:, :, 1]) + m[:, :, 2]) + m[:, :, 3]) * np.float32(0.25)).astype(np.float64)
    rms = np.sqrt((m * m).mean(-1) + 1e-6)
    want = np.zeros_like(out)
    want[:, :, j] = (c * m[:, :, j] / rms).astype(np.float32)
    np.testing.assert_allclose(out, want, rtol=1e-7, atol=0)
    # the weight scales each dim: doubling it doubles the (fp32) key exactly
    w = rng.uniform(0.5, 1.5, DIM).astype(np.float32)
    a = oracle.pool_ex(raw, 0, 50, f, w, nf | oracle.FLAG_NO_ROPE)
    b = oracle.pool_ex(raw, 0, 50, f, 2 * w, nf | oracle.FLAG_NO_ROPE)
    np.testing.assert_array_equal(b, 2 * a)
    # with rotation, the norm of the rotated key is that of the weighted normalized mean
    r = oracle.pool_ex(raw, 0, 50, oracle.yarn_freq(1e7, **oracle.YARN_1M), w, nf).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(w * m / rms[..., None], axis=-1),
                               rtol=1e-6)
    with pytest.raises(RuntimeError):   # a weight without the norm
        oracle.pool_ex(raw, 0, 50, f, w, 0)


def test_score_topk_ex_yarn_brute_force_and_relative_shift():
    rng = np.random.default_rng(34)
    f = oracle.yarn_freq(1e7, **oracle.YARN_1M)
    NB, R, k = 300, 6, 20
    raw = rng.standard_normal((1, 4 * NB, DIM)).astype(np.float32)
    pooled = oracle.pool_ex(raw, 0, NB, f)
    iq = rng.standard_normal((R, 4, DIM)).astype(np.float32)
    pos = rng.integers(4 * k, 4 * NB, R).astype(np.int32)
    seq = np.zeros(R, np.int32)
    sel, cnt, _, raw_s = oracle.score_topk_ex(iq, seq, pos, pooled, k, f, want_raw=True)
    for r in range(R):    # numpy fp64 brute force on the same rotations
        qr = np.stack([oracle.rope_freq(iq[r, h], int(pos[r]), f) for h in range(4)]).astype(np.float32)
        nc = (int(pos[r]) + 1) // 4
        dots = np.einsum("hd,bd->hb", qr.astype(np.float64), pooled[0, :nc].astype(np.float64))
        np.testing.assert_allclose(raw_s[r, :nc], np.maximum(dots, 0).sum(0), rtol=1e-12, atol=1e-12)
        order = np.lexsort((np.arange(nc), -raw_s[r, :nc]))[:k]
        np.testing.assert_array_equal(sel[r, :cnt[r]], np.sort(order))
    # scores depend only on query position minus key position: moving the
    # queries and the keys by 4*D tokens leaves them unchanged
    D = 1000
    raw2 = np.zeros((1, 4 * (NB + D), DIM), np.float32)
    raw2[0, 4 * D:] = raw[0]
    pooled2 = oracle.pool_ex(raw2, 0, NB + D, f)
    _, _, _, raw_t = oracle.score_topk_ex(iq, seq, pos + 4 * D, pooled2, k, f, want_raw=True)
    for r in range(R):
        nc = (int(pos[r]) + 1) // 4
        np.testing.assert_allclose(raw_t[r, D:D + nc], raw_s[r, :nc], rtol=2e-5, atol=2e-5)
