"""FP8 index keys on the GPU against the oracle, through the C-ABI.

The compressed keys are stored as E4M3 codes with one FP32 scale per key
("Qwen3.8-Flash-Next, Layer by Layer", section "Serving it": the indexer's
keys kept in FP8).  Pooled codes: bit-exact with RoPE off on integer inputs;
with RoPE, each code within one E4M3 step of the oracle's (the rotation's
last-bit differences can cross a rounding boundary).  Scores: the oracle
scores the GPU's own codes and scales; selections identical except near-ties
within 1e-3 relative of the k-th score, and identical on exact inputs.
"""
import math

import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128
THETA = 1.0e7


def _gpu_pool_fp8(raw_np, nb, flags=0, dtype="bf16"):
    import torch
    raw = dev(raw_np, dtype)
    B = raw_np.shape[0]
    codes = torch.zeros((B, nb, DIM), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((B, nb), dtype=torch.float32, device="cuda")
    qsa.pool_index_keys_fp8(raw, codes, scales, 0, nb, THETA, flags)
    return host(codes), host(scales), codes, scales


def _step(v):
    """E4M3 spacing at |v| (2^-9 below 2^-6)."""
    a = np.abs(v)
    return np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pool_fp8_integer_inputs_bit_exact(gpu, dtype):
    rng = np.random.default_rng(61)
    B, NB = 3, 700
    raw = rng.integers(-8, 9, size=(B, 4 * NB + 3, DIM)).astype(np.float32)
    raw = synth.bf16_bits(raw) if dtype == "bf16" else raw
    g_codes, g_scales, _, _ = _gpu_pool_fp8(raw, NB, qsa.FLAG_NO_ROPE, dtype)
    o_codes, o_scales = oracle.pool_fp8(raw, 0, NB, THETA, oracle.FLAG_NO_ROPE)
    np.testing.assert_array_equal(g_scales, o_scales)
    np.testing.assert_array_equal(g_codes, o_codes)


@pytest.mark.parametrize("flags", [0, qsa.FLAG_POOL_RMSNORM])
def test_pool_fp8_matches_oracle(gpu, flags):
    rng = np.random.default_rng(62 + flags)
    B, NB = 2, 2500
    raw = synth.bf16_bits(rng.standard_normal((B, 4 * NB, DIM)).astype(np.float32))
    g_codes, g_scales, _, _ = _gpu_pool_fp8(raw, NB, flags)
    o_codes, o_scales = oracle.pool_fp8(raw, 0, NB, THETA, flags)
    np.testing.assert_allclose(g_scales, o_scales, rtol=4e-7, atol=0)
    gv, ov = oracle.fp8_to_float(g_codes), oracle.fp8_to_float(o_codes)
    assert np.all(np.abs(gv - ov) <= _step(ov) * (1 + 1e-9)), "a code is more than one step away"
    assert np.mean(g_codes == o_codes) > 0.999


def _score_case(seed, B, NB, R, k):
    rng = np.random.default_rng(seed)
    raw = synth.bf16_bits(rng.standard_normal((B, 4 * NB, DIM)).astype(np.float32))
    iq = synth.bf16_bits(rng.standard_normal((R, 4, DIM)).astype(np.float32))
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    pos[:3] = [0, 4 * k - 2, 4 * NB - 1]          # no block, just below k blocks, every block
    return raw, iq, seq, pos


@pytest.mark.parametrize("path,R,NB", [("rows", 40, 9001), ("rows", 90, 2600), ("gemm", 90, 2600),
                                       ("gemm", 130, 5000)])
@pytest.mark.parametrize("k", [512, 37])
def test_score_topk_fp8_matches_oracle(gpu, path, R, NB, k):
    B = 2
    raw, iq, seq, pos = _score_case(71 + k, B, NB, R, k)
    g_codes, g_scales, codes, scales = _gpu_pool_fp8(raw, NB)
    flags = qsa.FLAG_SCORE_ROWS if path == "rows" else qsa.FLAG_SCORE_GEMM
    sel, cnt, sc = qsa.score_topk_fp8(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), codes, scales, NB, k, THETA,
                                      flags=flags)
    o_sel, o_cnt, o_sc, o_raw = oracle.score_topk_fp8(iq, seq, pos, g_codes, g_scales, k, THETA, want_raw=True)
    g_sel, g_cnt, g_sc = host(sel), host(cnt), host(sc)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, o_raw, exact=False)
    for r in range(R):
        n = g_cnt[r]
        want = o_raw[r, g_sel[r, :n]] / math.sqrt(128)
        np.testing.assert_allclose(g_sc[r, :n], want, rtol=1e-3, atol=1e-3)
        assert np.all(g_sc[r, n:] == 0)


@pytest.mark.parametrize("path", ["rows", "gemm"])
def test_score_topk_fp8_exact_keys_bit_exact(gpu, path):
    # integer keys with an element at 448 (scale exactly 1): codes are the
    # integers, every score is exact, so the selection (ties included) is too
    import torch
    rng = np.random.default_rng(73)
    B, NB, R, k = 2, 3000, 80, 64
    kv = rng.integers(-4, 5, size=(B, NB, DIM)).astype(np.float32)
    kv[..., 5] = 448.0
    g_codes = oracle.fp8_from_float(kv)                 # test input: exact codes
    g_scales = np.ones((B, NB), np.float32)
    iq = synth.bf16_bits(rng.integers(-3, 4, size=(R, 4, DIM)).astype(np.float32) / 64)
    iq_f = synth.bf16_to_f32(iq).reshape(R, 4, DIM)
    iq_f[:, :, 5] = 0.0                                 # keep the 448 column out of the dot products
    iq = synth.bf16_bits(iq_f)
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    flags = qsa.FLAG_NO_ROPE | (qsa.FLAG_SCORE_ROWS if path == "rows" else qsa.FLAG_SCORE_GEMM)
    codes = torch.from_numpy(g_codes).cuda()
    scales = torch.from_numpy(g_scales).cuda()
    sel, cnt, sc = qsa.score_topk_fp8(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), codes, scales, NB, k, THETA,
                                      flags=flags)
    o_sel, o_cnt, o_sc, _ = oracle.score_topk_fp8(iq, seq, pos, g_codes, g_scales, k, THETA, oracle.FLAG_NO_ROPE)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)
    np.testing.assert_array_equal(host(sc), o_sc)


def test_score_topk_fp8_long_pair_lists(gpu):
    # the merge's prefilter and its list-walking path on FP8 keys (scores
    # exact: integer codes, scale 1)
    import torch
    rng = np.random.default_rng(74)
    NB, R, k = 8192, 64, 512
    vals = np.ones(NB, np.float32)
    blocks = rng.permutation(NB)
    vals[blocks[:600]] = rng.choice(np.arange(129, 449, dtype=np.float32), size=600)
    vals[blocks[600:2200]] = 100.0
    kv = np.zeros((1, NB, DIM), np.float32)
    kv[0, :, 0] = vals
    kv[0, :, 1] = 448.0                                  # scale exactly 1
    g_codes = oracle.fp8_from_float(kv)
    g_scales = np.ones((1, NB), np.float32)
    iq = np.zeros((R, 4, DIM), np.float32)
    iq[:, 0, 0] = rng.integers(1, 5, R)
    iq = synth.bf16_bits(iq)
    seq = np.zeros(R, np.int32)
    pos = np.full(R, 4 * NB - 1, np.int32)
    sel, cnt, sc = qsa.score_topk_fp8(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), torch.from_numpy(g_codes).cuda(),
                                      torch.from_numpy(g_scales).cuda(), NB, k, THETA,
                                      flags=qsa.FLAG_NO_ROPE | qsa.FLAG_SCORE_GEMM)
    o_sel, o_cnt, o_sc, _ = oracle.score_topk_fp8(iq, seq, pos, g_codes, g_scales, k, THETA, oracle.FLAG_NO_ROPE)
    np.testing.assert_array_equal(host(cnt), o_cnt)
    np.testing.assert_array_equal(host(sel), o_sel)
    np.testing.assert_array_equal(host(sc), o_sc)


@pytest.mark.parametrize("name", ["decode-1m-draft", "chunk-256k"])
def test_fp8_full_size_sampled(gpu, name):
    # the bench workloads with FP8 keys: pooled codes on sampled blocks, then
    # the selection of sampled rows against the oracle on the GPU's keys
    import torch
    spec = synth.SPECS[name]
    w = synth.make(spec)
    raw = dev(w["raw_keys"], "bf16")
    B, nb = raw.shape[0], spec.n_blocks
    codes = torch.zeros((B, nb, DIM), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((B, nb), dtype=torch.float32, device="cuda")
    qsa.pool_index_keys_fp8(raw, codes, scales, 0, nb, spec.theta)
    del raw
    g_codes, g_scales = host(codes), host(scales)
    rng = np.random.default_rng(5)
    blk = np.sort(rng.choice(nb, size=min(nb, 4000), replace=False))
    o_codes, o_scales = oracle.pool_fp8(w["raw_keys"][:, : 4 * (int(blk[-1]) + 1)], 0, int(blk[-1]) + 1, spec.theta)
    gv, ov = oracle.fp8_to_float(g_codes[:, blk]), oracle.fp8_to_float(o_codes[:, blk])
    assert np.all(np.abs(gv - ov) <= _step(ov) * (1 + 1e-9))
    np.testing.assert_allclose(g_scales[:, blk], o_scales[:, blk], rtol=4e-7)
    R = w["idx_q"].shape[0]
    rows = np.arange(R) if R <= 64 else np.unique(np.concatenate([[0, R // 2, R - 1],
                                                                   rng.choice(R, 21, replace=False)]))
    max_nb = int((w["row_pos"].max() + 1) // 4)
    sel, cnt, _ = qsa.score_topk_fp8(dev(w["idx_q"], "bf16"), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"),
                                     codes, scales, max_nb, spec.top_k, spec.theta, want_scores=False)
    print(f"[fp8 full-size] {name}: checking rows {rows.tolist()}", flush=True)
    o_sel, o_cnt, _, o_raw = oracle.score_topk_fp8(w["idx_q"][rows], w["row_seq"][rows], w["row_pos"][rows], g_codes,
                                                   g_scales, spec.top_k, spec.theta, want_raw=True)
    check_selection(host(sel)[rows], host(cnt)[rows], o_sel, o_cnt, o_raw, exact=False)
