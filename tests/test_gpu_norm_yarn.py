"""The learned-weight normalization of the pooled key and YaRN-scaled RoPE on
the GPU, through qsa_pool_index_keys_ex / qsa_score_topk_ex, against the
oracle ("Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "Qwen Sparse
Attention": the averaged keys are normalized, then rotated; flozi.net guide
and aicontrolled journal: the native 262,144-token context extends to one
million tokens with YaRN).  Tolerances as in the contiguous parity tests:
pooled keys within 1 bf16 ulp, 99.9% bit-exact (fp32: 2e-6 relative);
selections identical except near-ties within 1e-3 relative of the k-th
score.  With the defaults (unit weight, yarn_factor 1) the _ex calls equal
the plain entry points bit for bit.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128
THETA = 1.0e7
Y = oracle.YARN_1M   # s = 4 over the native 262,144 tokens, ramp 1..32


def _yarn_rope():
    return qsa.rope(THETA, Y["s"], Y["L"], Y["alpha"], Y["beta"])


def _store(x, dtype):
    return synth.bf16_bits(x.astype(np.float32)) if dtype == "bf16" else x.astype(np.float32)


def _close_keys(got, want, dtype):
    if dtype == "bf16":
        diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
        assert diff.max() <= 1 and (diff == 0).mean() > 0.999
    else:
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=1e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("yarn", [False, True])
def test_pool_ex_matches_oracle(gpu, dtype, yarn):
    import torch
    rng = np.random.default_rng(300 + yarn)
    B, NB = 2, 1203
    raw = _store(rng.standard_normal((B, 4 * NB + 1, DIM)) * 2.0, dtype)
    w = rng.uniform(0.25, 2.0, DIM).astype(np.float32)
    flags = qsa.FLAG_POOL_RMSNORM
    freq = oracle.yarn_freq(THETA, **Y) if yarn else oracle.plain_freq(THETA)
    rp = _yarn_rope() if yarn else qsa.rope(THETA)
    pooled = dev(np.zeros((B, NB, DIM), raw.dtype), dtype)
    # a block offset as in a chunk: blocks [37, NB) only
    qsa.pool_index_keys_ex(dev(raw, dtype), pooled, 37, NB, rp, torch.from_numpy(w).cuda(), flags)
    got = host(pooled)
    want = oracle.pool_ex(raw, 37, NB, freq, w, flags)
    _close_keys(got[:, 37:], want[:, 37:], dtype)
    assert not np.any(got[:, :37])
    # YaRN alone (no norm)
    qsa.pool_index_keys_ex(dev(raw, dtype), pooled, 0, NB, rp, None, 0)
    _close_keys(host(pooled), oracle.pool_ex(raw, 0, NB, freq), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ex_defaults_equal_plain_entry_points(gpu, dtype):
    import torch
    rng = np.random.default_rng(310)
    B, NB, R, k = 2, 900, 70, 64
    raw = _store(rng.standard_normal((B, 4 * NB, DIM)), dtype)
    rd = dev(raw, dtype)
    a = dev(np.zeros((B, NB, DIM), raw.dtype), dtype)
    b = dev(np.zeros((B, NB, DIM), raw.dtype), dtype)
    for flags in (0, qsa.FLAG_POOL_RMSNORM):
        qsa.pool_index_keys(rd, a, 0, NB, THETA, flags)
        w = torch.ones(DIM, dtype=torch.float32, device="cuda") if flags else None
        qsa.pool_index_keys_ex(rd, b, 0, NB, qsa.rope(THETA), w, flags)
        np.testing.assert_array_equal(host(a), host(b))
        qsa.pool_index_keys_ex(rd, b, 0, NB, qsa.rope(THETA, 1.0, 262144.0), None, flags)  # factor 1: plain
        np.testing.assert_array_equal(host(a), host(b))
    iq = _store(rng.standard_normal((R, 4, DIM)), dtype)
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    args = (dev(iq, dtype), dev(seq, "i"), dev(pos, "i"), a, NB, k)
    x = [host(t) for t in qsa.score_topk(*args, THETA)]
    y = [host(t) for t in qsa.score_topk_ex(*args, qsa.rope(THETA))]
    for u, v in zip(x, y):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("path,R", [("rows", 24), ("gemm", 150)])
def test_score_topk_ex_yarn_matches_oracle(gpu, path, R):
    rng = np.random.default_rng(320 + R)
    B, NB, k = 2, 6000, 512
    raw = synth.bf16_bits(rng.standard_normal((B, 4 * NB, DIM)).astype(np.float32))
    freq = oracle.yarn_freq(THETA, **Y)
    rp = _yarn_rope()
    pooled = dev(np.zeros((B, NB, DIM), np.uint16), "bf16")
    qsa.pool_index_keys_ex(dev(raw, "bf16"), pooled, 0, NB, rp, None, 0)
    g_pooled = host(pooled)
    _close_keys(g_pooled, oracle.pool_ex(raw, 0, NB, freq), "bf16")
    iq = synth.bf16_bits(rng.standard_normal((R, 4, DIM)).astype(np.float32))
    seq = rng.integers(0, B, R).astype(np.int32)
    pos = rng.integers(0, 4 * NB, R).astype(np.int32)
    pos[:3] = [4 * NB - 1, 4 * k + 2, 3]
    flags = qsa.FLAG_SCORE_ROWS if path == "rows" else qsa.FLAG_SCORE_GEMM
    sel, cnt, sc = (host(t) for t in qsa.score_topk_ex(dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), pooled, NB,
                                                        k, rp, flags))
    o_sel, o_cnt, o_sc, o_raw = oracle.score_topk_ex(iq, seq, pos, g_pooled, k, freq, want_raw=True)
    check_selection(sel, cnt, o_sel, o_cnt, o_raw, exact=False)
    same = np.array([np.array_equal(sel[r], o_sel[r]) for r in range(R)])
    np.testing.assert_allclose(sc[same], o_sc[same], rtol=2e-5, atol=1e-5)
