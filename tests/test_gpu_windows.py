"""Selections whose visible range spans more than one emission window, through
the C-ABI, against the oracle ("Qwen3.8-Flash-Next: Day-0 Support in SGLang",
section "Qwen Sparse Attention": the best 512 blocks by s = 1/sqrt(128) *
sum_h ReLU(<q_h, kbar_b>), returned in block order).

Both selection paths write the kept blocks in block order through a bitmap of
the visible range taken one window at a time: the fused scorer's merge in
windows of 65,536 blocks, the split selection in windows of 262,144 blocks.
Rows here end just past a window boundary, exactly on one, and far beyond;
high-scoring blocks are planted on both sides of every boundary, so that kept
blocks sit in each window and at its edges.  Scores are checked too (they
travel with the kept entries), and a call without scores must select the
same blocks.
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


def _case(seed, NB, R, boundaries):
    rng = np.random.default_rng(seed)
    iq = rng.standard_normal((R, 4, DIM)).astype(np.float32)
    pooled = rng.standard_normal((1, NB, DIM)).astype(np.float32)
    # keys along the sum of every query head score high for every row (RoPE
    # is off, so the planted keys stay aligned with the queries)
    direction = iq.sum(axis=(0, 1))
    direction /= np.linalg.norm(direction)
    for edge in boundaries:
        for b in range(edge - 6, edge + 6):
            if 0 <= b < NB:
                pooled[0, b] = 12.0 * direction + 0.1 * rng.standard_normal(DIM)
    return synth.bf16_bits(iq), synth.bf16_bits(pooled)


@pytest.mark.parametrize("path,window,windows", [("gemm", 65536, 3), ("rows", 262144, 2)])
def test_selection_across_emission_windows(gpu, path, window, windows):
    NB = window * (windows - 1) + 9001          # a ragged last window
    edges = [window * i for i in range(1, windows)]
    # nc: every block; one window exactly; one block into the second; one block
    # into the last window; and a short row
    nc = [NB, window, window + 1, edges[-1] + 1, 700]
    pos = np.array([4 * c - 1 for c in nc], np.int32)
    R = len(pos)
    iq, pooled = _case(5 + windows, NB, R, edges)
    seq = np.zeros(R, np.int32)
    k = 512
    flags = qsa.FLAG_NO_ROPE | (qsa.FLAG_SCORE_GEMM if path == "gemm" else qsa.FLAG_SCORE_ROWS)
    print(f"[windows] path={path} NB={NB} rows={R}", flush=True)
    o_sel, o_cnt, _, o_raw = oracle.score_topk(iq, seq, pos, pooled, k, THETA, qsa.FLAG_NO_ROPE, want_raw=True)
    args = (dev(iq, "bf16"), dev(seq, "i"), dev(pos, "i"), dev(pooled, "bf16"), NB, k, THETA)
    sel, cnt, sc = qsa.score_topk(*args, flags=flags)
    g_sel, g_cnt, g_sc = host(sel), host(cnt), host(sc)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, o_raw, exact=False)
    # the planted blocks before each row's end are kept, on both sides of
    # every boundary the row reaches
    for r in range(R):
        kept = set(g_sel[r, :g_cnt[r]].tolist())
        for edge in edges:
            for b in range(edge - 6, edge + 6):
                if b < nc[r]:
                    assert b in kept, (r, b)
        n = g_cnt[r]
        np.testing.assert_allclose(g_sc[r, :n], o_raw[r, g_sel[r, :n]] / math.sqrt(128), rtol=1e-3, atol=1e-3)
    sel2, cnt2, _ = qsa.score_topk(*args, flags=flags, want_scores=False)
    np.testing.assert_array_equal(host(sel2), g_sel)
    np.testing.assert_array_equal(host(cnt2), g_cnt)
