"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (default score path, caller-provided workspaces, the chunk's
new blocks pooled on top of a pooled context).  The GPU runs every row.  The
oracle checks the selection of every row under the near-tie rule (prefill
rows in batches, so the oracle's raw scores stay in memory), and attention on
the GPU's own selection on a sample of rows (decode: every row), with the
tolerances of the small-size parity tests.  Prefill prints how many rows each
of the fused scorer's merge modes ranked.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128


def _sample_rows(R, n=24, seed=7):
    rng = np.random.default_rng(seed)
    rows = {0, R - 1, R // 2} | set(rng.choice(R, size=min(R, n), replace=False).tolist())
    return np.array(sorted(rows), np.int64)


def _prefill(spec):
    import torch
    w = synth.make(spec)
    dt = spec.dtype
    L, nb, k = spec.ctx, spec.n_blocks, spec.top_k
    first_new = (L - spec.chunk) // 4
    raw = dev(w["raw_keys"], dt)
    pooled_d = torch.zeros((1, nb, DIM), dtype=raw.dtype, device="cuda")
    if first_new:
        qsa.pool_index_keys(raw, pooled_d, 0, first_new, spec.theta)
    qsa.pool_index_keys(raw, pooled_d, first_new, nb, spec.theta)
    R, max_nb = spec.chunk, L // 4
    ws = torch.empty((max(qsa.score_topk_workspace_size(R, max_nb, k, qsa.BF16), 256),), dtype=torch.uint8,
                     device="cuda")
    seq, pos = dev(w["row_seq"], "i"), dev(w["row_pos"], "i")
    sel, cnt, _ = qsa.score_topk(dev(w["idx_q"], dt), seq, pos, pooled_d, max_nb, k, spec.theta,
                                 workspace=ws, want_scores=False)
    out, lse = qsa.sparse_attn_prefill(dev(w["q"], dt), seq, pos, dev(w["k_cache"], dt),
                                       dev(w["v_cache"], dt), sel, cnt)
    moff = qsa.score_topk_merge_modes_offset(R, max_nb, k, qsa.BF16)
    assert moff is not None   # many rows: the fused scorer
    modes = host(ws[moff:moff + 4 * R]).view(np.int32)
    counts = {qsa.MERGE_MODES[m]: int((modes == m).sum()) for m in sorted(qsa.MERGE_MODES)}
    print(f"[full-size] {spec.name}: rows per merge mode {counts}", flush=True)
    assert set(np.unique(modes).tolist()) <= set(qsa.MERGE_MODES)
    pooled = host(pooled_d)
    o_pooled = oracle.pool(w["raw_keys"], 0, nb, spec.theta)
    assert np.abs(pooled.astype(np.int32) - o_pooled.astype(np.int32)).max() <= 1
    g_sel_all, g_cnt_all = host(sel), host(cnt)
    batch = max(64, int(2.5e8 // (8 * nb)))   # rows per oracle call: its raw scores stay near 256 MB
    swaps = 0
    for r0 in range(0, R, batch):
        rr = np.arange(r0, min(R, r0 + batch))
        o_sel, o_cnt, _, o_raw = oracle.score_topk(w["idx_q"][rr], w["row_seq"][rr], w["row_pos"][rr], pooled,
                                                   k, spec.theta, want_raw=True)
        swaps += check_selection(g_sel_all[rr], g_cnt_all[rr], o_sel, o_cnt, o_raw, exact=False)
        del o_raw
        print(f"[full-size] {spec.name}: selections of rows {rr[0]}..{rr[-1]} match ({swaps} near-tie swaps)",
              flush=True)
    rows = _sample_rows(R)
    print(f"[full-size] {spec.name}: attention on rows {rows.tolist()}", flush=True)
    g_sel, g_cnt = g_sel_all[rows], g_cnt_all[rows]
    want, want_lse = oracle.sparse_attn_prefill(w["q"][rows], w["row_seq"][rows], w["row_pos"][rows],
                                                w["k_cache"], w["v_cache"], g_sel, g_cnt)
    assert_close_out(host(out)[rows], want, dt)
    np.testing.assert_allclose(host(lse)[rows], want_lse, rtol=1e-5, atol=1e-4)


def _decode(spec):
    import torch
    w = synth.make(spec)
    dt = spec.dtype
    B, nb, k = spec.batch, spec.n_blocks, spec.top_k
    raw = dev(w["raw_keys"], dt)
    pooled_d = torch.zeros((B, nb, DIM), dtype=raw.dtype, device="cuda")
    qsa.pool_index_keys(raw, pooled_d, 0, nb, spec.theta)
    del raw
    max_nb = int((w["row_pos"].max() + 1) // 4)
    code = qsa.BF16 if dt == "bf16" else qsa.F32
    ws = torch.empty((max(qsa.score_topk_workspace_size(B, max_nb, k, code), 256),), dtype=torch.uint8,
                     device="cuda")
    wsa = torch.empty((max(qsa.sparse_attn_decode_workspace_size(B, spec.q_per_seq, spec.Hq, DIM, k), 256),),
                      dtype=torch.uint8, device="cuda")
    sel, cnt, _ = qsa.score_topk(dev(w["idx_q"], dt), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"), pooled_d,
                                 max_nb, k, spec.theta, workspace=ws, want_scores=False)
    ts = None if w["tail_start"] is None else dev(w["tail_start"], "i")
    out, lse = qsa.sparse_attn_decode(dev(w["q"], dt), dev(w["attn_pos"], "i"), dev(w["k_cache"], dt),
                                      dev(w["v_cache"], dt), sel, cnt, ts, workspace=wsa)
    pooled = host(pooled_d)
    del pooled_d
    o_pooled = oracle.pool(w["raw_keys"], 0, nb, spec.theta)
    if dt == "bf16":
        assert np.abs(pooled.astype(np.int32) - o_pooled.astype(np.int32)).max() <= 1
    else:
        np.testing.assert_allclose(pooled, o_pooled, rtol=2e-6, atol=1e-6)
    del o_pooled
    print(f"[full-size] {spec.name}: checking all {B} sequences", flush=True)
    g_sel, g_cnt = host(sel), host(cnt)
    o_sel, o_cnt, _, o_raw = oracle.score_topk(w["idx_q"], w["row_seq"], w["row_pos"], pooled, k, spec.theta,
                                               want_raw=True)
    check_selection(g_sel, g_cnt, o_sel, o_cnt, o_raw, exact=False)
    for s in range(B):  # planted needles are found (all of them when they fit)
        planted = set(w["planted"][s].tolist())
        got = set(g_sel[s, :g_cnt[s]].tolist())
        assert planted <= got if len(planted) <= k else got <= planted
    want, want_lse = oracle.sparse_attn_decode(w["q"], w["attn_pos"], w["k_cache"], w["v_cache"], g_sel, g_cnt,
                                               w["tail_start"])
    assert_close_out(host(out), want, dt)
    np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_full_size(gpu, name):
    spec = synth.SPECS[name]
    if spec.kind == "prefill":
        _prefill(spec)
    else:
        _decode(spec)
