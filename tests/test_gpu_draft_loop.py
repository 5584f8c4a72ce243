"""The IndexShare draft loop over N steps on the GPU, through the C-ABI
("Qwen3.8-Flash-Next: Day-0 Support in SGLang", section "IndexShare MTP": the
selection taken at draft-extend serves every draft step, which adds the
positions drafted since; the indexer's ring and compressed cache keep up with
the drafted tokens).

One loop: the anchor at L-1 scores and selects once; draft step i (position
L+i) attends the captured selection plus [L, L+i] and appends its raw index key
to the ring, which completes block L/4 at the last step; the next anchor then
scores with that block visible.  Checked against the oracle at every step, and
each step's output against the row of one batched call over all N draft rows
(bit for bit: the same positions reach the same MFMA slots, the others carry
P = 0).
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, check_selection, dev, host

pytestmark = pytest.mark.gpu

DIM = 128


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 1, 128), (24, 2, 256)])
def test_draft_loop_shares_one_selection(gpu, Hq, Hkv, D):
    import torch
    N = 4
    spec = synth.scaled("decode-1m-draft", ctx=32768, q_per_seq=N, Hq=Hq, Hkv=Hkv, D=D)
    w = synth.make(spec)
    B, L, k, theta = spec.batch, spec.ctx, spec.top_k, spec.theta
    assert L % 4 == 0
    rng = np.random.default_rng(77)
    draft_keys = synth.bf16_bits(rng.standard_normal((B, N, DIM)).astype(np.float32))
    raw_ext = np.concatenate([w["raw_keys"], draft_keys], axis=1)     # [B][L+N][128]
    nb_alloc = (L + N) // 4 + 1
    # compressed cache [B][nb_alloc][128], contiguous per sequence: token t of
    # sequence s sits at slot s * 4 * nb_alloc + t
    pooled = torch.zeros((B, nb_alloc, DIM), dtype=torch.bfloat16, device="cuda")
    qsa.pool_index_keys(dev(w["raw_keys"], "bf16"), pooled, 0, L // 4, theta)
    ring = torch.zeros((B, 4, DIM), dtype=torch.bfloat16, device="cuda")    # block L/4 starts empty

    # draft-extend: the anchor selects once
    sel, cnt, _ = qsa.score_topk(dev(w["idx_q"], "bf16"), dev(w["row_seq"], "i"), dev(w["row_pos"], "i"), pooled,
                                 L // 4, k, theta, want_scores=False)
    o_pool = oracle.pool(raw_ext, 0, (L + N) // 4, theta)
    o_sel, o_cnt, _, o_raw = oracle.score_topk(w["idx_q"], w["row_seq"], w["row_pos"], o_pool[:, :L // 4], k,
                                               theta, want_raw=True)
    check_selection(host(sel), host(cnt), o_sel, o_cnt, o_raw, exact=False)
    g_sel, g_cnt = host(sel), host(cnt)

    kc, vc, q = dev(w["k_cache"], "bf16"), dev(w["v_cache"], "bf16"), dev(w["q"], "bf16")
    ts = dev(w["tail_start"], "i")
    assert np.all(w["tail_start"] == L)
    batched, batched_lse = qsa.sparse_attn_decode(q, dev(w["attn_pos"], "i"), kc, vc, sel, cnt, ts)
    batched, batched_lse = host(batched), host(batched_lse)
    for i in range(N):
        # draft step i: one row per sequence at position L + i, same selection
        pos_i = np.full((B, 1), L + i, np.int32)
        out, lse = qsa.sparse_attn_decode(q[:, i:i + 1].contiguous(), dev(pos_i, "i"), kc, vc, sel, cnt, ts)
        want, want_lse = oracle.sparse_attn_decode(w["q"][:, i:i + 1], pos_i, w["k_cache"], w["v_cache"], g_sel,
                                                   g_cnt, w["tail_start"])
        print(f"[draft loop] {Hq}/{Hkv}/{D} step {i}", flush=True)
        assert_close_out(host(out), want, "bf16")
        np.testing.assert_allclose(host(lse), want_lse, rtol=1e-5, atol=1e-4)
        np.testing.assert_array_equal(host(out)[:, 0], batched[:, i])
        np.testing.assert_array_equal(host(lse)[:, 0], batched_lse[:, i])
        # the drafted token's raw index key enters the ring
        slots = torch.tensor([s * 4 * nb_alloc + L + i for s in range(B)], dtype=torch.int64, device="cuda")
        qsa.pool_append(dev(draft_keys[:, i], "bf16"), torch.full((B,), L + i, dtype=torch.int32, device="cuda"),
                        slots, ring, pooled.view(B * nb_alloc, DIM), theta)

    # block L/4 completed at the last step: its compressed key is the oracle's
    np.testing.assert_array_equal(host(pooled)[:, L // 4], o_pool[:, L // 4])
    # the next draft-extend: an anchor at L + N - 1 sees the new block
    iq2 = synth.bf16_bits((rng.standard_normal((B, 4, DIM)) + 0.5).astype(np.float32))
    seq2 = np.arange(B, dtype=np.int32)
    pos2 = np.full(B, L + N - 1, np.int32)
    sel2, cnt2, _ = qsa.score_topk(dev(iq2, "bf16"), dev(seq2, "i"), dev(pos2, "i"), pooled, (L + N) // 4, k, theta,
                                   want_scores=False)
    o_sel2, o_cnt2, _, o_raw2 = oracle.score_topk(iq2, seq2, pos2, o_pool, k, theta, want_raw=True)
    check_selection(host(sel2), host(cnt2), o_sel2, o_cnt2, o_raw2, exact=False)
