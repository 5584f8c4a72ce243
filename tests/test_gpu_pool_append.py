"""Incremental decode pooling through the C-ABI (qsa_pool_append) against the
oracle, step by step: each request's raw keys go through its 4-slot ring one
decode step at a time, in a paged KV layout whose pages are shuffled; every
finished block's compressed key must land at full_slot / 4.  Tolerance as for
block pooling: 1 bf16 ulp (bit-exact with RoPE off), fp32 within rounding."""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import dev, host

pytestmark = pytest.mark.gpu

DIM = 128


def _run(dtype, flags, B, L, page_tokens, seed, stagger):
    import torch
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, DIM)).astype(np.float32)
    raw = synth.bf16_bits(x) if dtype == "bf16" else x
    slots = synth.paged_slots(rng, B, L, page_tokens)
    nslots = int(slots.max()) // 4 + 1
    sentinel = synth.bf16_bits(np.float32(-7.0)) if dtype == "bf16" else np.float32(-7.0)
    o_ring = np.zeros((B, 4, DIM), raw.dtype)
    o_comp = np.full((nslots, DIM), sentinel, raw.dtype)
    g_ring = dev(o_ring, dtype)
    g_comp = dev(o_comp, dtype)
    starts = rng.integers(0, 5, size=B) if stagger else np.zeros(B, np.int64)
    for step in range(L + 5):
        t = starts + step - 4 if stagger else starts + step   # staggered requests join late
        live = (t >= 0) & (t < L)
        r = np.nonzero(live)[0]
        if len(r) == 0:
            continue
        tt = t[r]
        keys = np.ascontiguousarray(raw[r, tt])
        pos = tt.astype(np.int32)
        fs = np.ascontiguousarray(slots[r, tt])
        # the live requests' rings, gathered (the kernel reads ring[i] for request i of the call)
        sub = o_ring[r].copy()
        oracle.pool_append(keys, pos, fs, sub, o_comp, 1e7, flags)
        o_ring[r] = sub
        g_sub = g_ring[torch.as_tensor(r, device="cuda")].contiguous()
        qsa.pool_append(dev(keys, dtype), dev(pos, "i"), dev(fs, "i"), g_sub, g_comp, 1e7, flags)
        g_ring[torch.as_tensor(r, device="cuda")] = g_sub
    gr, gc = host(g_ring), host(g_comp)
    if dtype == "bf16":
        assert np.abs(gc.astype(np.int32) - o_comp.astype(np.int32)).max() <= 1
        if flags & qsa.FLAG_NO_ROPE:
            np.testing.assert_array_equal(gc, o_comp)
    else:
        np.testing.assert_allclose(gc, o_comp, rtol=2e-6, atol=1e-6)
    np.testing.assert_array_equal(gr, o_ring)           # the rings hold the raw keys, bit for bit
    # untouched compressed slots keep their contents (no write outside finished blocks)
    done = set(int(slots[b, 4 * j]) // 4 for b in range(B) for j in range(L // 4))
    rest = [s_ for s_ in range(nslots) if s_ not in done]
    assert (gc[rest] == sentinel).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("flags", [0, qsa.FLAG_NO_ROPE, qsa.FLAG_POOL_RMSNORM])
def test_pool_append_matches_oracle(gpu, dtype, flags):
    _run(dtype, flags, B=5, L=43, page_tokens=16, seed=31, stagger=False)


def test_pool_append_staggered_requests(gpu):
    _run("bf16", 0, B=7, L=30, page_tokens=8, seed=32, stagger=True)


def test_pool_append_large_positions(gpu):
    # positions near 1M tokens: the rotation angle is formed in fp64 on both sides
    import torch
    rng = np.random.default_rng(33)
    B = 4
    t0 = 1048572                                         # block 262143 completes at t0 + 3
    keys = synth.bf16_bits(rng.standard_normal((4, B, DIM)).astype(np.float32))
    slots = (np.arange(B, dtype=np.int64) * 16 + 4)      # a page-aligned slot per request
    o_ring = np.zeros((B, 4, DIM), np.uint16)
    o_comp = np.zeros((B * 4 + 2, DIM), np.uint16)
    g_ring, g_comp = dev(o_ring, "bf16"), dev(o_comp, "bf16")
    for i in range(4):
        pos = np.full(B, t0 + i, np.int32)
        fs = slots + i
        oracle.pool_append(keys[i], pos, fs, o_ring, o_comp, 1e7)
        qsa.pool_append(dev(keys[i], "bf16"), dev(pos, "i"), dev(fs, "i"), g_ring, g_comp, 1e7)
    assert np.abs(host(g_comp).astype(np.int32) - o_comp.astype(np.int32)).max() <= 1
