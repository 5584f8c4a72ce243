"""The allocation-free decode entry point (qsa_sparse_attn_decode_noalloc)
against qsa_sparse_attn_decode, through the C-ABI: two calls in a row, the
second with a smaller input, each equal bit for bit to the workspace entry
point on the same inputs (the two share their kernels; only where the split
partials live differs).  Both are also checked against the oracle.
"""
import numpy as np
import pytest

import oracle
from block_sparse_long_amd import qsa, synth
from helpers import assert_close_out, dev, host

pytestmark = pytest.mark.gpu

DIM = 128


def _case(rng, B, Qn, Hq, Hkv, L, k, dtype):
    def store(x):
        return synth.bf16_bits(x.astype(np.float32)) if dtype == "bf16" else x.astype(np.float32)
    q = store(rng.standard_normal((B, Qn, Hq, DIM)))
    kc = store(rng.standard_normal((B, L + Qn, Hkv, DIM)))
    vc = store(rng.standard_normal((B, L + Qn, Hkv, DIM)))
    rpos = (L + np.arange(Qn))[None, :].repeat(B, 0).astype(np.int32)
    ts = np.full(B, L, np.int32)
    nc = L // 4
    n = min(k, nc)
    sel = np.full((B, k), -1, np.int32)
    for s in range(B):
        sel[s, :n] = np.sort(rng.choice(nc, size=n, replace=False))
    cnt = np.full(B, n, np.int32)
    return q, kc, vc, rpos, ts, sel, cnt


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_decode_equals_workspace_decode(gpu, dtype):
    rng = np.random.default_rng(2024)
    # the second call is smaller: fewer sequences, rows, kept blocks and positions
    for B, Qn, Hq, Hkv, L, k in ((4, 4, 8, 1, 9000, 512), (2, 2, 8, 2, 2100, 128)):
        q, kc, vc, rpos, ts, sel, cnt = _case(rng, B, Qn, Hq, Hkv, L, k, dtype)
        print(f"[no-alloc] {dtype} B={B} Qn={Qn} Hq={Hq} Hkv={Hkv} L={L} k={k}", flush=True)
        args = (dev(q, dtype), dev(rpos, "i"), dev(kc, dtype), dev(vc, dtype), dev(sel, "i"), dev(cnt, "i"),
                dev(ts, "i"))
        o_ws, l_ws = qsa.sparse_attn_decode(*args)
        o_na, l_na = qsa.sparse_attn_decode_noalloc(*args)
        np.testing.assert_array_equal(host(o_na), host(o_ws))
        np.testing.assert_array_equal(host(l_na), host(l_ws))
        want, want_lse = oracle.sparse_attn_decode(q, rpos, kc, vc, sel, cnt, ts)
        assert_close_out(host(o_na), want, dtype)
        np.testing.assert_allclose(host(l_na), want_lse, rtol=1e-5, atol=1e-4)
