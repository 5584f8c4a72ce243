"""Shared test helpers: host <-> device copies and the selection-parity rule."""
from __future__ import annotations

import numpy as np


def dev(arr, dtype_name: str):
    """numpy storage array (uint16 bf16 bits or float32 / int32) -> CUDA tensor."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.cuda()


def host(t) -> np.ndarray:
    """CUDA tensor -> numpy (bf16 as uint16 bit patterns)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_float(arr) -> np.ndarray:
    a = np.asarray(arr)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def check_selection(gpu_sel, gpu_cnt, ora_sel, ora_cnt, ora_raw, exact: bool, rel=1e-3, floor=1e-6):
    """Selection parity: identical sets, except (unless `exact`) swaps between
    blocks whose oracle scores both lie within rel*|s_k| (+ floor*max|s|) of
    the oracle's k-th score s_k.  Returns the number of near-tie swaps."""
    gpu_sel, ora_sel = np.asarray(gpu_sel), np.asarray(ora_sel)
    swaps = 0
    for r in range(ora_sel.shape[0]):
        assert int(gpu_cnt[r]) == int(ora_cnt[r]), f"row {r}: count {gpu_cnt[r]} != {ora_cnt[r]}"
        n = int(ora_cnt[r])
        g = gpu_sel[r]
        assert np.all(g[n:] == -1), f"row {r}: padding"
        assert np.all(np.diff(g[:n]) > 0), f"row {r}: not strictly ascending"
        G, O = set(g[:n].tolist()), set(ora_sel[r, :n].tolist())
        if G == O:
            continue
        assert not exact, f"row {r}: selection differs on exact inputs: {sorted(G ^ O)[:10]}"
        raw = ora_raw[r]
        s_k = min(raw[b] for b in O)
        tol = rel * abs(s_k) + floor * np.nanmax(np.abs(raw))
        for b in G ^ O:
            assert abs(raw[b] - s_k) <= tol, (f"row {r}: block {b} score {raw[b]} vs k-th {s_k} "
                                              f"(tol {tol})")
        swaps += len(G ^ O) // 2
    return swaps


def assert_close_out(got, want, dtype_name: str):
    """Attention output tolerance: bf16 2e-2 abs + 1e-2 rel; fp32 1e-4."""
    g, w = as_float(got), as_float(want)
    if dtype_name == "bf16":
        np.testing.assert_allclose(g, w, atol=2e-2, rtol=1e-2)
    else:
        np.testing.assert_allclose(g, w, atol=1e-4, rtol=1e-4)
