"""Seeded synthetic inputs for the QSA hot path.

This module holds only random draws and data layout: none of the method's
arithmetic (no pooling, rotation, scoring, selection or attention).  Both the
GPU path's tests/benchmark and the CPU oracle read the same arrays from here.

Distributions (all from ``numpy.random.Generator(PCG64(seed))``, drawn in a
fixed order):

* raw indexer keys, indexer queries, attention q/K/V: N(0, 1) in fp32, then
  rounded to bf16 (round-to-nearest-even) for bf16 workloads;
* planted blocks use a direction ``d`` supported on dims 60..63, the first
  halves of the four slowest rotary pairs (j = 60..63 with pairs (j, j+64)).
  Those pairs turn by at most ~0.3 rad over a 1M-token distance at
  theta = 1e7, so a planted key stays aligned with every query whatever the
  two positions are.  Every indexer query gets ``+ beta * d``; a planted
  block's four raw keys are ``gamma * d`` (plus small noise for needles).

Workloads (sizes as in the five benchmark configurations):

* ``decode-8k-f32``   4 seq x 1 row, 8,192-token context, fp32, Hq 8 / Hkv 1,
                      16 needles per sequence;
* ``prefill-32k``     one 32,768-token causal prefill, bf16, Hq 16 / Hkv 2,
                      64 broad planted blocks;
* ``decode-128k``     32 seq x 1 row, 131,072-token context, bf16, Hq 8 / Hkv 1,
                      16 needles per sequence;
* ``chunk-256k``      an 8,192-row chunk at the end of a 262,144-token context,
                      bf16, Hq 8 / Hkv 1, 96 runs of 8 adjacent planted blocks
                      with per-run amplitude;
* ``decode-1m-draft`` 4 seq x 4 draft rows sharing one selection, 1,048,576-
                      token context, bf16, Hq 8 / Hkv 1, 512 needles per
                      sequence (the selected set is known in advance).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DIM = 128
IDX_HEADS = 4
BLOCK = 4
PLANT_DIMS = (60, 61, 62, 63)
BETA = 4.0           # query component along d
GAMMA_NEEDLE = 16.0  # needle key amplitude along d
NEEDLE_NOISE = 0.1   # std of the needle keys' noise
GAMMA_BROAD = 12.0   # broad planted block amplitude


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def plant_direction() -> np.ndarray:
    d = np.zeros(DIM, np.float32)
    d[list(PLANT_DIMS)] = 0.5  # unit norm
    return d


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    kind: str            # "decode" or "prefill"
    dtype: str           # "bf16" or "f32"
    batch: int
    ctx: int             # tokens with indexer keys and K/V before the query rows
    Hq: int
    Hkv: int
    q_per_seq: int = 1   # decode rows per sequence
    draft: bool = False  # decode rows sit after the context and share one selection
    chunk: int = 0       # prefill rows (the last `chunk` tokens of the context)
    plant: str = "needle"
    n_plant: int = 16
    run_len: int = 1
    seed: int = 1000
    top_k: int = 512
    theta: float = 1.0e7
    D: int = 128

    @property
    def kv_len(self) -> int:
        return self.ctx + (self.q_per_seq if self.draft else 0)

    @property
    def n_blocks(self) -> int:
        return self.ctx // BLOCK

    @property
    def rows(self) -> int:
        """Query rows that run the indexer (anchors for decode)."""
        return self.batch if self.kind == "decode" else self.chunk

    @property
    def attn_rows(self) -> int:
        return self.batch * self.q_per_seq if self.kind == "decode" else self.chunk


SPECS = {
    "decode-8k-f32": Spec("decode-8k-f32", "decode", "f32", batch=4, ctx=8192, Hq=8, Hkv=1,
                          plant="needle", n_plant=16, seed=1001),
    "prefill-32k": Spec("prefill-32k", "prefill", "bf16", batch=1, ctx=32768, Hq=16, Hkv=2,
                        chunk=32768, plant="broad", n_plant=64, seed=1002),
    "decode-128k": Spec("decode-128k", "decode", "bf16", batch=32, ctx=131072, Hq=8, Hkv=1,
                        plant="needle", n_plant=16, seed=1003),
    "chunk-256k": Spec("chunk-256k", "prefill", "bf16", batch=1, ctx=262144, Hq=8, Hkv=1,
                       chunk=8192, plant="runs", n_plant=96, run_len=8, seed=1004),
    "decode-1m-draft": Spec("decode-1m-draft", "decode", "bf16", batch=4, ctx=1048576, Hq=8,
                            Hkv=1, q_per_seq=4, draft=True, plant="needle", n_plant=512,
                            seed=1005),
}
# The five benchmark configurations, in order.
CONFIG_ORDER = ["decode-8k-f32", "prefill-32k", "decode-128k", "chunk-256k", "decode-1m-draft"]


def scaled(name: str, **overrides) -> Spec:
    """A smaller copy of a workload (tests): override ctx, batch, chunk, ..."""
    return dataclasses.replace(SPECS[name], **overrides)


def _normal(rng, shape, chunk_elems=1 << 26) -> np.ndarray:
    """N(0,1) float32 of `shape`, drawn in fixed-size pieces (bounded memory)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for i in range(0, n, chunk_elems):
        m = min(chunk_elems, n - i)
        out[i:i + m] = rng.standard_normal(m, dtype=np.float32)
    return out.reshape(shape)


def _normal_dtype(rng, shape, dtype: str) -> np.ndarray:
    """N(0,1) in the workload's storage format (uint16 bf16 bits or float32)."""
    if dtype == "f32":
        return _normal(rng, shape)
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    piece = 1 << 26
    for i in range(0, n, piece):
        m = min(piece, n - i)
        out[i:i + m] = bf16_bits(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else bf16_bits(x)


def _from_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else bf16_to_f32(x)


def _pick_runs(rng, n_blocks: int, n_runs: int, run_len: int, lo: int = 0) -> np.ndarray:
    """Start blocks of `n_runs` non-overlapping runs of `run_len` blocks in [lo, n_blocks)."""
    taken = np.zeros(n_blocks, bool)
    starts = []
    while len(starts) < n_runs:
        s = int(rng.integers(lo, n_blocks - run_len + 1))
        if not taken[max(0, s - 1):s + run_len + 1].any():
            taken[s:s + run_len] = True
            starts.append(s)
    return np.array(sorted(starts), np.int64)


def make(spec: Spec, seed: Optional[int] = None) -> dict:
    """Draw every input of one workload.  Returns a dict of numpy arrays:

    raw_keys [B][ctx][128], idx_q [rows][4][128], row_seq [rows], row_pos [rows],
    q (decode: [B][Qn][Hq][D]; prefill: [rows][Hq][D]), attn_pos (decode:
    [B][Qn]), k_cache / v_cache [B][kv_len][Hkv][D], tail_start ([B] or None),
    planted [B][n] (planted block ids per sequence), plus the Spec.
    bf16 tensors are uint16 bit patterns.
    """
    rng = np.random.Generator(np.random.PCG64(spec.seed if seed is None else seed))
    B, L, dt = spec.batch, spec.ctx, spec.dtype
    d = plant_direction()
    nb = spec.n_blocks
    out = {"spec": spec}

    # raw indexer keys and their planted blocks
    raw = _normal_dtype(rng, (B, L, DIM), dt)
    planted = []
    for s in range(B):
        if spec.plant == "needle":
            # needles among the blocks visible to the last context token
            blocks = np.sort(rng.choice(nb, size=spec.n_plant, replace=False)).astype(np.int64)
            noise = rng.standard_normal((spec.n_plant, BLOCK, DIM), dtype=np.float32) * NEEDLE_NOISE
            vals = GAMMA_NEEDLE * d[None, None, :] + noise
            for i, b in enumerate(blocks):
                raw[s, BLOCK * b:BLOCK * b + BLOCK] = _to_storage(vals[i], dt)
        elif spec.plant == "broad":
            blocks = np.sort(rng.choice(nb, size=spec.n_plant, replace=False)).astype(np.int64)
            for b in blocks:
                raw[s, BLOCK * b:BLOCK * b + BLOCK] = _to_storage(
                    np.tile(GAMMA_BROAD * d, (BLOCK, 1)), dt)
        elif spec.plant == "runs":
            starts = _pick_runs(rng, nb, spec.n_plant, spec.run_len)
            amps = rng.uniform(2.5, 3.5, size=spec.n_plant) * 4.0
            blocks = []
            for st, a in zip(starts, amps):
                key = _to_storage(np.tile((a * d).astype(np.float32), (BLOCK * spec.run_len, 1)), dt)
                raw[s, BLOCK * st:BLOCK * (st + spec.run_len)] = key
                blocks.extend(range(st, st + spec.run_len))
            blocks = np.array(blocks, np.int64)
        else:
            blocks = np.zeros(0, np.int64)
        planted.append(blocks)
    out["raw_keys"] = raw
    out["planted"] = planted

    # indexer queries: N(0,1) + beta * d for every row and head
    rows = spec.rows
    iq = _normal(rng, (rows, IDX_HEADS, DIM)) + BETA * d[None, None, :]
    out["idx_q"] = _to_storage(iq, dt)
    if spec.kind == "decode":
        out["row_seq"] = np.arange(B, dtype=np.int32)
        out["row_pos"] = np.full(B, L - 1, np.int32)  # anchor: the last context token
        qn = spec.q_per_seq
        out["q"] = _normal_dtype(rng, (B, qn, spec.Hq, spec.D), dt)
        if spec.draft:
            out["attn_pos"] = (L + np.tile(np.arange(qn, dtype=np.int32), (B, 1))).astype(np.int32)
            out["tail_start"] = np.full(B, L, np.int32)
        else:
            assert qn == 1
            out["attn_pos"] = np.full((B, 1), L - 1, np.int32)
            out["tail_start"] = None
    else:
        assert B == 1 and 0 < spec.chunk <= L
        out["row_seq"] = np.zeros(rows, np.int32)
        out["row_pos"] = (L - spec.chunk + np.arange(rows)).astype(np.int32)
        out["q"] = _normal_dtype(rng, (rows, spec.Hq, spec.D), dt)
        out["attn_pos"] = None
        out["tail_start"] = None
    out["k_cache"] = _normal_dtype(rng, (B, spec.kv_len, spec.Hkv, spec.D), dt)
    out["v_cache"] = _normal_dtype(rng, (B, spec.kv_len, spec.Hkv, spec.D), dt)
    return out


def paged_slots(rng, batch: int, length: int, page_tokens: int = 16) -> np.ndarray:
    """Physical KV slots [batch][length] of a paged pool: each request's
    token t sits in page pages[r][t // page_tokens] at offset
    t % page_tokens; the pages of all requests are a random permutation of
    batch * ceil(length / page_tokens) pages.  page_tokens is a multiple of
    4, so the 4 tokens of a block share a page (page-aligned slots)."""
    assert page_tokens % BLOCK == 0
    npg = (length + page_tokens - 1) // page_tokens
    pages = rng.permutation(batch * npg).reshape(batch, npg).astype(np.int64)
    t = np.arange(length, dtype=np.int64)
    return pages[:, t // page_tokens] * page_tokens + (t % page_tokens)[None, :]


def page_table(rng, batch: int, length: int, page_tokens: int = 16, spare_pages: int = 0) -> np.ndarray:
    """Page table [batch][ceil(length / page_tokens)] int32 of a paged pool:
    logical page j of request r is physical page table[r][j]; the pages are a
    random choice of distinct pages among batch * npages + spare_pages (the
    rest stay unused).  Token t of request r is slot table[r][t // P] * P +
    t % P."""
    assert page_tokens % BLOCK == 0
    npg = (length + page_tokens - 1) // page_tokens
    pages = rng.permutation(batch * npg + spare_pages)[: batch * npg]
    return pages.reshape(batch, npg).astype(np.int32)


def to_float(x: np.ndarray, spec: Spec) -> np.ndarray:
    """Storage format -> float32 values."""
    return _from_storage(x, spec.dtype)
