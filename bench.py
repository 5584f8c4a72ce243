"""Throughput of the QSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--decode-workload NAME|none] [--no-cpu-baseline]
                    [--copy-calibration]
    python bench.py --rocprof-summary DIR [DIR ...]
    python bench.py --traffic-summary FETCH_DIR WRITE_DIR --workload NAME

Prints ONE JSON line.  The headline is prefill: one step is a whole pass of
the prefill path (pool the chunk's new blocks -> rotate index queries, score,
top-512 -> sparse attention) over the 8,192-token chunk at the end of a
262,144-token context; `value` is chunk tokens per second.  The decode
workload (4 sequences x 4 draft rows sharing one selection at 1,048,576
tokens) is timed in the same run and reported under "decode" in query rows
per second.  Inputs are seeded synthetic tensors resident in HBM before the
timed region; decode rotates three copies of its pooled keys and K/V so the
256 MiB Infinity Cache cannot serve a step from the previous one.

"roofline" is the dominant kernel's achieved rate (algorithmic flops or bytes
per launch / its average duration, from hipEvents the library records around
each launch on the launch stream) against MI355X's datasheet peak.
"cpu_baseline" is the CPU oracle, untuned, timed on a bounded sample of the
same workload on this host.

"traffic" is the kernel's measured memory traffic per launch (bytes L2 fetched
plus wrote, from rocprofv3's FETCH_SIZE and WRITE_SIZE counters scaled by what
the same counters read for a copy of known size), taken from
profiles/hbm_traffic_<workload>.txt, and null when the kernel's source has
changed since those counters were taken.  The two summary modes reduce
rocprofv3 CSV output (``--output-format csv -o run``) to those text files.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QSA prefill tokens/s @256K + decode queries/s @1M; % of HBM/MFMA peak"
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, datasheet
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA, datasheet
PEAK_F32_VALU_TFLOPS = 157.3
DIM = 128


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def to_dev(a):
    import torch
    if isinstance(a, torch.Tensor):   # drawn on the device already
        return a
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
    return t.cuda()


# ---------------------------------------------------------------------------
# algorithmic work per launch (what the method must compute / move)
# ---------------------------------------------------------------------------

def visible(t):
    return (np.asarray(t, np.int64) + 1) // 4


def positions_per_row(nc, t, k, tail_start=None):
    nc = np.asarray(nc, np.int64)
    t = np.asarray(t, np.int64)
    ts = 4 * nc if tail_start is None else np.asarray(tail_start, np.int64)
    return 4 * np.minimum(nc, k) + np.maximum(t - ts + 1, 0)


def prefill_work(spec, row_pos):
    eb = 2 if spec.dtype == "bf16" else 4
    nc = visible(row_pos)
    pairs = int(nc.sum())
    npos = positions_per_row(nc, row_pos, spec.top_k)
    new_blocks = spec.chunk // 4
    return {
        "pool_rope": ("hbm", new_blocks * (4 + 1) * DIM * eb, "B"),
        "score_rows_bf16": ("hbm", float(pairs) * DIM * eb, "B"),
        "select_rows": ("hbm", 4.0 * pairs, "B"),   # scans the fp32 scores once
        "attn_prefill": ("alu", 4.0 * spec.Hq * spec.D * float(npos.sum()), "flop"),
        "attn_prefill_mfma": ("mfma", 4.0 * spec.Hq * spec.D * float(npos.sum()), "flop"),
        "attn_prefill_mfma_d256": ("mfma", 4.0 * spec.Hq * spec.D * float(npos.sum()), "flop"),
        "attn_prefill_mfma_fp8kv": ("mfma", 4.0 * spec.Hq * spec.D * float(npos.sum()), "flop"),
        "score_filter": ("mfma", 2.0 * 4 * DIM * pairs, "flop"),
        "score_filter_fp8": ("mfma", 2.0 * 4 * DIM * pairs, "flop"),
        "pool_rope_fp8": ("hbm", new_blocks * (4 * DIM * eb + DIM + 4), "B"),
    }, pairs, float(npos.sum())


def decode_work(spec, anchor_pos, attn_pos, tail_start):
    eb = 2 if spec.dtype == "bf16" else 4
    nc = visible(anchor_pos)
    pairs = int(nc.sum())
    # K and V rows of each sequence's positions, read once per sequence
    kv_bytes = 0.0
    for s in range(spec.batch):
        P = 4 * min(int(nc[s]), spec.top_k)
        ts = int(tail_start[s]) if tail_start is not None else 4 * int(visible(attn_pos[s]).min())
        P += max(int(np.max(attn_pos[s])) - ts + 1, 0)
        kv_bytes += 2.0 * P * spec.Hkv * spec.D * eb
    q_bytes = 2.0 * spec.batch * spec.q_per_seq * spec.Hq * spec.D * eb
    kind = "score_rows_bf16" if spec.dtype == "bf16" else "score_rows_f32"
    return {
        kind: ("hbm", float(pairs) * DIM * eb, "B"),
        "score_rows_fp8": ("hbm", float(pairs) * (DIM + 4), "B"),   # codes and the scale of each key
        "select_rows": ("hbm", 4.0 * pairs, "B"),
        "select_collect": ("hbm", 4.0 * pairs, "B"),
        "select_final": ("hbm", 8.0 * spec.batch * spec.top_k, "B"),
        "attn_decode": ("hbm", kv_bytes + q_bytes, "B"),
        "attn_decode_mfma": ("hbm", kv_bytes + q_bytes, "B"),
        "attn_decode_mfma_d256": ("hbm", kv_bytes + q_bytes, "B"),
        "attn_decode_mfma_fp8kv": ("hbm", kv_bytes / eb + q_bytes, "B"),   # one byte per K/V element
    }, pairs


def _rate(work, ms):
    bound, amount, unit = work
    if unit == "flop":
        return amount / (ms * 1e-3) / 1e12, (PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_F32_VALU_TFLOPS), "TFLOP/s"
    return amount / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"


def roofline_for(name, work, kt_entry, traffic=None, trace=None):
    """kt_entry: kernel_times()'s record of the kernel.  `achieved` uses the
    mean launch time; the median / p10 / p90 launch times are reported with
    it, and the committed rocprofv3 trace's mean when one matches the
    kernel's current source (trace_avg_us, trace_frac)."""
    bound, amount, unit = work
    avg_ms, per_step = kt_entry[1], kt_entry[3]
    achieved, peak, u = _rate(work, avg_ms)
    r = {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": u,
         "frac": round(achieved / peak, 4), "per_launch": amount, "avg_us": round(avg_ms * 1e3, 2),
         "median_us": round(pct(per_step, 50) * 1e3, 2), "p10_us": round(pct(per_step, 10) * 1e3, 2),
         "p90_us": round(pct(per_step, 90) * 1e3, 2), "traffic": (traffic or {}).get(name)}
    if trace and name in trace:
        t_avg = trace[name]
        r["trace_avg_us"] = round(t_avg, 2)
        r["trace_frac"] = round(_rate(work, t_avg * 1e-3)[0] / peak, 4)
    return r


def pct(v, q):
    return float(np.percentile(np.asarray(v, np.float64), q))


def kernel_times(run_step, nsteps, names):
    """Per-kernel launch times over `nsteps` steps, from the hipEvents the
    library records around each launch on its launch stream.  Returns
    {kernel: (launches, mean ms per launch, ms per step, [per-step mean ms
    per launch])}; the list gives the median / p10 / p90."""
    import torch
    from block_sparse_long_amd import qsa
    torch.cuda.synchronize()
    per = {}
    for i in range(nsteps):
        qsa.profile_reset()
        qsa.profile_enable(True)
        run_step(i)
        torch.cuda.synchronize()
        qsa.profile_enable(False)
        for n in names:
            cnt, tot = qsa.profile_kernel_ms(n)
            if cnt:
                per.setdefault(n, []).append((cnt, tot))
    qsa.profile_reset()
    out = {}
    for n, v in per.items():
        c = sum(x[0] for x in v)
        t = sum(x[1] for x in v)
        out[n] = (c, t / c, t / nsteps, [x[1] / x[0] for x in v])
    return out


def kernel_table(kt, nsteps):
    return {n: {"launches_per_step": c / nsteps, "avg_us": round(a * 1e3, 2),
                "median_us": round(pct(v, 50) * 1e3, 2), "p10_us": round(pct(v, 10) * 1e3, 2),
                "p90_us": round(pct(v, 90) * 1e3, 2)}
            for n, (c, a, _, v) in kt.items()}


def step_times(run_step, n, offset=0):
    """Per-step durations (ms) of `n` steps, each bracketed by events on the
    current stream (the one the library launches on): median, p10, p90."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record()
        run_step(offset + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) for a, b in ev]
    return {"n": n, "median_ms": round(pct(d, 50), 4), "p10_ms": round(pct(d, 10), 4),
            "p90_ms": round(pct(d, 90), 4), "mean_ms": round(float(np.mean(d)), 4)}


def timed(run_step, steps, warmup):
    import torch
    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


ALL_KERNELS = ["pool_rope", "pool_rope_fp8", "pool_append", "rope_query", "score_rows_bf16", "score_rows_f32",
               "score_rows_fp8", "select_rows", "select_collect", "select_final", "score_sample",
               "score_sample_fp8", "sample_threshold", "score_filter", "score_filter_fp8", "select_merge",
               "attn_prefill_mfma", "attn_decode_mfma", "attn_prefill_mfma_d256", "attn_decode_mfma_d256",
               "attn_prefill_mfma_fp8kv", "attn_decode_mfma_fp8kv",
               "attn_prefill", "attn_decode", "attn_combine"]


# ---------------------------------------------------------------------------
# prefill workload
# ---------------------------------------------------------------------------

def bench_prefill(spec, steps, warmup, cpu_baseline, keys="bf16", w=None, kv="bf16", cpu_target_s=12.0):
    """keys "fp8": the compressed keys stored as E4M3 codes plus one scale per
    key (qsa_pool_index_keys_fp8 / qsa_score_topk_fp8); kv "fp8": the K/V
    cache as E4M3 codes with one scale per tensor (qsa_sparse_attn_*_fp8kv);
    everything else as with bf16."""
    import torch
    from block_sparse_long_amd import qsa, synth
    if w is None:
        t0 = time.perf_counter()
        w = synth.make(spec)
        log(f"{spec.name}: inputs drawn in {time.perf_counter() - t0:.1f}s")
    L, nb, k = spec.ctx, spec.n_blocks, spec.top_k
    first_new = (L - spec.chunk) // 4
    raw = to_dev(w["raw_keys"])
    fp8 = keys == "fp8"
    if fp8:
        codes = torch.zeros((1, nb, DIM), dtype=torch.uint8, device="cuda")
        scales = torch.zeros((1, nb), dtype=torch.float32, device="cuda")
        if first_new > 0:
            qsa.pool_index_keys_fp8(raw, codes, scales, 0, first_new, spec.theta)
    else:
        pooled = torch.zeros((1, nb, DIM), dtype=raw.dtype, device="cuda")
        if first_new > 0:  # the context before the chunk is already pooled
            qsa.pool_index_keys(raw, pooled, 0, first_new, spec.theta)
    iq, seq, pos = to_dev(w["idx_q"]), to_dev(w["row_seq"]), to_dev(w["row_pos"])
    q, kc, vc = to_dev(w["q"]), to_dev(w["k_cache"]), to_dev(w["v_cache"])
    fp8kv = kv == "fp8"
    if fp8kv:
        (kc, ks), (vc, vs) = quantize_kv(kc), quantize_kv(vc)
    R = spec.chunk
    max_nb = L // 4
    sel = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    ws = torch.empty((max(qsa.score_topk_workspace_size(R, max_nb, k, qsa.BF16), 256),), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((R, spec.Hq), dtype=torch.float32, device="cuda")

    def step(_i):
        if fp8:
            qsa.pool_index_keys_fp8(raw, codes, scales, first_new, nb, spec.theta)
            qsa.score_topk_fp8(iq, seq, pos, codes, scales, max_nb, k, spec.theta, sel_blocks=sel, sel_count=cnt,
                               workspace=ws, want_scores=False)
        else:
            qsa.pool_index_keys(raw, pooled, first_new, nb, spec.theta)
            qsa.score_topk(iq, seq, pos, pooled, max_nb, k, spec.theta, sel_blocks=sel, sel_count=cnt,
                           workspace=ws, want_scores=False)
        if fp8kv:
            qsa.sparse_attn_prefill_fp8kv(q, seq, pos, kc, vc, ks, vs, sel, cnt, out=out, lse=lse)
        else:
            qsa.sparse_attn_prefill(q, seq, pos, kc, vc, sel, cnt, out=out, lse=lse)

    ms = timed(step, steps, warmup)
    log(f"{spec.name} ({keys} keys, {kv} K/V): {ms:.3f} ms/step")
    st = step_times(step, max(30, steps))
    nprof = max(10, min(steps, 30))
    kt = kernel_times(step, nprof, ALL_KERNELS)
    work, pairs, npos = prefill_work(spec, w["row_pos"])
    kernels = kernel_table(kt, nprof)
    dom = max((n for n in kt if n in work), key=lambda n: kt[n][2])
    tr, trc = load_traffic(spec.name), load_trace(spec.name)
    res = {"ms_per_step": ms, "value": R / (ms * 1e-3), "step_ms": st, "kernels": kernels,
           "roofline": roofline_for(dom, work[dom], kt[dom], tr, trc),
           "rooflines": {n: roofline_for(n, work[n], kt[n], tr, trc) for n in kt if n in work},
           "pairs": pairs, "positions": npos}
    if cpu_baseline:
        res["cpu_baseline"] = cpu_prefill(spec, w, cpu_target_s)
    res["_inputs"] = w
    return res


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_prefill(spec, w, target_s=12.0):
    import oracle
    L, nb, k = spec.ctx, spec.n_blocks, spec.top_k
    first_new = (L - spec.chunk) // 4
    pooled = np.zeros((1, nb, DIM), w["raw_keys"].dtype)
    if first_new:  # the context before the chunk (not part of a step)
        oracle.pool(w["raw_keys"], 0, first_new, spec.theta, pooled=pooled)
    t0 = time.perf_counter()
    oracle.pool(w["raw_keys"], first_new, nb, spec.theta, pooled=pooled)
    t_pool = time.perf_counter() - t0

    def rows_time(rows):
        t = time.perf_counter()
        s, c, _, _ = oracle.score_topk(w["idx_q"][rows], w["row_seq"][rows], w["row_pos"][rows], pooled, k,
                                       spec.theta)
        oracle.sparse_attn_prefill(w["q"][rows], w["row_seq"][rows], w["row_pos"][rows], w["k_cache"],
                                   w["v_cache"], s, c)
        return time.perf_counter() - t

    R = spec.chunk
    n0 = max(oracle.threads(), 8)
    probe = np.linspace(R - 1, R // 2, n0).astype(np.int64)   # the heaviest (latest) rows
    tp = rows_time(probe)
    n = int(min(R, max(n0, n0 * target_s / max(tp, 1e-3))))
    rows = np.unique(np.linspace(0, R - 1, n).astype(np.int64))
    t = rows_time(rows)
    per_step = t_pool + t * R / len(rows)
    return {"value": R / per_step, "unit": "tokens/s", "cores": oracle.threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"pool of the chunk's {spec.chunk // 4} new blocks, then score/top-{k} and attention for "
                      f"{len(rows)} of {R} rows spread over the chunk ({t_pool + t:.1f}s); per-step time "
                      f"extrapolated to all rows"}


# ---------------------------------------------------------------------------
# decode workload
# ---------------------------------------------------------------------------

def bench_decode(spec, steps, warmup, cpu_baseline, copies=3, keys="bf16", w=None, kv="bf16", cpu_target_s=10.0):
    """keys / kv "fp8": as in bench_prefill."""
    import torch
    from block_sparse_long_amd import qsa, synth
    if w is None:
        t0 = time.perf_counter()
        w = synth.make(spec)
        log(f"{spec.name}: inputs drawn in {time.perf_counter() - t0:.1f}s")
    B, nb, k = spec.batch, spec.n_blocks, spec.top_k
    fp8 = keys == "fp8"
    raw = to_dev(w["raw_keys"])
    pooled_h = None
    if fp8:   # built before timing
        codes0 = torch.zeros((B, nb, DIM), dtype=torch.uint8, device="cuda")
        scales0 = torch.zeros((B, nb), dtype=torch.float32, device="cuda")
        qsa.pool_index_keys_fp8(raw, codes0, scales0, 0, nb, spec.theta)
        pooled0 = None
    else:
        pooled0 = torch.zeros((B, nb, DIM), dtype=raw.dtype, device="cuda")
        qsa.pool_index_keys(raw, pooled0, 0, nb, spec.theta)   # built before timing
        if cpu_baseline:
            pooled_h = pooled0[:1].cpu()
    del raw
    kc0, vc0 = to_dev(w["k_cache"]), to_dev(w["v_cache"])
    fp8kv = kv == "fp8"
    if fp8kv:
        (kc0, ks), (vc0, vs) = quantize_kv(kc0), quantize_kv(vc0)
    if fp8:
        kcodes = [codes0] + [codes0.clone() for _ in range(copies - 1)]
        kscales = [scales0] + [scales0.clone() for _ in range(copies - 1)]
    else:
        pooled = [pooled0] + [pooled0.clone() for _ in range(copies - 1)]
    kcs = [kc0] + [kc0.clone() for _ in range(copies - 1)]
    vcs = [vc0] + [vc0.clone() for _ in range(copies - 1)]
    iq, seq, apos = to_dev(w["idx_q"]), to_dev(w["row_seq"]), to_dev(w["row_pos"])
    q, rpos = to_dev(w["q"]), to_dev(w["attn_pos"])
    ts = None if w["tail_start"] is None else to_dev(w["tail_start"])
    max_nb = int(visible(w["row_pos"]).max())
    dcode = qsa.BF16 if spec.dtype == "bf16" else qsa.F32
    sel = torch.empty((B, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty((max(qsa.score_topk_workspace_size(B, max_nb, k, dcode), 256),), dtype=torch.uint8,
                     device="cuda")
    wsa = torch.empty((max(qsa.sparse_attn_decode_workspace_size(B, spec.q_per_seq, spec.Hq, spec.D, k), 256),),
                      dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((B, spec.q_per_seq, spec.Hq), dtype=torch.float32, device="cuda")

    def step(i):
        c = i % copies
        if fp8:
            qsa.score_topk_fp8(iq, seq, apos, kcodes[c], kscales[c], max_nb, k, spec.theta, sel_blocks=sel,
                               sel_count=cnt, workspace=ws, want_scores=False)
        else:
            qsa.score_topk(iq, seq, apos, pooled[c], max_nb, k, spec.theta, sel_blocks=sel, sel_count=cnt,
                           workspace=ws, want_scores=False)
        if fp8kv:
            qsa.sparse_attn_decode_fp8kv(q, rpos, kcs[c], vcs[c], ks, vs, sel, cnt, ts, out=out, lse=lse,
                                         workspace=wsa)
        else:
            qsa.sparse_attn_decode(q, rpos, kcs[c], vcs[c], sel, cnt, ts, out=out, lse=lse, workspace=wsa)

    ms = timed(step, steps, warmup)
    log(f"{spec.name} ({keys} keys, {kv} K/V): {ms:.3f} ms/step")
    st = step_times(step, max(30, min(steps, 100)))
    nprof = max(10, min(steps, 30))
    kt = kernel_times(step, nprof, ALL_KERNELS)
    work, pairs = decode_work(spec, w["row_pos"], w["attn_pos"], w["tail_start"])
    kernels = kernel_table(kt, nprof)
    dom = max((n for n in kt if n in work), key=lambda n: kt[n][2])
    rows = spec.batch * spec.q_per_seq
    tr, trc = load_traffic(spec.name), load_trace(spec.name)
    res = {"workload": spec.name, "value": rows / (ms * 1e-3), "unit": "query rows/s", "ms_per_step": ms,
           "step_ms": st, "kernels": kernels, "roofline": roofline_for(dom, work[dom], kt[dom], tr, trc),
           "rooflines": {n: roofline_for(n, work[n], kt[n], tr, trc) for n in kt if n in work}}
    if not fp8 and not fp8kv:
        res["pool_append"] = bench_pool_append(spec)
    if not fp8 and not fp8kv and spec.draft:
        res["draft_loop"] = bench_draft_loop(spec, iq, seq, apos, pooled, kcs, vcs, q, ts, max_nb, ws,
                                             max(steps, 10), warmup)
    if cpu_baseline and not fp8 and not fp8kv:
        res["cpu_baseline"] = cpu_decode(spec, w, pooled_h, cpu_target_s)
    res["_inputs"] = w
    return res


def quantize_kv(x):
    """bf16 cache on the device -> (E4M3 codes as uint8, per-tensor scale
    amax / 448), converted by torch's float8_e4m3fn (OCP E4M3, nearest-even)."""
    import torch
    amax = float(x.abs().max().float().item())
    scale = amax / 448.0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    flat_x, flat_c = x.view(-1), codes.view(-1)
    step = 1 << 28                                  # bounded fp32 temporaries
    for i in range(0, flat_x.numel(), step):
        flat_c[i:i + step] = (flat_x[i:i + step].float() / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def serving_shape_inputs(spec, w, Hq=24, Hkv=2, D=256, seed=2024):
    """The workload's index inputs with attention at the serving head layout
    (24 query heads over 2 KV heads, head dim 256): q, K and V are drawn
    N(0,1) in bf16 on the device from a seeded generator (a host draw of the
    1M-token caches would take minutes); the index side is unchanged."""
    import dataclasses
    import torch
    s2 = dataclasses.replace(spec, Hq=Hq, Hkv=Hkv, D=D)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    w2 = dict(w)
    B, L = spec.batch, spec.kv_len
    qshape = (B, spec.q_per_seq, Hq, D) if spec.kind == "decode" else (spec.chunk, Hq, D)
    w2["q"] = torch.randn(qshape, generator=g, device="cuda", dtype=torch.bfloat16)
    w2["k_cache"] = torch.randn((B, L, Hkv, D), generator=g, device="cuda", dtype=torch.bfloat16)
    w2["v_cache"] = torch.randn((B, L, Hkv, D), generator=g, device="cuda", dtype=torch.bfloat16)
    return s2, w2


def bench_draft_loop(spec, iq, seq, apos, pooled, kcs, vcs, q, ts, max_nb, ws, steps, warmup):
    """The IndexShare draft loop: the anchor selects once, then each of the N
    draft steps attends with one row per sequence (position ctx + i) over the
    shared selection plus the positions drafted since, and appends the
    drafted token's raw index key to the ring (completing a block at the last
    step).  One loop = 1 selection + N one-row attention calls + N appends;
    rows/s counts the N x batch draft rows."""
    import torch
    from block_sparse_long_amd import qsa
    B, N, L, k = spec.batch, spec.q_per_seq, spec.ctx, spec.top_k
    copies = len(pooled)
    qs = [q[:, i:i + 1].contiguous() for i in range(N)]
    ps = [torch.full((B, 1), L + i, dtype=torch.int32, device="cuda") for i in range(N)]
    outs = [torch.empty_like(x) for x in qs]
    lses = [torch.empty((B, 1, spec.Hq), dtype=torch.float32, device="cuda") for _ in range(N)]
    wsa = torch.empty((max(qsa.sparse_attn_decode_workspace_size(B, 1, spec.Hq, spec.D, k), 256),),
                      dtype=torch.uint8, device="cuda")
    sel = torch.empty((B, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B,), dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    keys = torch.randn((N, B, DIM), generator=g, device="cuda").to(pooled[0].dtype)
    ring = torch.zeros((B, 4, DIM), dtype=pooled[0].dtype, device="cuda")
    comp = torch.zeros((B * (N // 4 + 2), DIM), dtype=pooled[0].dtype, device="cuda")
    tpos = [torch.full((B,), L + i, dtype=torch.int32, device="cuda") for i in range(N)]
    slots = [torch.tensor([b * 4 * (N // 4 + 2) + L % 4 + i for b in range(B)], dtype=torch.int64, device="cuda")
             for i in range(N)]

    def loop(j):
        c = j % copies
        qsa.score_topk(iq, seq, apos, pooled[c], max_nb, k, spec.theta, sel_blocks=sel, sel_count=cnt,
                       workspace=ws, want_scores=False)
        for i in range(N):
            qsa.sparse_attn_decode(qs[i], ps[i], kcs[c], vcs[c], sel, cnt, ts, out=outs[i], lse=lses[i],
                                   workspace=wsa)
            qsa.pool_append(keys[i], tpos[i], slots[i], ring, comp, spec.theta)

    ms = timed(loop, steps, warmup)
    kt = kernel_times(loop, 5, ALL_KERNELS)
    log(f"{spec.name} draft loop ({N} steps): {ms:.3f} ms/loop")
    return {"draft_steps": N, "ms_per_loop": round(ms, 4), "value": round(B * N / (ms * 1e-3), 1),
            "unit": "draft rows/s",
            "kernels": {n: {"launches_per_loop": c / 5, "avg_us": round(a * 1e3, 2)} for n, (c, a, _, _) in kt.items()}}


def paged_layout(spec, page_tokens, seed=77):
    """A shuffled page table for the workload's sequences (synth.page_table)
    and, on the device, the slot of every token and the key slot of every
    block: token p of sequence s -> table[s][p / P] * P + p % P; block b ->
    slot(4b) / 4."""
    import torch
    from block_sparse_long_amd import synth
    rng = np.random.default_rng(seed)
    table_h = synth.page_table(rng, spec.batch, spec.kv_len, page_tokens=page_tokens, spare_pages=spec.batch)
    table = torch.from_numpy(table_h).cuda()
    P, bpp = page_tokens, page_tokens // 4
    n_pages = int(table_h.max()) + 1
    p = torch.arange(spec.kv_len, device="cuda")
    tok_slot = table[:, p // P].long() * P + p % P                          # [B][kv_len]
    b = torch.arange(spec.n_blocks, device="cuda")
    key_slot = table[:, b // bpp].long() * bpp + b % bpp                   # [B][n_blocks]
    return table, n_pages, tok_slot, key_slot


def scatter_rows(x, slots, n_slots):
    """[B][n][...] -> [n_slots][...] with row (s, i) at slots[s][i]."""
    import torch
    out = torch.zeros((n_slots,) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    out.index_copy_(0, slots.reshape(-1), x.reshape((-1,) + tuple(x.shape[2:])))
    return out


def bench_paged(spec, w, steps, warmup, page_tokens=16):
    """The workload with the compressed keys and the K/V in a paged pool of
    page_tokens-token pages (qsa_*_paged): prefill pools the chunk's blocks
    straight into the pool, then scores and attends through the table; decode
    scores and attends through it.  Same inputs as the contiguous run."""
    import torch
    from block_sparse_long_amd import qsa
    table, n_pages, tok_slot, key_slot = paged_layout(spec, page_tokens)
    P, k = page_tokens, spec.top_k
    raw = to_dev(w["raw_keys"])
    B, nb = spec.batch, spec.n_blocks
    kp = scatter_rows(to_dev(w["k_cache"]), tok_slot, n_pages * P)
    vp = scatter_rows(to_dev(w["v_cache"]), tok_slot, n_pages * P)
    keys = torch.zeros((n_pages * P // 4, DIM), dtype=raw.dtype, device="cuda")
    iq, seq, pos = to_dev(w["idx_q"]), to_dev(w["row_seq"]), to_dev(w["row_pos"])
    q = to_dev(w["q"])
    dcode = qsa.BF16 if spec.dtype == "bf16" else qsa.F32
    R = iq.shape[0]
    max_nb = int(visible(w["row_pos"]).max())
    sel = torch.empty((R, k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((R,), dtype=torch.int32, device="cuda")
    ws = torch.empty((max(qsa.score_topk_workspace_size(R, max_nb, k, dcode), 256),), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    if spec.kind == "prefill":
        first_new = (spec.ctx - spec.chunk) // 4
        if first_new > 0:  # the context before the chunk, pooled before timing
            qsa.pool_index_keys_paged(raw, table, P, 0, first_new, spec.theta, pooled=keys)
        lse = torch.empty((R, spec.Hq), dtype=torch.float32, device="cuda")

        def step(_i):
            qsa.pool_index_keys_paged(raw, table, P, first_new, nb, spec.theta, pooled=keys)
            qsa.score_topk_paged(iq, seq, pos, table, P, max_nb, k, spec.theta, pooled=keys, sel_blocks=sel,
                                 sel_count=cnt, workspace=ws, want_scores=False)
            qsa.sparse_attn_prefill_paged(q, seq, pos, kp, vp, table, P, sel, cnt, out=out, lse=lse)
        rows = R
    else:
        qsa.pool_index_keys_paged(raw, table, P, 0, nb, spec.theta, pooled=keys)
        # three copies of the pools, used in turn (as in bench_decode): the
        # 268 MB of compressed keys would otherwise partly stay in the 256 MB
        # Infinity Cache between steps
        keys_c = [keys] + [keys.clone() for _ in range(2)]
        kp_c = [kp] + [kp.clone() for _ in range(2)]
        vp_c = [vp] + [vp.clone() for _ in range(2)]
        rpos = to_dev(w["attn_pos"])
        ts = None if w["tail_start"] is None else to_dev(w["tail_start"])
        lse = torch.empty((B, spec.q_per_seq, spec.Hq), dtype=torch.float32, device="cuda")
        wsa = torch.empty((max(qsa.sparse_attn_decode_workspace_size(B, spec.q_per_seq, spec.Hq, spec.D, k), 256),),
                          dtype=torch.uint8, device="cuda")

        def step(i):
            c = i % 3
            qsa.score_topk_paged(iq, seq, pos, table, P, max_nb, k, spec.theta, pooled=keys_c[c], sel_blocks=sel,
                                 sel_count=cnt, workspace=ws, want_scores=False)
            qsa.sparse_attn_decode_paged(q, rpos, kp_c[c], vp_c[c], table, P, sel, cnt, ts, out=out, lse=lse,
                                         workspace=wsa)
        rows = B * spec.q_per_seq
    ms = timed(step, steps, warmup)
    log(f"{spec.name} (paged pool, {P}-token pages): {ms:.3f} ms/step")
    nprof = max(3, min(steps, 10))
    kt = kernel_times(step, nprof, ALL_KERNELS)
    return {"page_tokens": P, "value": round(rows / (ms * 1e-3), 1),
            "unit": "tokens/s" if spec.kind == "prefill" else "query rows/s", "ms_per_step": round(ms, 4),
            "kernels": kernel_table(kt, nprof)}


def bench_pool_append(spec, launches=50):
    """Incremental decode pooling for the workload's batch: every launch
    completes a block for every request (the costlier case), with the
    compressed keys in a paged layout.  Per-launch time from the library's
    hipEvents; bytes are what the step must move (new key in, 3 ring keys
    in, ring slot and compressed key out)."""
    import torch
    from block_sparse_long_amd import qsa, synth
    B = spec.batch
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    rng = np.random.default_rng(7)
    slots = torch.from_numpy(synth.paged_slots(rng, B, 4 * launches, 16)).cuda()
    keys = torch.randn((launches, B, DIM), device="cuda").to(dt)
    ring = torch.zeros((B, 4, DIM), dtype=dt, device="cuda")
    comp = torch.zeros((int(slots.max().item()) // 4 + 1, DIM), dtype=dt, device="cuda")
    pos = torch.full((B,), spec.ctx + 3, dtype=torch.int32, device="cuda")
    fs = [slots[:, 4 * j + 3].contiguous() for j in range(launches)]
    for j in range(3):
        qsa.pool_append(keys[j], pos, fs[j], ring, comp, spec.theta)
    torch.cuda.synchronize()
    qsa.profile_reset()
    qsa.profile_enable(True)
    for j in range(launches):
        qsa.pool_append(keys[j], pos, fs[j], ring, comp, spec.theta)
    torch.cuda.synchronize()
    qsa.profile_enable(False)
    n, tot = qsa.profile_kernel_ms("pool_append")
    qsa.profile_reset()
    eb = 2 if spec.dtype == "bf16" else 4
    return {"batch": B, "avg_us": round(tot / max(n, 1) * 1e3, 2), "bytes_per_launch": B * 6 * DIM * eb,
            "bound": "latency"}


def cpu_decode(spec, w, pooled_h, target_s=10.0, max_passes=64):
    """The oracle's decode step (score/top-k of a sequence's anchor, then the
    attention of its rows), over the workload's sequences in turn until about
    target_s seconds have passed.  pooled_h holds the first sequence's pooled
    keys; the others are pooled by the oracle before timing."""
    import torch
    import oracle
    k = spec.top_k
    p = pooled_h
    first = (p.view(torch.int16).numpy().view(np.uint16) if p.dtype == torch.bfloat16 else p.numpy())
    B = spec.batch
    pooled = [first] + [oracle.pool(w["raw_keys"][s:s + 1], 0, spec.n_blocks, spec.theta) for s in range(1, B)]
    rows, passes = 0, 0
    t0 = time.perf_counter()
    while passes < max_passes:
        s = passes % B
        sl = slice(s, s + 1)
        sel, cnt, _, _ = oracle.score_topk(w["idx_q"][sl], np.zeros(1, np.int32), w["row_pos"][sl], pooled[s], k,
                                           spec.theta)
        ts = None if w["tail_start"] is None else w["tail_start"][sl]
        oracle.sparse_attn_decode(w["q"][sl], w["attn_pos"][sl], w["k_cache"][sl], w["v_cache"][sl], sel, cnt, ts)
        rows += spec.q_per_seq
        passes += 1
        if time.perf_counter() - t0 >= target_s and passes >= B:
            break
    t = time.perf_counter() - t0
    return {"value": rows / t, "unit": "query rows/s", "cores": oracle.threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": f"{passes} sequence steps over the {B} sequences (each: score/top-{k} of the anchor over "
                      f"{int(visible(w['row_pos'][0]))} blocks, then attention of its {spec.q_per_seq} rows) "
                      f"in {t:.1f}s"}


# ---------------------------------------------------------------------------
# rocprofv3 summaries and measured traffic
# ---------------------------------------------------------------------------

CSRC = os.path.join(ROOT, "block_sparse_long_amd", "csrc")
HEADERS = ["qsa_internal.h", "qsa_device.h", "qsa_wg.h"]
KERNEL_SOURCE = {"pool_rope": "pool.hip", "pool_append": "pool.hip", "rope_query": "pool.hip", "score_rows_bf16": "score.hip",
                 "score_rows_f32": "score.hip", "select_rows": "select.hip",
                 "select_collect": "select.hip", "select_final": "select.hip", "score_sample": "score_fused.hip",
                 "sample_threshold": "score_fused.hip", "score_filter": "score_fused.hip",
                 "select_merge": "score_fused.hip", "attn_prefill_mfma": "attn_mfma.hip",
                 "attn_decode_mfma": "attn_mfma.hip", "attn_prefill_mfma_d256": "attn_mfma.hip",
                 "attn_decode_mfma_d256": "attn_mfma.hip", "attn_prefill_mfma_fp8kv": "attn_mfma.hip",
                 "attn_decode_mfma_fp8kv": "attn_mfma.hip", "attn_prefill": "attn.hip", "attn_decode": "attn.hip",
                 "attn_combine": "attn.hip", "pool_rope_fp8": "pool.hip", "score_rows_fp8": "score.hip",
                 "score_sample_fp8": "score_fused.hip", "score_filter_fp8": "score_fused.hip"}
COPY_BYTES = 1 << 30
XCDS, SIMDS = 8, 256 * 4   # MI355X: 8 XCDs, 256 CUs of 4 SIMDs


def source_digest(kernel):
    """Digest of the source a kernel is built from (its file and the shared headers)."""
    h = hashlib.sha256()
    for f in [KERNEL_SOURCE[kernel]] + HEADERS:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_kernel_name(full):
    """libqsa's launch name of a kernel from its demangled rocprofv3 name, else None."""
    base = full.split("(")[0].replace("void ", "").strip()
    if not base.startswith("qsa::"):
        return "copy" if "neg_kernel" in full else None
    base = base[5:]
    tmpl = base[base.find("<"):] if "<" in base else ""
    base = base.split("<")[0]
    if base == "attn_kernel":
        return "attn_decode" if tmpl.rstrip(">").strip().endswith("true") else "attn_prefill"
    if base.startswith("attn_combine"):
        return "attn_combine"
    if base in ("score_sample_kernel", "score_filter_kernel") and tmpl.startswith("<true"):
        return base[:-7] + "_fp8"   # the FP8-key instance
    if base in ("attn_prefill_mfma_kernel", "attn_decode_mfma_kernel"):  # <head dim, K/V element>
        return base[:-7] + ("_d256" if tmpl.startswith("<256") else "") + ("_fp8kv" if "char" in tmpl else "")
    return base[:-7] if base.endswith("_kernel") else base


def copy_calibration():
    """A copy of known size for scaling memory counters: one elementwise pass
    (negation) that reads COPY_BYTES and writes COPY_BYTES, three times."""
    import torch
    src = torch.ones((COPY_BYTES // 2,), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def _csvs(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def kernel_trace_stats(d):
    """{kernel: (launches, avg_us, median_us, p10_us, p90_us, min_us, max_us)}
    from a --kernel-trace run."""
    per = {}
    for f in _csvs(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            n = short_kernel_name(r["Kernel_Name"])
            if n is None:
                continue
            per.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {n: (len(v), sum(v) / len(v), pct(v, 50), pct(v, 10), pct(v, 90), min(v), max(v))
            for n, v in per.items()}


def counter_means(d):
    """{kernel: {counter: mean value per dispatch}} from a --pmc run."""
    acc = {}
    for f in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            n = short_kernel_name(r["Kernel_Name"])
            if n is None:
                continue
            key = (n, r["Counter_Name"])
            acc.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
            acc[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    out = {}
    for (n, c), per in acc.items():
        out.setdefault(n, {})[c] = sum(per.values()) / len(per)
    return out


def rocprof_summary(dirs):
    merged = {}  # counters of every directory (one --pmc pass each), per kernel
    for d in dirs:
        for n, c in counter_means(d).items():
            merged.setdefault(n, {}).update(c)
    for d in dirs:
        print(f"# rocprofv3 output: {d}")
        st = kernel_trace_stats(d)
        if st:
            print("# kernel  name  source_digest  launches  avg_us  median_us  p10_us  p90_us  min_us  max_us")
            for n, (c, a, med, p10, p90, lo, hi) in sorted(st.items(), key=lambda x: -x[1][0] * x[1][1]):
                dg = source_digest(n) if n in KERNEL_SOURCE else "-"
                print(f"kernel {n:<24} {dg} {c:>6} {a:>10.2f} {med:>10.2f} {p10:>10.2f} {p90:>10.2f} {lo:>10.2f} "
                      f"{hi:>10.2f}")
        for f in _csvs(d, "kernel_stats.csv"):  # rocprofv3's own --stats table
            print(f"# {os.path.basename(f)}: kernel, calls, average ns, min ns, max ns")
            for r in csv.DictReader(open(f)):
                n = short_kernel_name(r["Name"]) or r["Name"][:40]
                print(f"  {n:<20} {r['Calls']:>6} {float(r['AverageNs']):>12.0f} {r['MinNs']:>10} {r['MaxNs']:>10}")
    cm = merged
    if cm:
        print("# counters  name  source_digest  counter=mean per dispatch ...  [derived]")
        print(f"# derived: mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} XCDs * {SIMDS} SIMDs); "
              "coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES; "
              "valu_per_mfma = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA")
    for n in sorted(cm):
        c = cm[n]
        dg = source_digest(n) if n in KERNEL_SOURCE else "-"
        der = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
            der.append(f"mfma_busy={c['SQ_VALU_MFMA_BUSY_CYCLES'] / (c['GRBM_GUI_ACTIVE'] / XCDS * SIMDS):.4f}")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in c and c.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            der.append(f"coexec={c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.4f}")
        if "SQ_INSTS_VALU" in c and c.get("SQ_INSTS_MFMA"):
            der.append(f"valu_per_mfma={(c['SQ_INSTS_VALU'] - c['SQ_INSTS_MFMA']) / c['SQ_INSTS_MFMA']:.3f}")
        print(f"counters {n:<20} {dg} " + "  ".join(f"{k}={v:.6g}" for k, v in sorted(c.items())) +
              ("  [" + " ".join(der) + "]" if der else ""))


def traffic_summary(fetch_dir, write_dir, workload):
    """Measured bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    scaled so that the calibration copy reads and writes COPY_BYTES."""
    fm, wm = counter_means(fetch_dir), counter_means(write_dir)
    fcopy, wcopy = fm["copy"]["FETCH_SIZE"], wm["copy"]["WRITE_SIZE"]
    ff, fw = COPY_BYTES / (fcopy * 1024.0), COPY_BYTES / (wcopy * 1024.0)
    print(f"# workload {workload}: memory traffic per launch (bytes), from rocprofv3 --pmc FETCH_SIZE "
          f"({fetch_dir}) and --pmc WRITE_SIZE ({write_dir})")
    print(f"# calibration copy of {COPY_BYTES} B: FETCH_SIZE {fcopy:.1f} KiB -> factor {ff:.4f}; "
          f"WRITE_SIZE {wcopy:.1f} KiB -> factor {fw:.4f}")
    print("# kernel  source_digest  fetch_bytes  write_bytes  traffic_bytes")
    for n in sorted(set(fm) & set(wm)):
        if n == "copy" or n not in KERNEL_SOURCE:
            continue
        fb = fm[n]["FETCH_SIZE"] * 1024.0 * ff
        wb = wm[n]["WRITE_SIZE"] * 1024.0 * fw
        print(f"kernel {n} {source_digest(n)} {fb:.0f} {wb:.0f} {fb + wb:.0f}")


def load_trace(workload):
    """{kernel: mean launch time in us} from profiles/kernel_trace_<workload>.txt
    (a rocprofv3 --kernel-trace run of this bench on that workload alone),
    for kernels whose source still matches the digest recorded there."""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.txt")
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        p = line.split()
        if len(p) == 10 and p[0] == "kernel" and p[1] in KERNEL_SOURCE and p[2] == source_digest(p[1]):
            out[p[1]] = float(p[4])
    return out


def load_traffic(workload):
    """{kernel: bytes per launch} from profiles/hbm_traffic_<workload>.txt, for
    kernels whose source still matches the digest recorded with the counters."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        p = line.split()
        if len(p) == 6 and p[0] == "kernel" and p[1] in KERNEL_SOURCE and p[2] == source_digest(p[1]):
            out[p[1]] = float(p[5])
    return out


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="chunk-256k")
    ap.add_argument("--decode-workload", default="decode-1m-draft")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", dest="fp8", action="store_false",
                    help="skip the extra runs with FP8 index keys")
    ap.add_argument("--no-paged", dest="paged", action="store_false",
                    help="skip the extra runs on a paged pool")
    ap.add_argument("--no-serving-shape", dest="serving", action="store_false",
                    help="skip the extra runs with attention at 24 q / 2 KV heads, head dim 256")
    ap.add_argument("--no-other-workloads", dest="others", action="store_false",
                    help="skip the side entries for the other three workloads (decode-8k-f32, prefill-32k, "
                         "decode-128k)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a copy of known size first (for scaling memory counters)")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="DIR")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: libqsa runs the QSA hot path on one GPU only (asked for {args.gpus}); "
              "sharding across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch
    from block_sparse_long_amd import qsa, synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    qsa.load()
    if args.copy_calibration:
        copy_calibration()
    cpu = not args.no_cpu_baseline
    spec = synth.SPECS[args.workload]
    if spec.kind == "prefill":
        pre = bench_prefill(spec, args.steps, args.warmup, cpu)
        value, unit, ms = pre["value"], "tokens/s", pre["ms_per_step"]
        main_res = pre
    else:
        pre = bench_decode(spec, args.steps * 10, args.warmup * 10, cpu)
        value, unit, ms = pre["value"], pre["unit"], pre["ms_per_step"]
        main_res = pre
    fp8_res, serve_res, paged_res = {}, {}, {}
    if args.paged:
        paged_res[spec.name] = bench_paged(spec, pre["_inputs"], args.steps if spec.kind == "prefill" else
                                           args.steps * 10, args.warmup * 10)
    if args.serving and spec.dtype == "bf16":
        s2, w2 = serving_shape_inputs(spec, pre["_inputs"])
        if spec.kind == "prefill":
            serve_res[spec.name] = bench_prefill(s2, args.steps, args.warmup, False, w=w2)
        else:
            serve_res[spec.name] = bench_decode(s2, args.steps * 10, args.warmup * 10, False, w=w2)
        del w2
    fp8kv_res = {}
    if args.fp8 and spec.dtype == "bf16":
        if spec.kind == "prefill":
            fp8_res[spec.name] = bench_prefill(spec, args.steps, args.warmup, False, keys="fp8", w=pre["_inputs"])
            fp8kv_res[spec.name] = bench_prefill(spec, args.steps, args.warmup, False, keys="fp8", kv="fp8",
                                                 w=pre["_inputs"])
        else:
            fp8_res[spec.name] = bench_decode(spec, args.steps * 10, args.warmup * 10, False, keys="fp8", w=pre["_inputs"])
            fp8kv_res[spec.name] = bench_decode(spec, args.steps * 10, args.warmup * 10, False, keys="fp8", kv="fp8",
                                                w=pre["_inputs"])
    pre.pop("_inputs", None)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic (seeded N(0,1) with planted blocks)",
        "config": {"workload": spec.name, "context": spec.ctx, "rows": spec.attn_rows, "batch": spec.batch,
                   "Hq": spec.Hq, "Hkv": spec.Hkv, "head_dim": spec.D, "index_heads": 4, "index_dim": 128,
                   "block": 4, "top_k": spec.top_k, "rope_theta": spec.theta},
        "step_ms": main_res["step_ms"],
        "roofline": main_res["roofline"],
        "cpu_baseline": main_res.get("cpu_baseline"),
        "kernels": main_res["kernels"],
        "rooflines": main_res["rooflines"],
    }
    if args.decode_workload != "none" and spec.kind == "prefill":
        dspec = synth.SPECS[args.decode_workload]
        dec = bench_decode(dspec, args.steps * 10, args.warmup * 10, cpu)
        if args.fp8 and dspec.dtype == "bf16":
            fp8_res[dspec.name] = bench_decode(dspec, args.steps * 10, args.warmup * 10, False, keys="fp8",
                                               w=dec["_inputs"])
            fp8kv_res[dspec.name] = bench_decode(dspec, args.steps * 10, args.warmup * 10, False, keys="fp8", kv="fp8",
                                                 w=dec["_inputs"])
        if args.paged:
            paged_res[dspec.name] = bench_paged(dspec, dec["_inputs"], args.steps * 10, args.warmup * 10)
        if args.serving and dspec.dtype == "bf16":
            s2, w2 = serving_shape_inputs(dspec, dec["_inputs"])
            serve_res[dspec.name] = bench_decode(s2, args.steps * 10, args.warmup * 10, False, w=w2)
            del w2
        dec.pop("_inputs", None)
        line["decode"] = {k: v for k, v in dec.items()}
        line["decode"]["config"] = {"context": dspec.ctx, "batch": dspec.batch, "q_per_seq": dspec.q_per_seq,
                                    "Hq": dspec.Hq, "Hkv": dspec.Hkv, "top_k": dspec.top_k,
                                    "steps": args.steps * 10}
    if args.others:
        # the other workloads, each timed as its own step with its own roofline
        # (not the headline): value, per-step median / p10 / p90, the
        # dominant kernel against its peak, and the oracle on a short sample
        line["other_workloads"] = {}
        for name in synth.CONFIG_ORDER:
            if name in (spec.name, args.decode_workload):
                continue
            o = synth.SPECS[name]
            if o.kind == "prefill":
                r = bench_prefill(o, args.steps, args.warmup, cpu, cpu_target_s=5.0)
                unit_o = "tokens/s"
            else:
                r = bench_decode(o, args.steps * 10, args.warmup * 10, cpu, cpu_target_s=3.0)
                unit_o = r["unit"]
            r.pop("_inputs", None)
            line["other_workloads"][name] = {
                "value": round(r["value"], 1), "unit": unit_o, "ms_per_step": round(r["ms_per_step"], 4),
                "step_ms": r["step_ms"], "dtype": o.dtype,
                "config": {"context": o.ctx, "rows": o.attn_rows, "batch": o.batch, "Hq": o.Hq, "Hkv": o.Hkv,
                           "head_dim": o.D, "top_k": o.top_k},
                "roofline": r["roofline"], "cpu_baseline": r.get("cpu_baseline"), "kernels": r["kernels"]}
            del r
    if fp8_res:
        # the same workloads with the compressed index keys in FP8 E4M3 (one
        # FP32 scale per key); not the headline: the headline keeps bf16 keys
        line["fp8_keys"] = {}
        for name, r in fp8_res.items():
            r.pop("_inputs", None)
            line["fp8_keys"][name] = {"value": round(r["value"], 1),
                                      "unit": "tokens/s" if "workload" not in r else r["unit"],
                                      "ms_per_step": round(r["ms_per_step"], 4), "kernels": r["kernels"],
                                      "roofline": r["roofline"]}
    if fp8kv_res:
        # FP8 index keys and an FP8 K/V cache (E4M3, one scale per tensor)
        line["fp8_keys_kv"] = {}
        for name, r in fp8kv_res.items():
            r.pop("_inputs", None)
            line["fp8_keys_kv"][name] = {"value": round(r["value"], 1),
                                         "unit": "tokens/s" if "workload" not in r else r["unit"],
                                         "ms_per_step": round(r["ms_per_step"], 4), "kernels": r["kernels"],
                                         "rooflines": {n: v for n, v in r["rooflines"].items()
                                                       if n.startswith("attn")}}
    if paged_res:
        # the same workloads on a paged pool (compressed keys and K/V)
        line["paged_pool"] = paged_res
    if serve_res:
        # the same workloads with attention at the serving head layout (24
        # query heads, 2 KV heads, head dim 256); index side unchanged
        line["serving_shape"] = {}
        for name, r in serve_res.items():
            r.pop("_inputs", None)
            line["serving_shape"][name] = {"Hq": 24, "Hkv": 2, "head_dim": 256, "value": round(r["value"], 1),
                                           "unit": "tokens/s" if "workload" not in r else r["unit"],
                                           "ms_per_step": round(r["ms_per_step"], 4), "kernels": r["kernels"],
                                           "rooflines": {n: v for n, v in r["rooflines"].items()
                                                         if n.startswith("attn")}}
            if "draft_loop" in r:
                line["serving_shape"][name]["draft_loop"] = r["draft_loop"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
