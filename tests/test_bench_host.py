"""bench.py's host logic, without a GPU: the one-GPU guard, the algorithmic
work each roofline is computed from, the mapping of rocprofv3 kernel names to
the library's launch names, the kernel-trace and counter summaries, and the
rule that measured traffic is used only while a kernel's source still matches
the digest recorded with the counters."""
import csv
import dataclasses
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_prefill_work_counts_pairs_and_positions(bench):
    from block_sparse_long_amd import synth
    spec = synth.scaled("chunk-256k", ctx=64, chunk=8, top_k=4)
    row_pos = np.arange(56, 64)                    # t = 56..63: nc = 14..16, tails 1..4 -> 0..3
    work, pairs, npos = bench.prefill_work(spec, row_pos)
    nc = (row_pos + 1) // 4
    assert pairs == int(nc.sum())
    tails = row_pos - 4 * nc + 1
    assert npos == float((4 * np.minimum(nc, 4) + tails).sum())
    assert work["score_filter"] == ("mfma", 2.0 * 4 * 128 * pairs, "flop")
    assert work["attn_prefill_mfma"] == ("mfma", 4.0 * spec.Hq * spec.D * npos, "flop")
    wide = dataclasses.replace(spec, Hq=24, Hkv=2, D=256)
    assert bench.prefill_work(wide, row_pos)[0]["attn_prefill_mfma_d256"][1] == 4.0 * 24 * 256 * npos


def test_decode_work_bytes(bench):
    from block_sparse_long_amd import synth
    spec = synth.scaled("decode-1m-draft", ctx=4096, batch=2, top_k=8)
    anchor = np.full(2, 4095)
    attn_pos = 4096 + np.tile(np.arange(4), (2, 1))
    tail_start = np.full(2, 4096)
    work, pairs = bench.decode_work(spec, anchor, attn_pos, tail_start)
    assert pairs == 2 * 1024
    assert work["score_rows_bf16"][1] == 2 * 1024 * 128 * 2
    assert work["score_rows_fp8"][1] == 2 * 1024 * (128 + 4)
    # each sequence reads 8 kept blocks (32 positions) and 4 drafted positions of K and V
    kv = 2 * 2.0 * (32 + 4) * spec.Hkv * spec.D * 2
    q = 2.0 * 2 * 4 * spec.Hq * spec.D * 2
    assert work["attn_decode_mfma"][1] == kv + q
    assert work["attn_decode_mfma_fp8kv"][1] == kv / 2 + q   # one byte per K/V element


def test_roofline_fraction(bench):
    r = bench.roofline_for("score_filter", ("mfma", 1.25e12, "flop"), (3, 1.0, 1.0, [0.9, 1.0, 1.1]),
                           {"score_filter": 123.0})
    assert r["achieved"] == pytest.approx(1250.0) and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(0.5) and r["traffic"] == 123.0
    assert r["median_us"] == 1000.0 and r["p10_us"] == 920.0 and r["p90_us"] == 1080.0
    r = bench.roofline_for("score_rows_bf16", ("hbm", 4e6, "B"), (1, 0.001, 0.001, [0.001]), None)
    assert r["achieved"] == pytest.approx(4000.0) and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(0.5) and r["traffic"] is None


@pytest.mark.parametrize("name,short", [
    ("void qsa::score_filter_kernel<false>(qsa::FusedScoreArgs)", "score_filter"),
    ("void qsa::score_filter_kernel<true>(qsa::FusedScoreArgs)", "score_filter_fp8"),
    ("void qsa::score_sample_kernel<true>(qsa::FusedScoreArgs)", "score_sample_fp8"),
    ("void qsa::sample_threshold_kernel<4>(qsa::FusedScoreArgs)", "sample_threshold"),
    ("qsa::score_rows_bf16_kernel(unsigned short const*, int const*)", "score_rows_bf16"),
    ("void qsa::attn_prefill_mfma_kernel<128, unsigned short>(qsa::AttnArgs, int)", "attn_prefill_mfma"),
    ("void qsa::attn_prefill_mfma_kernel<256, unsigned short>(qsa::AttnArgs, int)", "attn_prefill_mfma_d256"),
    ("void qsa::attn_decode_mfma_kernel<128, unsigned char>(qsa::AttnArgs)", "attn_decode_mfma_fp8kv"),
    ("void qsa::attn_decode_mfma_kernel<256, unsigned char>(qsa::AttnArgs)", "attn_decode_mfma_d256_fp8kv"),
    ("void qsa::attn_kernel<float, 64, true>(qsa::AttnArgs)", "attn_decode"),
    ("void qsa::attn_kernel<unsigned short, 16, false>(qsa::AttnArgs)", "attn_prefill"),
    ("void qsa::attn_combine_kernel<unsigned short, 256>(float const*, int, void*, float*)", "attn_combine"),
    ("void at::native::(anonymous namespace)::neg_kernel(...)", "copy"),
    ("void at::native::vectorized_elementwise_kernel<4>(...)", None),
])
def test_short_kernel_names(bench, name, short):
    assert bench.short_kernel_name(name) == short


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_kernel_trace_and_counter_summaries(bench, tmp_path):
    k = "void qsa::score_filter_kernel<false>(qsa::FusedScoreArgs)"
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [{"Kernel_Name": k, "Start_Timestamp": 1000, "End_Timestamp": 5000},
                {"Kernel_Name": k, "Start_Timestamp": 9000, "End_Timestamp": 11000},
                {"Kernel_Name": "other", "Start_Timestamp": 0, "End_Timestamp": 7}])
    st = bench.kernel_trace_stats(str(tmp_path / "t"))
    assert st == {"score_filter": (2, 3.0, 3.0, 2.2, 3.8, 2.0, 4.0)}   # launches, mean, median, p10, p90, min, max
    # counters are summed over a dispatch's rows (one per XCD or instance), then averaged over dispatches
    _write_csv(str(tmp_path / "c" / "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"],
               [{"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Dispatch_Id": 1, "Counter_Value": 10},
                {"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Dispatch_Id": 1, "Counter_Value": 30},
                {"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Dispatch_Id": 2, "Counter_Value": 60}])
    assert bench.counter_means(str(tmp_path / "c")) == {"score_filter": {"FETCH_SIZE": 50.0}}


def test_traffic_is_used_only_while_the_source_matches(bench, tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    good = bench.source_digest("score_filter")
    with open(tmp_path / "profiles" / "hbm_traffic_w.txt", "w") as f:
        f.write("# kernel  source_digest  fetch_bytes  write_bytes  traffic_bytes\n")
        f.write(f"kernel score_filter {good} 1 2 3\n")
        f.write("kernel select_merge 0000000000000000 4 5 9\n")
        f.write("kernel not_a_kernel abc 1 1 2\n")
    assert bench.load_traffic("w") == {"score_filter": 3.0}
    assert bench.load_traffic("missing") == {}


def test_trace_is_used_only_while_the_source_matches(bench, tmp_path, monkeypatch, capsys):
    # a summary written by --rocprof-summary is read back by load_trace
    k = "void qsa::score_filter_kernel<false>(qsa::FusedScoreArgs)"
    m = "void qsa::select_merge_kernel<false>(qsa::FusedScoreArgs, int*, int*, float*)"
    _write_csv(str(tmp_path / "t" / "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [{"Kernel_Name": k, "Start_Timestamp": 0, "End_Timestamp": 500_000},
                {"Kernel_Name": k, "Start_Timestamp": 0, "End_Timestamp": 520_000},
                {"Kernel_Name": m, "Start_Timestamp": 0, "End_Timestamp": 80_000}])
    bench.rocprof_summary([str(tmp_path / "t")])
    lines = capsys.readouterr().out.splitlines()   # select_merge's line as if its source had changed since
    text = "\n".join(ln.replace(bench.source_digest("select_merge"), "0000000000000000")
                     if ln.startswith("kernel select_merge") else ln for ln in lines) + "\n"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    with open(tmp_path / "profiles" / "kernel_trace_w.txt", "w") as f:
        f.write(text)
    assert bench.load_trace("w") == {"score_filter": 510.0}      # select_merge's digest no longer matches
    assert bench.load_trace("missing") == {}
    r = bench.roofline_for("score_filter", ("mfma", 5.0e11, "flop"), (1, 0.5, 0.5, [0.5]), None,
                           bench.load_trace("w"))
    assert r["frac"] == 0.4 and r["trace_avg_us"] == 510.0 and r["trace_frac"] == round(5.0e11 / 510e-6 / 2.5e15, 4)


def test_counter_summary_is_digest_stamped_with_derived_rates(bench, tmp_path, capsys):
    k = "void qsa::score_filter_kernel<false>(qsa::FusedScoreArgs)"
    rows = []
    for name, val in [("SQ_VALU_MFMA_BUSY_CYCLES", 4.0e8), ("GRBM_GUI_ACTIVE", 8.0e6), ("SQ_INSTS_VALU", 5.0e6),
                      ("SQ_INSTS_MFMA", 1.0e6), ("SQ_VALU_MFMA_COEXEC_CYCLES", 1.0e8)]:
        rows.append({"Kernel_Name": k, "Counter_Name": name, "Dispatch_Id": 1, "Counter_Value": val})
    _write_csv(str(tmp_path / "c" / "run_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"], rows)
    bench.rocprof_summary([str(tmp_path / "c")])
    line = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("counters score_filter")][0]
    assert bench.source_digest("score_filter") in line
    # busy cycles over (GUI cycles per XCD x SIMDs): 4e8 / (8e6 / 8 * 1024)
    assert f"mfma_busy={4.0e8 / (8.0e6 / 8 * 1024):.4f}" in line
    assert "coexec=0.2500" in line and "valu_per_mfma=4.000" in line
