"""bench.py's host logic, without a GPU: the refusals, the work counts the
throughput figures divide by, the profile summarisers and the rule that ties
recorded HBM traffic to the kernel sources it was measured on."""
import contextlib
import csv
import io
import os
import subprocess
import sys

import pytest
import torch

import bench
import gqa_workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_gpu_exits_with_a_message():
    r = _run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""


def _brute_pairs(Lq, Lk, causal, keep=None, lens=None):
    n = 0
    for i in range(Lq):
        for j in range(Lk):
            if causal and j > Lk - Lq + i:
                continue
            if lens is not None and j >= lens:
                continue
            if keep is not None and keep[i][j] == 0:
                continue
            n += 1
    return n


@pytest.mark.parametrize("Lq,Lk", [(1, 1), (7, 7), (5, 12), (64, 64), (3, 100)])
@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_match_a_count(Lq, Lk, causal):
    assert bench.visible_pairs(Lq, Lk, causal) == _brute_pairs(Lq, Lk, causal)


@pytest.mark.parametrize("L,n", [(10, 0), (10, 1), (10, 7), (10, 10), (33, 32)])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_pairs_match_a_count(L, n, causal):
    assert bench.varlen_pairs(L, n, causal) == _brute_pairs(L, L, causal, lens=n)


@pytest.mark.parametrize("causal", [True, False])
def test_mask_pairs_match_a_count(causal):
    m = wl.random_mask((2, 9, 13), 0.4, 77)
    want = sum(_brute_pairs(9, 13, causal, keep=m[b].tolist()) for b in range(2))
    assert bench.mask_pairs(m, causal) == want


def test_prefill_flops_of_the_named_workloads():
    """4 d h_q flops per visible (row, key) pair, B sequences."""
    w = wl.WORKLOADS["worked_example_prefill_bf16"]
    assert bench.prefill_flops(w) == 4 * 32 * 8 * 64 * 1024 * 1024  # 68.72 GFLOP
    w = wl.WORKLOADS["long_context_prefill_bf16"]
    assert bench.prefill_flops(w) == 4 * 64 * 128 * (32768 * 32769 // 2)  # 17.593 TFLOP
    w = wl.WORKLOADS["chunked_prefill_bf16"]
    assert bench.prefill_flops(w) == 4 * 64 * 128 * bench.visible_pairs(2048, 32768, True)


def test_decode_bytes_count_each_cached_row_once_per_kv_head():
    w = wl.WORKLOADS["batched_decode_bf16"]
    seqlens = torch.tensor([3, 0, 5], dtype=torch.int32)
    # rows x h_kv x d x (K and V) x 2 bytes
    assert bench.decode_kv_bytes(w, seqlens) == (3 + 0 + 5) * 8 * 128 * 2 * 2
    wa = wl.WORKLOADS["batched_decode_append_bf16"]
    # with the append, the new rows are read once and written once: 2 rows a sequence
    assert bench.decode_kv_bytes(wa, seqlens) == (8 + 2 * wa.B) * 8 * 128 * 2 * 2


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


def _capture(fn, *a):
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        fn(*a)
    return buf.getvalue()


def test_trace_summary_takes_the_last_dispatches(tmp_path):
    """The summary of a kernel covers its last K dispatches (the timed ones)."""
    rows = []
    t = 0
    for i, dur in enumerate([900, 800, 100, 110, 120]):  # slow ones first (clock ramp)
        rows.append({"Kernel_Name": "void gqa::(anonymous namespace)::k<1>(A)", "Grid_Size": "64",
                     "Start_Timestamp": str(t), "End_Timestamp": str(t + dur * 1000)})
        t += dur * 1000 + 5
    p = tmp_path / "trace.csv"
    _write_csv(p, rows)
    out = _capture(bench.trace_summary, str(p), 3)
    line = [ln for ln in out.splitlines() if "gqa::k<1>" in ln][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[2:] == ["5", "3", "110.000", "100.000", "120.000"]


def test_pmc_summary_averages_per_dispatch(tmp_path):
    rows = []
    for d, vals in ((1, (10.0, 5.0)), (2, (30.0, 7.0))):  # two dispatches, two counter rows each
        for v in vals:
            rows.append({"Kernel_Name": "void gqa::(anonymous namespace)::k<1>(A)", "Grid_Size": "64",
                         "Dispatch_Id": str(d), "Counter_Name": "FETCH_SIZE", "Counter_Value": str(v)})
    p = tmp_path / "pmc.csv"
    _write_csv(p, rows)
    out = _capture(bench.pmc_summary, str(p))
    line = [ln for ln in out.splitlines() if "FETCH_SIZE" in ln][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[3:] == ["26.0", "2"]  # (15 + 37) / 2 per dispatch


def test_recorded_traffic_requires_the_current_sources(tmp_path, monkeypatch):
    """A traffic row counts only while its source digest matches the sources;
    a decode call adds the merge row."""
    dp = bench.source_digest(bench.KERNEL_SOURCES["prefill"])
    dd = bench.source_digest(bench.KERNEL_SOURCES["decode"])
    table = tmp_path / "traffic.md"
    table.write_text(
        "| kind | workload | source digest | fetch bytes | write bytes |\n"
        "|---|---|---|---|---|\n"
        f"| prefill | wa | {dp} | 100 | 20 |\n"
        f"| prefill | wb | 0000000000000000 | 100 | 20 |\n"
        f"| decode | wd | {dd} | 1000 | 3 |\n"
        f"| decode_merge | all | {dd} | 40 | 2 |\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(table))
    assert bench.recorded_traffic("prefill", "wa") == 120
    assert bench.recorded_traffic("prefill", "wb") is None  # taken on other sources
    assert bench.recorded_traffic("prefill", "absent") is None
    assert bench.recorded_traffic("decode", "wd") == 1000 + 3 + 40 + 2


def test_committed_traffic_rows_name_known_kernels_and_positive_bytes():
    """The committed summary parses: every row has a 16-hex-digit digest and
    positive byte counts."""
    n = 0
    for line in open(bench.TRAFFIC_SUMMARY):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) < 5 or cells[0] not in ("prefill", "decode", "decode_merge"):
            continue
        assert len(cells[2]) == 16 and int(cells[2], 16) >= 0
        assert float(cells[3]) > 0 and float(cells[4]) > 0
        n += 1
    assert n >= 8


def test_code_only_ignores_comments_and_layout():
    """The source digest follows the code: comments and whitespace do not
    change it, any token of code does, and comment markers inside string or
    character literals are code."""
    base = 'int f(int x) {\n    return x + 1;  // one more\n}\n'
    assert bench.code_only(base) == bench.code_only("/* header */\nint f(int x)\n{ return x + 1; }")
    assert bench.code_only(base) != bench.code_only(base.replace("x + 1", "x + 2"))
    assert bench.code_only('const char *s = "a // b";') == 'const char *s = "a // b";'
    assert bench.code_only("char c = '/'; // x") == "char c = '/';"
    assert bench.code_only('a /* b */ c') == "a c"
