"""Host logic of bench.py that runs without a GPU: the multi-GPU refusal, the
rocprofv3 database summaries that feed profiles/, and the rule that a
counter summary is used only while its kernel's sources are unchanged."""

import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line


def _kernel_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, grid_x int, grid_y int, grid_z int, workgroup_x int, "
                "vgpr_count int, accum_vgpr_count int, lds_size int, scratch_size int, duration int)")
    con.executemany("insert into kernels values (?,?,?,?,?,?,?,?,?,?)", rows)
    con.commit()
    con.close()


def _counter_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?,?,?)", rows)
    con.commit()
    con.close()


def test_kernel_trace_summary(tmp_path):
    db = str(tmp_path / "kt.db")
    k = "void nk::(anonymous namespace)::attn_decode_kernel<128, 16, false, 2, 16>(nk::AttnArgs)"
    _kernel_db(db, [(k, 4096, 1, 1, 64, 68, 0, 0, 0, 50000), (k, 4096, 1, 1, 64, 68, 0, 0, 0, 54000),
                    ("other", 64, 1, 1, 64, 8, 0, 0, 0, 1000)])
    text = bench.rocpd_summary(db, "title", "the command")
    lines = text.splitlines()
    assert lines[0] == "# title" and lines[1] == "# command: the command"
    row = [l for l in lines if l.startswith("attn_decode_kernel<128, 16, false, 2, 16>")][0]
    cells = [c.strip() for c in row.split("|")]
    assert cells[6] == "2"                               # calls
    assert float(cells[7]) == pytest.approx(52.0)        # average us
    assert float(cells[8]) == pytest.approx(50.0) and float(cells[9]) == pytest.approx(54.0)
    # the kernel with the most total time comes first
    assert lines[4].startswith("attn_decode_kernel")


def test_counter_average_and_calibration(tmp_path):
    db = str(tmp_path / "pmc.db")
    _counter_db(db, [("attn_decode_kernel<128, 16, false, 2, 16>", "FETCH_SIZE", 100.0),
                     ("attn_decode_kernel<128, 16, false, 2, 16>", "FETCH_SIZE", 300.0),
                     ("attn_decode_kernel<128, 16, true, 6, 32>", "FETCH_SIZE", 1e6),
                     ("attn_decode_kernel<128, 16, false, 2, 16>", "WRITE_SIZE", 7.0)])
    avg, n = bench.rocpd_counter(db, "attn_decode_kernel<128, 16, false", "FETCH_SIZE")
    assert (avg, n) == (200.0, 2)
    assert bench.rocpd_counter(db, "no such kernel", "FETCH_SIZE") == (None, 0)


def test_traffic_is_used_only_for_unchanged_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "ragged_paged_kv_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in set(bench.KERNEL_SOURCES):
        (csrc / f).write_text("// " + f)
    kernel = "attn_decode_kernel<128, 16, false"
    rec = {"kernel": kernel, "bytes_per_launch": 123.0,
           "source_hash": bench.source_hash(bench.family_sources(kernel))}
    (prof / "traffic_decode_bf16.json").write_text(json.dumps(rec))
    assert bench.load_traffic("decode_bf16") == 123.0
    (csrc / "attn_prefill.hip").write_text("// another kernel changed")
    assert bench.load_traffic("decode_bf16") == 123.0            # not one of the decode kernel's sources
    (csrc / "attn_decode.hip").write_text("// the decode kernel changed")
    assert bench.load_traffic("decode_bf16") is None
    assert bench.load_traffic("no_such_key") is None


def test_mfma_summary(tmp_path):
    db = str(tmp_path / "mfma.db")
    k = "attn_prefill_kernel<128, 16, false, 8>"
    _counter_db(db, [(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0), (k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 3000.0),
                     (k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0), (k, "GRBM_GUI_ACTIVE", 80.0),
                     (k, "SQ_BUSY_CYCLES", 5.0), ("prefill_plan_kernel", "GRBM_GUI_ACTIVE", 1e9)])
    rec = bench.rocpd_mfma(db, "attn_prefill_kernel<128, 16, false", simds=64, gui_instances=8,
                           flops_per_launch=512.0 * 1000)
    assert rec["dispatches"] == 2
    assert rec["mfma_flops_per_dispatch"] == pytest.approx(512.0 * 2000)     # 512 flops per MOPS unit
    assert rec["executed_over_algorithmic"] == pytest.approx(2.0)
    assert rec["active_cycles"] == pytest.approx(10.0)                       # one XCD's share
    assert rec["mfma_busy_frac"] == pytest.approx(1024.0 / (10.0 * 64))


def test_cpu_baseline_pool_reports_each_kind():
    """The host baseline runs the oracle in a process pool over row blocks
    and reports one rate per kind of work, with the pool's process count as
    its cores."""
    import concurrent.futures as cf
    import multiprocessing as mp

    assert 1 <= bench.cpu_cores() <= bench.CPU_MAX_WORKERS
    with cf.ProcessPoolExecutor(2, mp_context=mp.get_context("spawn")) as pool:
        res = bench.cpu_baseline("tiny_prefill_f32", 0.5, pool, 2)
    assert set(res) == {"prefill"}
    r = res["prefill"]
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert "2 processes" in r["sample"]
