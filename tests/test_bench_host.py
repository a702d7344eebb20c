"""Host-side behaviour of bench.py that needs no GPU: the one-GPU guard, the
shader-clock sampler's switches, and the source hash that ties committed
counter summaries to the kernel code they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_clock_sampler_reads_sysfs_and_starts_no_tool(tmp_path, monkeypatch):
    """The clock comes from the pp_dpm_sclk text in this process (no subprocess,
    so nothing is exec'd from a process that may have touched the GPU)."""
    txt = "0: 500Mhz\n1: 1843Mhz *\n2: 2400Mhz\n"
    assert bench.parse_sclk(txt) == 1843.0
    assert bench.parse_sclk("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.parse_sclk("") is None
    f = tmp_path / "pp_dpm_sclk"
    f.write_text(txt)
    import subprocess as sp

    def no_subprocess(*a, **k):
        raise AssertionError("the clock sampler must not start a process")

    monkeypatch.setattr(sp, "run", no_subprocess)
    monkeypatch.setattr(sp, "Popen", no_subprocess)
    monkeypatch.setattr(bench, "_sclk_path", lambda pci=None: str(f))
    with bench.ClockSampler() as clk:
        import time
        time.sleep(0.3)
    assert clk.mhz() == 1843.0
    with bench.ClockSampler(enabled=False) as clk:
        pass
    assert clk.path is None and clk.mhz() is None


def test_clock_path_of_a_missing_device_is_none():
    assert bench._sclk_path((0xffff, 0xff, 0x1f)) is None


def test_stratified_sample_covers_each_stratum():
    import numpy as np
    import workloads as W
    w = W.get("ctx256k_rank3")
    rows = bench.stratified_rows(w, 512)
    assert len(rows) == 512 == len(set(rows))
    assert all(0 <= r < w.Nq + w.Rb for r in rows)
    c = 16384
    # first and last rows of both query chunks (chunks 3 and 12), early in the list
    head = set(rows[:40])
    assert {0, c - 1, c, 2 * c - 1} <= head
    # branch rows of the anchors at the chunk starts (positions 3c and 12c)
    assert w.Nq + 0 in rows and w.Nq + 7 * c in rows
    # depth 1 and depth 7 rows
    depth = [(r - w.Nq) % 7 for r in rows if r >= w.Nq]
    assert 0 in depth and 6 in depth
    # packed sequences: first and last row of every sequence
    w2 = W.get("qwen3_8b_16k")
    rows2 = set(bench.stratified_rows(w2, 512))
    for s in range(w2.num_seqs):
        assert int(w2.cu_seqlens[s]) in rows2 and int(w2.cu_seqlens[s + 1]) - 1 in rows2
    # deterministic
    assert bench.stratified_rows(w, 512) == rows
    del np


def test_cpu_baseline_extrapolates_by_pair_count():
    import workloads as W
    from workloads.inputs import make_inputs
    w = W.get("ctx256k_rank3_chunk64")
    t = make_inputs(w, grads=True)
    r = bench.cpu_baseline(w, t, 0.5)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["rows_timed"] >= 1
    assert r["pairs_timed"] == sum(bench.row_pairs(w, bench.stratified_rows(w, 512)[:r["rows_timed"]]))
    key = "extrapolated CPU time (%d cores)" % r["cores"]
    # "seconds" is rounded to 0.01 s and the extrapolation to 0.1 s
    ratio = r["pairs_full"] / r["pairs_timed"]
    assert abs(r[key] - r["seconds"] * ratio) <= 0.05 + 0.005 * ratio + 1e-6 * r[key]
    assert r["host"]["os_cpu_count"] == os.cpu_count()


def test_kernel_source_hash_ignores_comment_only_edits(tmp_path, monkeypatch):
    csrc = tmp_path / "speculative_draft_branch_amd" / "csrc"
    csrc.mkdir(parents=True)
    f = csrc / "k.hip"
    f.write_text("int a = 1;  // one\n\n// note\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash(["k.hip"])
    f.write_text("int a = 1;  // a different comment\n// another note\n\nint b = 2;   \n")
    assert bench.kernel_source_hash(["k.hip"]) == h0
    f.write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash(["k.hip"]) != h0


@pytest.mark.parametrize("kernel", ["main_fwd", "main_bwd_dq", "main_bwd_dkdv"])
def test_committed_counter_summaries_parse(kernel):
    path = os.path.join(ROOT, "profiles", f"{kernel}_ctx256k_rank3_pmc.json")
    with open(path) as fh:
        d = json.load(fh)
    assert d["kernel"] == kernel and d["hbm_bytes_per_launch"] > 0
    assert len(d["source_hash"]) == 16 and len(d["commands"]) == 2
