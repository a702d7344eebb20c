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


def test_clock_sampler_off_when_disabled_or_under_a_profiler(monkeypatch):
    monkeypatch.delenv("LD_PRELOAD", raising=False)
    monkeypatch.delenv("HSA_TOOLS_LIB", raising=False)
    assert bench.ClockSampler(enabled=False).tool is None
    # a preloaded profiler library would initialise the GPU inside the tool's
    # process before it execs its interpreter: the sampler must not start it
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    assert bench.ClockSampler().tool is None
    monkeypatch.delenv("LD_PRELOAD")
    monkeypatch.setenv("HSA_TOOLS_LIB", "librocprofiler64.so")
    assert bench.ClockSampler().tool is None
    with bench.ClockSampler(enabled=False) as clk:
        pass
    assert clk.mhz() is None


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
