"""The host planner (csrc/plan.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer.

plan.cpp is plain C++ that turns a caller's problem description into the
plan the kernels run (row key ranges, query and key tiles, launch orders), so
it is built here with g++ and the sanitizers, apart from the HIP library, and
driven by tests/host/plan_sanitize.cpp: seeded random problems (sequence,
query, anchor and branch layouts, head maps, both dtypes and head sizes) must
build, each with one malformation at a time must be refused with the
documented status, and a full-size 256K-token plan must build. Any memory or
undefined-behaviour error aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_draft_branch_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "host", "plan_sanitize.cpp"),
           "-o", exe]
    subprocess.run(cmd, check=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (1, 2, 3):
        r = subprocess.run([exe, str(seed), "400"], capture_output=True, text=True, timeout=300, env=env)
        if "does not come first in initial library list" in r.stderr:
            pytest.skip("this environment preloads a library ahead of the ASan runtime")
        assert r.returncode == 0, r.stdout + r.stderr
        assert " 0 failures" in r.stdout, r.stdout
