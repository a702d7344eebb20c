"""branch_attn_fwd_noalloc (the forward on the library's fixed per-GPU scratch)
against branch_attn_fwd with a workspace, through the C ABI: two calls in a
row, the second with a smaller problem, each equal bitwise to the workspace
call and within the bf16 tolerances of the oracle; a problem larger than the
scratch is refused before any work is enqueued."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads.configs import custom, TTT, BLOCK
from workloads.inputs import make_inputs

from gpu_util import say, dev, host, check_out, f64_all

pytestmark = pytest.mark.gpu

sda = pytest.importorskip("speculative_draft_branch_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(plan, g):
    o, ob = torch.empty_like(g["q"]), torch.empty_like(g["qb"])
    lse = torch.empty((plan.hq, plan.Nq), dtype=torch.float32, device="cuda")
    lseb = torch.empty((plan.hq, plan.Rb), dtype=torch.float32, device="cuda")
    return o, lse, ob, lseb


def _compare(w):
    t = make_inputs(w)
    plan = sda.Plan.from_workload(w)
    need = plan.workspace_bytes(0)
    say(f"[noalloc] {w.name}: N={w.N} Nq={w.Nq} Rb={w.Rb} scratch need {need} of {sda.fwd_noalloc_max_bytes()}")
    assert need <= sda.fwd_noalloc_max_bytes()
    g = {k: dev(v) for k, v in t.items()}
    ref = _outputs(plan, g)
    sda.branch_attn_fwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"], *ref, sda.workspace(plan, 0))
    got = _outputs(plan, g)
    for x in got:  # garbage in the outputs: every element must be written
        x.fill_(float("nan"))
    sda.branch_attn_fwd_noalloc(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"], *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "ob", "lseb"), got, ref):
        assert torch.equal(a, b), name
    fr = oracle.forward(oracle.Problem.from_workload(w), f64_all(t))
    check_out("o", host(got[0]), fr["o"], w.dtype, "o")
    check_out("lse", host(got[1]), fr["lse"], w.dtype, "lse")
    check_out("ob", host(got[2]), fr["ob"], w.dtype, "o")
    check_out("lseb", host(got[3]), fr["lseb"], w.dtype, "lse")


def test_noalloc_forward_matches_workspace_forward_two_calls():
    # first a larger problem, then a smaller one: the scratch keeps the first
    # call's contents, which the second must not depend on
    _compare(W.get("ctx256k_rank3_chunk64"))
    _compare(custom("small", "bf16", 12, 4, 64, [37, 70, 5, 150], None,
                    [0, 2, 36, 37, 50, 106, 107, 111, 200, 261], [2, 3, 1, 4, 3, 0, 2, 16, 7, 5],
                    [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK, BLOCK, TTT, TTT], std=1.0, seed=5))


def test_noalloc_forward_float32_plan():
    _compare(W.get("tiny_f32"))


def test_noalloc_refuses_a_problem_beyond_the_scratch():
    w = W.get("qwen3_8b_16k_div16")
    w.cu_seqlens = np.array([0, 65536], np.int32)
    w.q_pos = np.arange(65536, dtype=np.int32)
    w.anchors = np.arange(0, 65536, 2, dtype=np.int32)
    w.cu_branch = (np.arange(len(w.anchors) + 1) * 7).astype(np.int32)
    w.modes = np.zeros(len(w.anchors), np.uint8)
    plan = sda.Plan.from_workload(w)
    assert plan.workspace_bytes(0) > sda.fwd_noalloc_max_bytes()
    q = torch.empty((1, 1), device="cuda")  # never read: the size check comes first
    from speculative_draft_branch_amd._abi import check
    with pytest.raises(sda.BranchAttnError) as e:
        check(sda.lib.branch_attn_fwd_noalloc(plan.handle, *([q.data_ptr()] * 10), None),
              "branch_attn_fwd_noalloc")
    assert e.value.status == sda.BA_EWORKSPACE
    assert "scratch" in str(e.value)
