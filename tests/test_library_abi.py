"""The C-ABI library on the CPU: it loads, exports every function include/branch_attn.h
declares, validates problems with the documented statuses, and its plan agrees
with the oracle on visible-pair counts (no GPU needed: planning is host code)."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as W
from workloads.configs import custom, TTT, BLOCK

sda = pytest.importorskip("speculative_draft_branch_amd")
from speculative_draft_branch_amd import Plan, BranchAttnError, BA_EINVAL, BA_EUNSUPPORTED, BA_BF16, BA_F32  # noqa

import oracle

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")


def _declared_functions():
    text = "".join(open(os.path.join(INCLUDE, f)).read() for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)
    skip = {"if", "sizeof", "defined", "extern", "typedef"}
    return sorted({n for n in names if n not in skip and (n.startswith(("ba_", "branch_attn_")) or n in (
        "lse_merge",))})


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(sda.library_path())
    declared = _declared_functions()
    assert "branch_attn_fwd" in declared and "lse_merge" in declared and "ba_plan_create" in declared
    assert "branch_attn_fwd_noalloc" in declared
    for name in declared:
        assert hasattr(lib, name), name
    from speculative_draft_branch_amd import tapchannel
    assert set(declared) == set(sda.exported_symbols()) | set(tapchannel.SYMBOLS)
    assert sda.abi_version() == 1


def _plan(**kw):
    base = dict(dtype=BA_BF16, num_q_heads=4, num_kv_heads=2, head_dim=128, cu_seqlens=[0, 5, 9],
                q_pos=None, anchors=[1, 6], cu_branch=[0, 2, 5], modes=[TTT, BLOCK])
    base.update(kw)
    return Plan(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=6, num_kv_heads=4), BA_EINVAL),
    (dict(head_dim=96), BA_EUNSUPPORTED),
    (dict(cu_seqlens=[1, 5, 9]), BA_EINVAL),
    (dict(cu_seqlens=[0, 5, 4]), BA_EINVAL),
    (dict(q_pos=[0, 3, 3]), BA_EINVAL),
    (dict(q_pos=[0, 9]), BA_EINVAL),
    (dict(anchors=[6, 1]), BA_EINVAL),
    (dict(anchors=[1, 9]), BA_EINVAL),
    (dict(cu_branch=[0, 3, 2]), BA_EINVAL),
    (dict(cu_branch=[1, 2, 5]), BA_EINVAL),
    (dict(cu_branch=[0, 2, 40]), BA_EINVAL),
    (dict(modes=[TTT, 7]), BA_EINVAL),
    (dict(kv_head_of=[0, 0, 0, 1]), BA_EINVAL),
    (dict(kv_head_of=[0, 1, 2, 1]), BA_EINVAL),
    (dict(dtype=5), BA_EINVAL),
])
def test_plan_rejects_malformed_problems(kw, status):
    with pytest.raises(BranchAttnError) as e:
        _plan(**kw)
    assert e.value.status == status


def test_plan_accepts_edge_cases():
    # no branches, single-token sequences, empty sequences, a strided kv_head_of map
    p = _plan(anchors=[], cu_branch=[0], modes=[])
    assert p.Rb == 0 and p.Nq == 9
    p = _plan(cu_seqlens=[0, 1, 1, 2, 9], anchors=[0, 1], cu_branch=[0, 1, 3], modes=[TTT, BLOCK])
    assert p.N == 9 and p.Rb == 3
    p = _plan(kv_head_of=[0, 1, 0, 1])
    assert p.Nq == 9
    p = _plan(q_pos=[], anchors=[4], cu_branch=[0, 3], modes=[TTT])
    assert p.Nq == 0 and p.Rb == 3


def _pairs_oracle(w):
    c = oracle.pair_counts(oracle.Problem.from_workload(w))
    return (c["main"], c["branch_prefix"], c["branch_local"])


@pytest.mark.parametrize("name", W.names())
def test_plan_pair_counts_match_oracle(name):
    w = W.get(name)
    p = Plan.from_workload(w)
    assert p.pairs == _pairs_oracle(w)
    assert (p.N, p.Nq, p.Rb) == (w.N, w.Nq, w.Rb)
    # every row lands in exactly one query tile; each tile covers <= 128 MFMA rows
    G = w.num_q_heads // w.num_kv_heads
    rt = max(1, 128 // G)
    assert p.n_qtiles >= -(-(w.Nq + w.Rb) // rt)


def test_plan_pair_counts_tiny_cases():
    w = custom("t", "bf16", 4, 2, 64, [5, 7, 4], [1, 4, 5, 9, 13, 15], [0, 2, 5, 6, 11, 12, 15],
               [2, 3, 1, 4, 3, 0, 2], [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK])
    assert Plan.from_workload(w).pairs == _pairs_oracle(w)


def test_workspace_sizes_cover_partials():
    w = W.get("ctx256k_rank3_chunk64")
    p = Plan.from_workload(w)
    f32 = 4
    partial = w.Rb * w.num_q_heads * (w.head_dim + 1) * f32  # one float32 (O, LSE) partial of the branch rows
    # bf16 takes the branch keys inside the main kernel: no partial at all, only
    # the metadata and the transposed main and branch V tiles (the branch tiles
    # per forward unit, which together cover every branch key at least once)
    vt = (-(-w.N // 64) + -(-w.Rb // 64)) * 64 * w.num_kv_heads * w.head_dim * 2
    assert vt <= p.workspace_bytes(0) < vt + partial // 8
    pf = Plan.from_workload(W.get("tiny_f32"))
    wf = W.get("tiny_f32")
    # float32: both partials of the split path
    assert pf.workspace_bytes(0) >= 2 * wf.Rb * wf.num_q_heads * (wf.head_dim + 1) * f32
    assert p.workspace_bytes(1) >= (w.Nq + w.Rb) * w.num_q_heads * (w.head_dim + 1) * f32
    assert 0 < p.workspace_bytes(2) <= p.workspace_bytes(0)


def _key_tiles_unsplit(w):
    bk = 384 if (w.dtype == "bf16" and w.head_dim == 64) else 256
    cu = w.cu_seqlens
    return sum(-(-int(cu[i + 1] - cu[i]) // bk) for i in range(len(cu) - 1))


@pytest.mark.parametrize("name,splits", [("ctx256k_rank3", False), ("gptoss_128k_mixed", False),
                                         ("qwen3_8b_16k", True), ("qwen3_8b_16k_div16", True)])
def test_backward_key_tiles_split_only_where_one_tile_outweighs_a_units_share(name, splits):
    """A bf16 plan splits a key tile's query range in two (never more) only when
    that tile costs more than 1/256 of the whole kernel per kv head; such plans
    carry float32 dK, dV accumulators in the backward workspace."""
    w = W.get(name)
    p = Plan.from_workload(w)
    base = _key_tiles_unsplit(w)
    n_split = p.n_ktiles - base
    assert (n_split > 0) == splits and 0 <= n_split <= base
    if splits:  # the backward workspace holds the two float32 accumulators
        acc = 2 * w.N * w.num_kv_heads * w.head_dim * 4
        assert p.workspace_bytes(1) > acc


def test_float32_plans_never_split_key_tiles():
    w = W.get("tiny_f32")
    p = Plan.from_workload(w)
    assert p.n_ktiles == _key_tiles_unsplit(w)


def test_timing_api_without_launches():
    """The opt-in timing calls work on the host alone: names for every kernel id,
    zero totals when nothing was recorded, and argument checks."""
    sda.timing_reset()
    sda.timing_enable(True)
    sda.timing_enable(False)
    rec = sda.timing_read()
    assert {"main_fwd", "main_bwd_dq", "main_bwd_dkdv", "lse_merge", "branch_local_fwd"} <= set(rec)
    assert all(v == (0.0, 0) for v in rec.values())
    lib = sda.lib
    assert lib.ba_timing_kernel_name(-1) is None
    assert lib.ba_timing_kernel_name(lib.ba_timing_kernels()) is None
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.ba_timing_read(lib.ba_timing_kernels(), ctypes.byref(ms), ctypes.byref(n)) == BA_EINVAL


def test_entry_points_reject_bad_arguments_without_touching_the_gpu():
    """Structural argument errors are reported before anything is enqueued."""
    w = W.get("tiny_f32")
    p = Plan.from_workload(w)
    lib = sda.lib
    # NULL plan, NULL tensors, short workspace, misaligned pointers
    assert lib.branch_attn_fwd(None, *([None] * 10), None, 0, None) == BA_EINVAL
    fake = 1 << 40  # never dereferenced: checks fail first
    args = [fake] * 6 + [fake] * 4
    assert lib.branch_attn_fwd(p.handle, *args, None, 0, None) == sda.BA_EWORKSPACE
    assert lib.branch_attn_fwd(p.handle, *args, fake, 16, None) == sda.BA_EWORKSPACE
    bad = list(args)
    bad[0] = fake + 2
    assert lib.branch_attn_fwd(p.handle, *bad, fake, p.workspace_bytes(0), None) == BA_EINVAL
    assert lib.lse_merge(10, 2, 6, fake, fake, fake, fake, fake, 0, fake, None) == BA_EINVAL  # d/4 must divide 64
    assert lib.lse_merge(10, 2, 64, fake, fake, fake, fake, fake, 7, fake, None) == BA_EINVAL  # bad dtype


def test_ring_step_rejects_bad_windows_without_touching_the_gpu():
    """ba_ring_step_fwd: bf16 plans only; 0 <= win_lo <= win_hi <= N; checks come first."""
    lib = sda.lib
    fake = 1 << 40  # never dereferenced
    pf = Plan.from_workload(W.get("tiny_f32"))
    assert lib.ba_ring_step_fwd(pf.handle, fake, fake, fake, fake, 0, 8, fake, fake, fake,
                                pf.workspace_bytes(2), None) == sda.BA_EUNSUPPORTED
    w = W.get("qwen3_8b_16k_div16")
    p = Plan.from_workload(w)
    ws = p.workspace_bytes(2)
    for lo, hi in ((-1, 5), (10, 5), (w.N - 3, w.N + 1)):
        assert lib.ba_ring_step_fwd(p.handle, fake, fake, fake, fake, lo, hi, fake, fake, fake, ws, None) == BA_EINVAL
    assert lib.ba_ring_step_fwd(p.handle, fake, fake, fake, fake, 0, 64, fake, fake, fake, 16, None) == \
        sda.BA_EWORKSPACE
    assert lib.ba_ring_step_fwd(p.handle, fake, fake, fake + 2, fake, 0, 64, fake, fake, fake, ws, None) == BA_EINVAL
    # an empty window is accepted and enqueues nothing (no stream, no device access)
    assert lib.ba_ring_step_fwd(p.handle, fake, fake, None, None, 5, 5, fake, fake, fake, ws, None) == sda.BA_OK
