"""GPU parity of the ring step (ba_ring_step_fwd): main-key windows delivered one
at a time, as a context-parallel ring delivers K/V chunks, merged into a running
(O, LSE), against the oracle's ring form and against the single pass."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import speculative_draft_branch_amd as sda
import workloads as W
from workloads.configs import custom, TTT, BLOCK
from workloads.inputs import make_inputs

from gpu_util import say, dev, host, check_out, f64_all

pytestmark = pytest.mark.gpu


def _run_ring(w, windows):
    """Every window through ba_ring_step_fwd, each from its own K/V copy."""
    t = make_inputs(w)
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    R, hq, d = w.Nq + w.Rb, w.num_q_heads, w.head_dim
    o_run = torch.zeros((R, hq, d), dtype=torch.float32, device="cuda")
    lse_run = torch.full((hq, R), float("-inf"), dtype=torch.float32, device="cuda")
    ws = sda.workspace(plan, 2)
    for lo, hi in windows:
        k_win, v_win = g["k"][lo:hi].clone(), g["v"][lo:hi].clone()
        sda.ba_ring_step_fwd(plan, g["q"], g["qb"], k_win, v_win, lo, hi, o_run, lse_run, ws)
    torch.cuda.synchronize()
    return t, plan, g, ws, host(o_run), host(lse_run)


def _check_against_oracle(w, t, windows, o_run, lse_run):
    o_ref, l_ref = oracle.ring_forward(oracle.Problem.from_workload(w), f64_all(t), windows)
    seen = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse_run), seen), "rows with no key in any window must stay at -inf"
    assert np.all(o_run[~seen.T] == 0.0)
    check_out("o_run", o_run, o_ref, "bf16", "o")
    check_out("lse_run", np.where(seen, lse_run, 0.0), np.where(seen, l_ref, 0.0), "bf16", "lse")


def test_zigzag_ring_of_rank3_matches_oracle_and_single_pass():
    """Rank 3 of a CP=8 zigzag layout (16 chunks, rank r holds chunks r and 15-r):
    the chunk pairs in the order the ring brings them, each chunk its own window;
    chunks past the rank's last key arrive as empty windows."""
    w = W.get("ctx256k_rank3_chunk64")
    chunk = 64
    windows = []
    for s in range(8):
        r = (3 - s) % 8
        for c in (r, 15 - r):
            lo, hi = min(c * chunk, w.N), min((c + 1) * chunk, w.N)
            windows.append((lo, hi))
    say(f"[ring] {w.name}: {len(windows)} windows, N={w.N}")
    t, plan, g, ws, o_run, lse_run = _run_ring(w, windows)
    _check_against_oracle(w, t, windows, o_run, lse_run)
    # the single pass of the same main-key part
    hq, d = w.num_q_heads, w.head_dim
    o = torch.empty_like(g["q"])
    lse = torch.empty((hq, w.Nq), dtype=torch.float32, device="cuda")
    o_pre = torch.empty((w.Rb, hq, d), dtype=torch.float32, device="cuda")
    lse_pre = torch.empty((hq, w.Rb), dtype=torch.float32, device="cuda")
    sda.ba_main_fwd(plan, g["q"], g["qb"], g["k"], g["v"], o, lse, o_pre, lse_pre, ws)
    torch.cuda.synchronize()
    check_out("ring vs single pass, o", o_run, np.concatenate([host(o), host(o_pre)]), "bf16", "o")
    check_out("ring vs single pass, lse", lse_run, np.concatenate([host(lse), host(lse_pre)], axis=1), "bf16", "lse")


RAGGED = {
    # packed sequences of odd lengths, every branch mode; window edges fall inside
    # sequences and inside 64-key tiles, one window is empty
    "mixed_d128": (lambda: custom("rm", "bf16", 4, 2, 128, [37, 70, 5, 150], None,
                                  [0, 2, 36, 37, 50, 106, 107, 111, 200, 261], [2, 3, 1, 4, 3, 0, 2, 16, 7, 5],
                                  [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK, BLOCK, TTT, TTT], std=1.0, seed=6),
                   [(101, 180), (0, 23), (64, 64), (180, 262), (23, 64), (64, 100), (100, 101)]),
    # GQA 8:1 at d=64, a query subset, windows 1 to 150 keys wide
    "qsubset_d64": (lambda: custom("rq", "bf16", 16, 2, 64, [300, 41], list(range(5, 341, 7)),
                                   list(range(3, 341, 11)), [7] * 31, [TTT] * 31, std=1.0, seed=6),
                    [(299, 300), (150, 299), (0, 1), (1, 150), (300, 341)]),
    # only some windows arrive: rows whose keys all lie elsewhere keep (0, -inf)
    "partial_cover": (lambda: custom("rp", "bf16", 4, 2, 128, [37, 70, 5, 150], None, [0, 50, 200], [3, 16, 7],
                                     [TTT, BLOCK, TTT], std=1.0, seed=6),
                      [(120, 190), (0, 30)]),
}


@pytest.mark.parametrize("name", list(RAGGED))
def test_ring_ragged_windows_match_oracle(name):
    build, windows = RAGGED[name]
    w = build()
    say(f"[ring] {name}: N={w.N} Nq={w.Nq} Rb={w.Rb} windows={windows}")
    t, _, _, _, o_run, lse_run = _run_ring(w, windows)
    _check_against_oracle(w, t, windows, o_run, lse_run)
