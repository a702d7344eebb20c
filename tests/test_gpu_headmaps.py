"""GPU parity, against the dense CPU oracle, of GQA head maps other than the
contiguous one, group sizes that do not divide the 128-row MFMA tile, and
softmax scales other than 1/sqrt(d): forward and backward element by element,
plus one ring-step and one split-path case with a strided map.

A group size G that does not divide 128 leaves 128 mod G padding rows in every
query tile, so every backward key tile takes the masked dK/dV path; a strided
or permuted map sends the q heads of one kv group to scattered output columns;
a non-default scale reaches the forward's exponent, the dQ kernel and the dK/dV
kernel's scaled staged Q.
"""
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

GRADS = ("dq", "dk", "dv", "dqb", "dkb", "dvb")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# Packed sequences with ragged lengths (one longer than two backward key tiles),
# every branch mode, a zero-length branch, a 32-row branch and anchors at
# sequence starts.
SEQS = [37, 611, 5, 150]
ANCH = [0, 2, 36, 37, 50, 106, 300, 647, 648, 652, 700, 801]
LENS = [2, 3, 1, 4, 7, 0, 32, 16, 7, 5, 16, 7]
MODES = [TTT, BLOCK, TTT, BLOCK, TTT, TTT, TTT, BLOCK, TTT, TTT, BLOCK, TTT]


def _strided(hq, hkv):
    return np.arange(hq, dtype=np.int32) % hkv


def _permuted(hq, hkv, seed):
    m = np.repeat(np.arange(hkv, dtype=np.int32), hq // hkv)
    return np.random.default_rng(seed).permutation(m).astype(np.int32)


def _case(name, dtype, hq, hkv, d, kv_head_of=None, scale=0.0, std=1.0):
    w = custom(name, dtype, hq, hkv, d, SEQS, None, ANCH, LENS, MODES, std=std, seed=7)
    w.kv_head_of = kv_head_of
    w.softmax_scale = scale
    return w


CASES = {
    # strided maps h % Hkv
    "strided_g4_d128": lambda: _case("s4", "bf16", 16, 4, 128, _strided(16, 4)),
    "strided_g8_d64": lambda: _case("s8", "bf16", 16, 2, 64, _strided(16, 2)),
    # group sizes that do not divide 128 (padding rows in every tile)
    "g3_d128": lambda: _case("g3", "bf16", 12, 4, 128),
    "g3_d64_strided": lambda: _case("g3s", "bf16", 12, 4, 64, _strided(12, 4)),
    "g5_d64": lambda: _case("g5", "bf16", 20, 4, 64),
    "g5_d128_permuted": lambda: _case("g5p", "bf16", 20, 4, 128, _permuted(20, 4, 1)),
    "g7_d128": lambda: _case("g7", "bf16", 28, 4, 128),
    "g7_d64_permuted": lambda: _case("g7p", "bf16", 28, 4, 64, _permuted(28, 4, 2)),
    # softmax scale other than 1/sqrt(d)
    "scale0.3_d128": lambda: _case("sc", "bf16", 8, 2, 128, scale=0.3, std=0.5),
    "scale0.3_d64_strided": lambda: _case("scs", "bf16", 16, 2, 64, _strided(16, 2), scale=0.3, std=0.5),
    "scale0.05_g3_d128": lambda: _case("scg", "bf16", 12, 4, 128, _strided(12, 4), scale=0.05),
    # float32 element type with a strided G = 3 map and a scale
    "f32_g3_strided_scale": lambda: _case("f3", "f32", 6, 2, 128, _strided(6, 2), scale=0.2),
    # more kv heads than the eight XCDs (the work counters: two home heads per
    # XCD for some XCDs, one for others)
    "hkv12_g2_d128": lambda: _case("h12", "bf16", 24, 12, 128),
    "hkv16_g1_d64_strided": lambda: _case("h16", "bf16", 16, 16, 64, _strided(16, 16)),
}


def _fwd_bwd(w, t):
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    o, lse, ob, lseb = sda.fwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"])
    grads = sda.bwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"], o, lse, ob, lseb, g["do"], g["dob"])
    torch.cuda.synchronize()
    return plan, g, (o, lse, ob, lseb), dict(zip(GRADS, grads))


@pytest.mark.parametrize("name", list(CASES))
def test_head_map_group_size_scale_fwd_bwd_parity(name):
    w = CASES[name]()
    say(f"[headmap] {name}: Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} dtype={w.dtype} "
        f"map={None if w.kv_head_of is None else w.kv_head_of.tolist()} scale={w.softmax_scale} "
        f"N={w.N} Rb={w.Rb}")
    t = make_inputs(w, grads=True)
    _, _, (o, lse, ob, lseb), got = _fwd_bwd(w, t)
    p = oracle.Problem.from_workload(w)
    t64 = f64_all(t)
    ref = oracle.forward(p, t64)
    check_out("o", host(o), ref["o"], w.dtype, "o")
    check_out("ob", host(ob), ref["ob"], w.dtype, "o")
    check_out("lse", host(lse), ref["lse"], w.dtype, "lse")
    check_out("lseb", host(lseb), ref["lseb"], w.dtype, "lse")
    gref = oracle.backward(p, t64, ref)
    for k_ in GRADS:
        check_out(k_, host(got[k_]), gref[k_], w.dtype, "grad")


def test_head_map_changes_the_result():
    """The strided map is not a relabelling the kernels could ignore: with it the
    output differs from the contiguous map's by far more than the tolerance."""
    w = CASES["strided_g4_d128"]()
    a = _fwd_bwd(w, make_inputs(w, grads=True))[2][0]
    w.kv_head_of = None
    b = _fwd_bwd(w, make_inputs(w, grads=True))[2][0]
    diff = float((a.float() - b.float()).abs().max())
    say(f"  strided vs contiguous map: max |dO| = {diff:.3f}")
    assert diff > 0.1


def test_split_path_with_strided_map():
    """ba_main_fwd and ba_branch_local_fwd partials and their lse_merge, strided map, G = 3."""
    w = _case("sp", "bf16", 12, 4, 128, _strided(12, 4), scale=0.1)
    say(f"[headmap split] Hq=12 Hkv=4 strided scale=0.1 N={w.N} Rb={w.Rb}")
    t = make_inputs(w)
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    hq, d = w.num_q_heads, w.head_dim
    o = torch.empty_like(g["q"])
    lse = torch.empty((hq, w.Nq), dtype=torch.float32, device="cuda")
    o_pre = torch.empty((w.Rb, hq, d), dtype=torch.float32, device="cuda")
    lse_pre = torch.empty((hq, w.Rb), dtype=torch.float32, device="cuda")
    o_loc, lse_loc = torch.empty_like(o_pre), torch.empty_like(lse_pre)
    ws = sda.workspace(plan, 2)
    sda.ba_main_fwd(plan, g["q"], g["qb"], g["k"], g["v"], o, lse, o_pre, lse_pre, ws)
    sda.ba_branch_local_fwd(plan, g["qb"], g["kb"], g["vb"], o_loc, lse_loc, ws)
    ob = torch.empty((w.Rb, hq, d), dtype=torch.float32, device="cuda")
    lseb = torch.empty_like(lse_pre)
    sda.lse_merge(o_pre, lse_pre, o_loc, lse_loc, ob, lseb)
    torch.cuda.synchronize()
    merged, part = oracle.split_forward(oracle.Problem.from_workload(w), f64_all(t))
    check_out("o_main", host(o), part["o_main"], "bf16", "o")
    check_out("lse_main", host(lse), part["lse_main"], "bf16", "lse")
    check_out("ob_main", host(o_pre), part["ob_main"], "bf16", "o")
    check_out("lseb_main", host(lse_pre), part["lseb_main"], "bf16", "lse")
    check_out("ob_loc", host(o_loc), part["ob_loc"], "bf16", "o")
    check_out("lseb_loc", host(lse_loc), part["lseb_loc"], "bf16", "lse")
    check_out("ob_merged", host(ob), merged["ob"], "bf16", "o")
    check_out("lseb_merged", host(lseb), merged["lseb"], "bf16", "lse")


@pytest.mark.parametrize("d", [128, 64])
def test_ring_step_with_strided_map(d):
    """Ragged windows through ba_ring_step_fwd with a strided G = 5 map and a scale."""
    w = _case("rs", "bf16", 20, 4, d, _strided(20, 4), scale=0.11)
    windows = [(400, 803), (0, 37), (37, 200), (200, 400), (803, 803)]
    say(f"[headmap ring] d={d} Hq=20 Hkv=4 strided N={w.N} windows={windows}")
    t = make_inputs(w)
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    R, hq = w.Nq + w.Rb, w.num_q_heads
    o_run = torch.zeros((R, hq, d), dtype=torch.float32, device="cuda")
    lse_run = torch.full((hq, R), float("-inf"), dtype=torch.float32, device="cuda")
    ws = sda.workspace(plan, 2)
    for lo, hi in windows:
        sda.ba_ring_step_fwd(plan, g["q"], g["qb"], g["k"][lo:hi].clone(), g["v"][lo:hi].clone(), lo, hi,
                             o_run, lse_run, ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.ring_forward(oracle.Problem.from_workload(w), f64_all(t), windows)
    check_out("o_run", host(o_run), o_ref, "bf16", "o")
    check_out("lse_run", host(lse_run), l_ref, "bf16", "lse")


@pytest.mark.timeout(600)
def test_full_size_strided_map_sampled_rows():
    """The 16K Qwen3-like workload with a strided head map: sampled rows against
    the oracle's row evaluation."""
    from gpu_util import sample_rows, gather_rows, oracle_rows
    w = W.get("qwen3_8b_16k")
    w.kv_head_of = _strided(32, 8)
    say(f"[headmap full] {w.name} strided map")
    t = make_inputs(w)
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    o, lse, ob, lseb = sda.fwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"])
    torch.cuda.synchronize()
    rows = sample_rows(w, n_random=16, seed=3)
    O, L = gather_rows(o, ob, lse, lseb, rows, w.Nq)
    Oref, Lref = oracle_rows(w, t, rows)
    check_out("o(sampled)", O, Oref, "bf16", "o")
    check_out("lse(sampled)", L, Lref, "bf16", "lse")
