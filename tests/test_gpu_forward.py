"""GPU parity of the forward pass against the CPU oracle (MI355X only).

Reduced-size workloads are compared element by element with the dense fp64
oracle; the full-size workloads on sampled rows (each row's full visible key
set) and on full-scale closed forms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads.configs import custom, TTT, BLOCK
from workloads.inputs import make_inputs, to_f32, bf16_round_bits

from gpu_util import (say, dev, host, check_out, f64_all, sample_rows, gather_rows, oracle_rows, TOL)

pytestmark = pytest.mark.gpu

sda = pytest.importorskip("speculative_draft_branch_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _edge(name, dtype, d, hq, hkv, seqs, q_pos, anchors, lens, modes, std=1.0, qk_scale=1.0):
    w = custom(name, dtype, hq, hkv, d, seqs, q_pos, anchors, lens, modes, std=std, seed=3)
    w.qk_scale = qk_scale
    return w


def make_inputs_scaled(w, grads=False):
    """Seeded inputs; Q and K (main and branch) multiplied by the workload's
    qk_scale, a power of two, so the bf16 values stay exact."""
    t = make_inputs(w, grads=grads)
    s = getattr(w, "qk_scale", 1.0)
    if s != 1.0:
        for key in ("q", "qb", "k", "kb"):
            x = to_f32(t[key]) * np.float32(s)
            t[key] = bf16_round_bits(x) if t[key].dtype == np.uint16 else x
    return t


EDGE = {
    # every mode, a zero-length branch, anchors at sequence starts, GQA 2:1, ragged tails
    "mixed_bf16_d128": lambda: _edge("m", "bf16", 128, 4, 2, [37, 70, 5, 150], None,
                                     [0, 2, 36, 37, 50, 106, 107, 111, 200, 261], [2, 3, 1, 4, 3, 0, 2, 16, 7, 5],
                                     [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK, BLOCK, TTT, TTT]),
    "mixed_f32_d64": lambda: _edge("m", "f32", 64, 4, 2, [37, 70, 5, 150], None,
                                   [0, 2, 36, 37, 50, 106, 107, 111, 200, 261], [2, 3, 1, 4, 3, 0, 2, 16, 7, 5],
                                   [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK, BLOCK, TTT, TTT]),
    # a subset of positions are queries; GQA 8:1 at d=64
    "qsubset_bf16_d64": lambda: _edge("q", "bf16", 64, 16, 2, [300, 41], list(range(5, 341, 7)),
                                      list(range(3, 341, 11)), [7] * len(range(3, 341, 11)),
                                      [TTT] * len(range(3, 341, 11))),
    # no branches at all (plain packed causal attention)
    "nobranch_bf16_d128": lambda: _edge("n", "bf16", 128, 8, 8, [129, 1, 64, 200], None, [], [], []),
    # single-token sequences and an empty sequence
    "tiny_seqs_f32_d128": lambda: _edge("t", "f32", 128, 2, 1, [1, 1, 0, 3, 1], None, [0, 1, 3, 5],
                                        [2, 1, 32, 3], [TTT, BLOCK, BLOCK, TTT]),
    # no main query rows, branches only
    "branches_only_bf16": lambda: _edge("b", "bf16", 128, 4, 1, [90], [], [0, 17, 89], [5, 16, 32],
                                        [TTT, BLOCK, TTT]),
    # Q and K x4 (N(0,1)*0.5 inputs): a peaked softmax exercises the online rescaling
    "peaked_bf16_d128": lambda: _edge("p", "bf16", 128, 4, 2, [300, 211], None, list(range(0, 511, 3)),
                                      [7] * len(range(0, 511, 3)), [TTT] * len(range(0, 511, 3)), std=0.5,
                                      qk_scale=4.0),
    # branches longer than 16 rows in both modes at GQA 8:1, d=64 (two 16-key blocks per branch)
    "long_branches_bf16_d64": lambda: _edge("l", "bf16", 64, 16, 2, [120, 60], None, [0, 40, 119, 130, 179],
                                            [17, 32, 20, 24, 9], [BLOCK, BLOCK, TTT, TTT, BLOCK]),
    # no GQA (128 base rows per tile) with 32-row branches of both modes on every
    # third token: a unit's branch keys span three or four 64-key tiles and
    # start off a tile boundary
    "g1_long_branches_bf16_d128": lambda: _edge("g1", "bf16", 128, 4, 4, [301, 197], None, list(range(1, 498, 3)),
                                                [32 - (i % 3) for i in range(166)],
                                                [TTT if i % 2 else BLOCK for i in range(166)]),
    "g1_long_branches_bf16_d64": lambda: _edge("g1", "bf16", 64, 4, 4, [301, 197], None, list(range(1, 498, 3)),
                                               [32 - (i % 3) for i in range(166)],
                                               [TTT if i % 2 else BLOCK for i in range(166)]),
    "peaked_bf16_d64": lambda: _edge("p", "bf16", 64, 16, 2, [700], None, list(range(0, 700, 16)),
                                     [16] * len(range(0, 700, 16)), [BLOCK] * len(range(0, 700, 16)), std=0.5,
                                     qk_scale=4.0),
}

DENSE = ["tiny_f32", "qwen3_8b_16k_div16", "ctx256k_rank3_chunk64", "ctx256k_rank3_chunk80", "dflash_64k_1024",
         "gptoss_128k_mixed_2048"]


def _run_fwd(w, t):
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    o, lse, ob, lseb = sda.fwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"])
    torch.cuda.synchronize()
    return plan, g, (o, lse, ob, lseb)


def _dense_check(w):
    say(f"[fwd dense] {w.name}: N={w.N} Nq={w.Nq} Rb={w.Rb} dtype={w.dtype} d={w.head_dim}")
    t = make_inputs_scaled(w)
    _, _, (o, lse, ob, lseb) = _run_fwd(w, t)
    ref = oracle.forward(oracle.Problem.from_workload(w), f64_all(t))
    check_out("o", host(o), ref["o"], w.dtype, "o")
    check_out("ob", host(ob), ref["ob"], w.dtype, "o")
    check_out("lse", host(lse), ref["lse"], w.dtype, "lse")
    check_out("lseb", host(lseb), ref["lseb"], w.dtype, "lse")


@pytest.mark.parametrize("name", DENSE)
def test_forward_dense_parity(name):
    _dense_check(W.get(name))


@pytest.mark.parametrize("name", list(EDGE))
def test_forward_edge_cases(name):
    _dense_check(EDGE[name]())


@pytest.mark.parametrize("d", [128, 64])
def test_forward_rising_scores_force_rescale(d):
    """Scores that rise by far more than 2^64 (in units of exp2) along each
    sequence, so the softmax reference taken from the first key tile must be
    raised several times. Q = 0.5 and K rows = a(pos) * 1 with a = (pos // 16) / 2:
    every product and sum is exact in bf16 / fp32, and the oracle decides."""
    w = _edge("r", "bf16", d, 4, 2, [600, 70], None, [5, 300, 599, 650], [7, 3, 16, 5],
              [TTT, BLOCK, TTT, BLOCK])
    t = make_inputs(w)
    t["q"] = bf16_round_bits(np.full(to_f32(t["q"]).shape, 0.5, np.float32))
    t["qb"] = bf16_round_bits(np.full(to_f32(t["qb"]).shape, 0.5, np.float32))
    k = np.zeros(to_f32(t["k"]).shape, np.float32)
    for s0, s1 in zip(w.cu_seqlens[:-1], w.cu_seqlens[1:]):
        pos = np.arange(s1 - s0)
        k[s0:s1] = ((pos // 16) / 2.0).astype(np.float32)[:, None, None]
    t["k"] = bf16_round_bits(k)
    grow = float(k.max()) * 0.5 * d / math.sqrt(d) / math.log(2.0)  # largest score, log2 units
    say(f"[fwd rescale] d={d}: largest score {grow:.1f} (log2 units)")
    assert grow > 96  # the first key tile tops out near 12 (d = 128) or 9 (d = 64)
    _, _, (o, lse, ob, lseb) = _run_fwd(w, t)
    ref = oracle.forward(oracle.Problem.from_workload(w), f64_all(t))
    check_out("o", host(o), ref["o"], "bf16", "o")
    check_out("ob", host(ob), ref["ob"], "bf16", "o")
    check_out("lse", host(lse), ref["lse"], "bf16", "lse")
    check_out("lseb", host(lseb), ref["lseb"], "bf16", "lse")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_8b_16k", "dflash_64k", "ctx256k_rank3", "gptoss_128k_mixed"])
def test_forward_full_size_sampled_rows(name):
    w = W.get(name)
    say(f"[fwd sampled] {w.name}: N={w.N} Nq={w.Nq} Rb={w.Rb}")
    t = make_inputs(w)
    _, _, (o, lse, ob, lseb) = _run_fwd(w, t)
    rows = sample_rows(w, n_random=12 if name == "ctx256k_rank3" else 20)
    O, L = gather_rows(o, ob, lse, lseb, rows, w.Nq)
    Oref, Lref = oracle_rows(w, t, rows)
    check_out("o(sampled)", O, Oref, w.dtype, "o")
    check_out("lse(sampled)", L, Lref, w.dtype, "lse")
    # whole-tensor sanity at full size: finite everywhere, LSE >= the largest
    # single score bound is not checkable cheaply, but LSE must be finite
    assert torch.isfinite(lse).all() and torch.isfinite(lseb).all()
    assert torch.isfinite(o.float()).all() and torch.isfinite(ob.float()).all()


@pytest.mark.timeout(600)
def test_zero_keys_closed_form_full_scale():
    """K = Kb = 0 at the 256K share: every score is 0, so LSE_r = ln n_r exactly
    for every row (n_r from the structure alone) and O_r is the mean of the
    visible V rows (checked on sampled rows with float64 prefix sums)."""
    w = W.get("ctx256k_rank3")
    say(f"[fwd K=0] {w.name}")
    t = make_inputs(w)
    t["k"][:] = 0
    t["kb"][:] = 0
    plan, g, (o, lse, ob, lseb) = _run_fwd(w, t)
    # n_r closed forms: main t - cu[s] + 1; TTT query j: a - cu[s] + 1 + j
    n_main = w.q_pos.astype(np.float64) + 1.0          # one sequence starting at 0
    L = np.diff(w.cu_branch)
    j = np.arange(w.Rb) - np.repeat(w.cu_branch[:-1], L) + 1
    n_br = np.repeat(w.anchors.astype(np.float64), L) + 1.0 + j
    lse_h, lseb_h = host(lse), host(lseb)
    err = max(np.abs(lse_h - np.log(n_main)[None]).max(), np.abs(lseb_h - np.log(n_br)[None]).max())
    say(f"  lse vs ln(n): max_abs={err:.3e}")
    assert err <= TOL["bf16"]["lse_abs"]
    # O for sampled rows: mean of the visible V rows
    from workloads.inputs import to_f32
    v = to_f32(t["v"]).astype(np.float64)
    pre = np.concatenate([np.zeros((1,) + v.shape[1:]), np.cumsum(v, axis=0)])
    vb = to_f32(t["vb"]).astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    rows = sample_rows(w, n_random=64, seed=5)
    O, _ = gather_rows(o, ob, lse, lseb, rows, w.Nq)
    ref = np.zeros_like(O)
    for i, r in enumerate(rows):
        if r < w.Nq:
            tt = int(w.q_pos[r])
            tot, n = pre[tt + 1], tt + 1
        else:
            b = r - w.Nq
            m = int(np.searchsorted(w.cu_branch, b, side="right") - 1)
            a, b0 = int(w.anchors[m]), int(w.cu_branch[m])
            tot, n = pre[a + 1] + vb[b0:b + 1].sum(axis=0), a + 1 + (b - b0 + 1)
        ref[i] = np.repeat(tot / n, G, axis=0)
    check_out("o(K=0, sampled)", O, ref, "bf16", "o")


def test_split_path_pieces_match_oracle_partials():
    """ba_main_fwd partials, ba_branch_local_fwd partials and lse_merge of the two,
    each against the oracle's split of the same problem."""
    w = W.get("ctx256k_rank3_chunk80")
    say(f"[split] {w.name}")
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


def test_lse_merge_against_oracle_and_edge_cases():
    rng = np.random.default_rng(11)
    rows, heads, d = 1000, 3, 128
    oa, ob = rng.standard_normal((rows, heads, d)), rng.standard_normal((rows, heads, d))
    la, lb = rng.standard_normal((heads, rows)) * 4, rng.standard_normal((heads, rows)) * 4
    la[0, :10] = -np.inf               # empty partial a
    oa[:10, 0] = 0.0
    lb[1, 5:20] = -np.inf              # empty partial b
    ob[5:20, 1] = 0.0
    la[2, 30:40] = lb[2, 30:40] = -np.inf   # both empty
    oa[30:40, 2] = ob[30:40, 2] = 0.0
    oa, ob, la, lb = (x.astype(np.float32) for x in (oa, ob, la, lb))
    ref_o, ref_l = oracle.lse_merge(oa, la, ob, lb)
    ga, gb = torch.from_numpy(oa).cuda(), torch.from_numpy(ob).cuda()
    gla, glb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    out = torch.empty_like(ga)
    lo = torch.empty_like(gla)
    sda.lse_merge(ga, gla, gb, glb, out, lo)
    torch.cuda.synchronize()
    got_o, got_l = host(out), host(lo)
    assert not np.isnan(got_o).any() and not np.isnan(got_l).any()
    assert np.all(np.isneginf(got_l[2, 30:40])) and np.all(got_o[30:40, 2] == 0)
    fin = np.isfinite(ref_l)
    assert np.abs(got_l[fin] - ref_l[fin]).max() <= 1e-5
    assert np.abs(got_o - ref_o).max() <= 1e-5
    # in place on (o_a, lse_a), bf16 output variant
    outb = torch.empty((rows, heads, d), dtype=torch.bfloat16, device="cuda")
    sda.lse_merge(ga, gla, gb, glb, outb, gla)
    sda.lse_merge(ga, torch.from_numpy(la).cuda(), gb, glb, ga, torch.from_numpy(la).cuda())
    torch.cuda.synchronize()
    assert np.abs(host(outb) - ref_o).max() <= 2e-2
    assert np.abs(host(ga) - ref_o).max() <= 1e-5
    assert np.abs(host(gla)[fin] - ref_l[fin]).max() <= 1e-5


def test_forward_is_deterministic():
    w = W.get("qwen3_8b_16k_div16")
    t = make_inputs(w)
    _, g, a = _run_fwd(w, t)
    _, _, b = _run_fwd(w, t)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
