"""GPU parity of the backward pass against the CPU oracle (MI355X only).

Reduced-size workloads: every gradient element by element against the dense
fp64 oracle. Full-size workloads: dQ of sampled rows (exact per row), dK/dV of
the last keys of a sequence (every row that sees them is summed exactly), and
the gradient-sum identities over whole tensors.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads.configs import custom, TTT, BLOCK
from workloads.inputs import make_inputs, to_f32

from gpu_util import say, dev, host, check_out, f64_all, f32_views, sample_rows

pytestmark = pytest.mark.gpu

sda = pytest.importorskip("speculative_draft_branch_amd")

GRADS = ("dq", "dk", "dv", "dqb", "dkb", "dvb")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, t):
    plan = sda.Plan.from_workload(w)
    g = {k: dev(v) for k, v in t.items()}
    o, lse, ob, lseb = sda.fwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"])
    grads = sda.bwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"], o, lse, ob, lseb, g["do"], g["dob"])
    torch.cuda.synchronize()
    return plan, g, (o, lse, ob, lseb), dict(zip(GRADS, grads))


EDGE = {
    "mixed_bf16_d128": lambda: custom("m", "bf16", 4, 2, 128, [37, 70, 5, 150], None,
                                      [0, 2, 36, 37, 50, 106, 107, 111, 200, 261], [2, 3, 1, 4, 3, 0, 2, 16, 7, 5],
                                      [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK, BLOCK, TTT, TTT], std=1.0, seed=4),
    "mixed_f32_d128": lambda: custom("m", "f32", 4, 2, 128, [37, 70, 5, 150], None,
                                     [0, 2, 36, 37, 50, 106, 107, 111, 200, 261], [2, 3, 1, 4, 3, 0, 2, 16, 7, 5],
                                     [TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK, BLOCK, TTT, TTT], std=1.0, seed=4),
    "qsubset_bf16_d64": lambda: custom("q", "bf16", 16, 2, 64, [300, 41], list(range(5, 341, 7)),
                                       list(range(3, 341, 11)), [7] * 31, [TTT] * 31, std=1.0, seed=4),
    "nobranch_bf16_d128": lambda: custom("n", "bf16", 8, 8, 128, [129, 1, 64, 200], None, [], [], [], seed=4),
    "branches_only_bf16": lambda: custom("b", "bf16", 4, 1, 128, [90], [], [0, 17, 89], [5, 16, 32],
                                         [TTT, BLOCK, TTT], seed=4),
    # no GQA with 32-row branches on every third token: branch keys of a unit span
    # several 64-key tiles (the dq kernel's branch tiles)
    "g1_long_branches_bf16_d128": lambda: custom("g1", "bf16", 4, 4, 128, [301, 197], None, list(range(1, 498, 3)),
                                                 [32 - (i % 3) for i in range(166)],
                                                 [TTT if i % 2 else BLOCK for i in range(166)], std=1.0, seed=4),
    "g1_long_branches_bf16_d64": lambda: custom("g1", "bf16", 4, 4, 64, [301, 197], None, list(range(1, 498, 3)),
                                                [32 - (i % 3) for i in range(166)],
                                                [TTT if i % 2 else BLOCK for i in range(166)], std=1.0, seed=4),
    # branches longer than 16 rows in both modes at GQA 8:1, d=64 (two 16-key blocks per branch)
    "long_branches_bf16_d64": lambda: custom("l", "bf16", 16, 2, 64, [120, 60], None, [0, 40, 119, 130, 179],
                                             [17, 32, 20, 24, 9], [BLOCK, BLOCK, TTT, TTT, BLOCK], std=1.0, seed=4),
}

DENSE = ["tiny_f32", "qwen3_8b_16k_div16", "ctx256k_rank3_chunk64", "ctx256k_rank3_chunk80", "dflash_64k_1024",
         "gptoss_128k_mixed_2048"]


def _dense_check(w):
    say(f"[bwd dense] {w.name}: N={w.N} Nq={w.Nq} Rb={w.Rb} dtype={w.dtype} d={w.head_dim}")
    t = make_inputs(w, grads=True)
    _, _, _, got = _run(w, t)
    p = oracle.Problem.from_workload(w)
    t64 = f64_all(t)
    ref = oracle.backward(p, t64, oracle.forward(p, t64))
    for name in GRADS:
        check_out(name, host(got[name]), ref[name], w.dtype, "grad")


@pytest.mark.parametrize("name", DENSE)
def test_backward_dense_parity(name):
    _dense_check(W.get(name))


@pytest.mark.parametrize("name", list(EDGE))
def test_backward_edge_cases(name):
    _dense_check(EDGE[name]())


def _identity_checks(w, t, got):
    """Per kv head: sum over all key rows of dK is 0; sum of dV equals the sum of
    dO over the group's rows. Bounds scale with the bf16 rounding of the terms."""
    G = w.num_q_heads // w.num_kv_heads
    for g in range(w.num_kv_heads):
        dk = torch.cat([got["dk"][:, g].float(), got["dkb"][:, g].float()]).double()
        dv = torch.cat([got["dv"][:, g].float(), got["dvb"][:, g].float()]).double()
        n = dk.shape[0]
        sdk = dk.sum(0)
        bound_k = 8.0 * (n ** 0.5) * dk.pow(2).mean().sqrt().item() * 2.0 ** -8
        assert sdk.abs().max().item() <= bound_k + 1e-3, (g, sdk.abs().max().item(), bound_k)
        heads = slice(g * G, (g + 1) * G)
        do_sum = (torch.from_numpy(to_f32(t["do"][:, heads]).astype(np.float64)).sum((0, 1))
                  + torch.from_numpy(to_f32(t["dob"][:, heads]).astype(np.float64)).sum((0, 1)))
        err = (dv.sum(0).cpu() - do_sum).abs().max().item()
        bound_v = 8.0 * (n ** 0.5) * dv.pow(2).mean().sqrt().item() * 2.0 ** -8
        say(f"  kv head {g}: |sum dK|={sdk.abs().max().item():.3e} (bound {bound_k:.3e}), "
            f"|sum dV - sum dO|={err:.3e} (bound {bound_v:.3e})")
        assert err <= bound_v + 1e-3


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["ctx256k_rank3", "gptoss_128k_mixed", "qwen3_8b_16k", "dflash_64k"])
def test_backward_full_size(name):
    w = W.get(name)
    say(f"[bwd full] {w.name}: N={w.N} Nq={w.Nq} Rb={w.Rb}")
    t = make_inputs(w, grads=True)
    plan, g, _, got = _run(w, t)
    for k_ in GRADS:
        assert torch.isfinite(got[k_].float()).all(), k_
    _identity_checks(w, t, got)
    p = oracle.Problem.from_workload(w)
    tv = f32_views(t)
    # dQ of sampled rows, exact per row
    rows = sample_rows(w, n_random=8, seed=9)
    say(f"  dq of {len(rows)} sampled rows")
    ref = oracle.backward_rows(p, tv, rows)
    Nq = w.Nq
    got_rows = np.stack([host(got["dq"][r]) if r < Nq else host(got["dqb"][r - Nq]) for r in rows])
    check_out("dq(sampled rows)", got_rows, ref, "bf16", "grad")
    # dK/dV of the last 8 keys of the last sequence: sum over every row that sees them
    s = w.num_seqs - 1
    lo, hi = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
    u0 = hi - 8
    see = [i for i in range(Nq) if u0 <= int(w.q_pos[i]) < hi]
    for m in range(w.A):
        a = int(w.anchors[m])
        if u0 <= a < hi:
            see += [Nq + b for b in range(int(w.cu_branch[m]), int(w.cu_branch[m + 1]))]
    acc = {"dk": np.zeros((w.N, w.num_kv_heads, w.head_dim)), "dv": np.zeros((w.N, w.num_kv_heads, w.head_dim)),
           "dkb": np.zeros((w.Rb, w.num_kv_heads, w.head_dim)), "dvb": np.zeros((w.Rb, w.num_kv_heads, w.head_dim))}
    say(f"  exact dK/dV of keys {u0}..{hi - 1}: {len(see)} rows")
    for c0 in range(0, len(see), 16):
        oracle.backward_rows(p, tv, see[c0:c0 + 16], acc)
        say(f"    oracle rows {c0 + len(see[c0:c0 + 16])}/{len(see)}")
    check_out("dk(last keys)", host(got["dk"][u0:hi]), acc["dk"][u0:hi], "bf16", "grad")
    check_out("dv(last keys)", host(got["dv"][u0:hi]), acc["dv"][u0:hi], "bf16", "grad")


def test_backward_is_deterministic():
    """Every gradient element is written by one workgroup, or (plans with split
    key tiles) is the sum of at most two float32 atomic adds into zero, which
    does not depend on their order, so two runs agree bitwise."""
    w = W.get("ctx256k_rank3_chunk64")
    t = make_inputs(w, grads=True)
    _, _, _, a = _run(w, t)
    _, _, _, b = _run(w, t)
    for k_ in GRADS:
        assert torch.equal(a[k_], b[k_]), k_
