"""Pins of the CPU oracle against facts that do not come from the oracle itself:
a hand-worked mask fixture, an independent fp64 brute force, library attention
(torch SDPA), closed forms (K = 0, V = const, a peaked softmax), merge
identities, locality, finite differences, autograd and gradient identities.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import Problem
import workloads as W
from workloads.configs import custom, TTT, BLOCK
from workloads.inputs import make_inputs, to_f32
import brute_force

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(t):
    return {k: to_f32(v).astype(np.float64) for k, v in t.items()}


def _tiny(name="t", hq=4, hkv=2, d=8, seqs=(5, 7, 4), q_pos=None, anchors=(0, 2, 5, 6, 11, 12, 15),
          lens=(2, 3, 1, 4, 3, 0, 2), modes=(TTT, BLOCK, TTT, BLOCK, TTT, TTT, BLOCK), seed=1, dtype="f32"):
    return custom(name, dtype, hq, hkv, d, list(seqs), q_pos, list(anchors), list(lens), list(modes),
                  std=1.0, seed=seed, passes=("fwd", "bwd"))


TINY_CASES = {
    # several sequences, every mode, a zero-length branch, anchors at sequence starts, GQA 2:1
    "mixed": dict(),
    # only some main positions are queries
    "qsubset": dict(q_pos=[1, 4, 5, 9, 13, 15]),
    # no GQA, a single sequence, TTT everywhere
    "ttt_all": dict(hq=2, hkv=2, seqs=(9,), anchors=tuple(range(9)), lens=(3,) * 9, modes=(TTT,) * 9),
    # blocks only, GQA 4:1
    "blocks": dict(hq=4, hkv=1, seqs=(8, 8), anchors=(3, 7, 11, 15), lens=(4, 4, 4, 4), modes=(BLOCK,) * 4),
    # no branches at all
    "nobranch": dict(anchors=(), lens=(), modes=()),
    # single-token sequences
    "single_tokens": dict(seqs=(1, 1, 3, 1), anchors=(0, 1, 4), lens=(2, 1, 2), modes=(TTT, BLOCK, TTT)),
}


def _case(name):
    return _tiny(name, **TINY_CASES[name])


# --------------------------------------------------------------------------
# mask

def _read_golden_mask():
    hdr, rows = {}, {}
    with open(os.path.join(GOLDEN, "mask_tiny.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":")
            vals = [int(x) for x in val.split()]
            if key.isdigit():
                rows[int(key)] = vals
            else:
                hdr[key] = vals
    return hdr, rows


def test_mask_matches_hand_worked_fixture():
    hdr, rows = _read_golden_mask()
    p = Problem(1, 1, 4, hdr["cu_seqlens"], hdr["q_pos"], hdr["anchors"], hdr["cu_branch"], hdr["modes"])
    mask = oracle.dense_mask(p)
    assert mask.shape == (14, 14)
    for r, keys in rows.items():
        assert sorted(np.nonzero(mask[r])[0].tolist()) == keys, r
    # and the independent key walk agrees with the fixture too
    for r, keys in rows.items():
        vk = brute_force.visible_keys(hdr["cu_seqlens"], hdr["q_pos"], hdr["anchors"], hdr["cu_branch"],
                                      hdr["modes"], r)
        got = sorted(u if kind == "main" else 7 + u for kind, u in vk)
        assert got == keys, r


@pytest.mark.parametrize("name", list(TINY_CASES))
def test_mask_matches_key_walk(name):
    w = _case(name)
    p = Problem.from_workload(w)
    mask = oracle.dense_mask(p)
    for r in range(p.Nq + p.Rb):
        vk = brute_force.visible_keys(w.cu_seqlens, w.q_pos, w.anchors, w.cu_branch, w.modes, r)
        got = sorted(u if kind == "main" else p.N + u for kind, u in vk)
        assert got == np.nonzero(mask[r])[0].tolist()


# --------------------------------------------------------------------------
# forward vs brute force and library attention

@pytest.mark.parametrize("name", list(TINY_CASES))
def test_forward_matches_brute_force(name):
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    f = oracle.forward(p, t)
    bf = brute_force.brute_forward(w.cu_seqlens, w.q_pos, w.anchors, w.cu_branch, w.modes,
                                   t["q"], t["k"], t["v"], t["qb"], t["kb"], t["vb"],
                                   w.num_q_heads // w.num_kv_heads, 1.0 / math.sqrt(w.head_dim))
    for r, per_head in enumerate(bf):
        for h, (o, lse) in enumerate(per_head):
            if r < p.Nq:
                go, gl = f["o"][r, h], f["lse"][h, r]
            else:
                go, gl = f["ob"][r - p.Nq, h], f["lseb"][h, r - p.Nq]
            np.testing.assert_allclose(go, o, rtol=0, atol=1e-12)
            assert abs(gl - lse) < 1e-12


# Explicit GQA head maps and a softmax scale other than 1/sqrt(d): q head h reads
# kv head kv_head_of[h]. Group sizes 3 and 5 (not powers of two), a strided map,
# a seeded permutation.
HEADMAP_CASES = {
    "strided_g3": dict(hq=6, hkv=2, kv_head_of=[0, 1, 0, 1, 0, 1], scale=0.37),
    "perm_g5": dict(hq=10, hkv=2, kv_head_of=[1, 0, 0, 1, 1, 0, 1, 0, 0, 1], scale=None),
    "contig_g3_scale": dict(hq=3, hkv=1, kv_head_of=None, scale=1.9),
}


def _headmap_case(name):
    c = HEADMAP_CASES[name]
    w = _tiny(name, hq=c["hq"], hkv=c["hkv"], d=8)
    w.kv_head_of = None if c["kv_head_of"] is None else np.asarray(c["kv_head_of"], np.int32)
    w.softmax_scale = c["scale"] or 0.0
    return w


@pytest.mark.parametrize("name", list(HEADMAP_CASES))
def test_forward_with_head_map_and_scale_matches_brute_force(name):
    w = _headmap_case(name)
    p = Problem.from_workload(w)
    c = HEADMAP_CASES[name]
    scale = c["scale"] or 1.0 / math.sqrt(w.head_dim)
    assert p.scale == scale
    kvmap = c["kv_head_of"] if c["kv_head_of"] is not None else w.num_q_heads // w.num_kv_heads
    t = _f64(make_inputs(w))
    f = oracle.forward(p, t)
    bf = brute_force.brute_forward(w.cu_seqlens, w.q_pos, w.anchors, w.cu_branch, w.modes,
                                   t["q"], t["k"], t["v"], t["qb"], t["kb"], t["vb"], kvmap, scale)
    for r, per_head in enumerate(bf):
        for h, (o, lse) in enumerate(per_head):
            if r < p.Nq:
                go, gl = f["o"][r, h], f["lse"][h, r]
            else:
                go, gl = f["ob"][r - p.Nq, h], f["lseb"][h, r - p.Nq]
            np.testing.assert_allclose(go, o, rtol=0, atol=1e-12)
            assert abs(gl - lse) < 1e-12


@pytest.mark.parametrize("name", list(HEADMAP_CASES))
def test_backward_with_head_map_and_scale_matches_autograd(name):
    """fp64 autograd of masked softmax attention, K/V expanded per q head by the map."""
    w = _headmap_case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w, grads=True))
    g = oracle.backward(p, t, oracle.forward(p, t))
    mask = torch.from_numpy(oracle.dense_mask(p))
    Q = torch.tensor(np.concatenate([t["q"], t["qb"]]), requires_grad=True)
    K = torch.tensor(np.concatenate([t["k"], t["kb"]]), requires_grad=True)
    V = torch.tensor(np.concatenate([t["v"], t["vb"]]), requires_grad=True)
    dO = torch.tensor(np.concatenate([t["do"], t["dob"]]))
    c = HEADMAP_CASES[name]
    idx = torch.tensor(c["kv_head_of"] if c["kv_head_of"] is not None
                       else [h // (p.hq // p.hkv) for h in range(p.hq)])
    scale = c["scale"] or 1.0 / math.sqrt(w.head_dim)
    Ke, Ve = K.index_select(1, idx), V.index_select(1, idx)
    S = torch.einsum("rhd,khd->hrk", Q, Ke) * scale
    S = S.masked_fill(~mask, float("-inf"))
    O = torch.einsum("hrk,khd->rhd", torch.softmax(S, dim=-1), Ve)
    (O * dO).sum().backward()
    nq, n = p.Nq, p.N
    for got, ref in ((g["dq"], Q.grad[:nq]), (g["dqb"], Q.grad[nq:]), (g["dk"], K.grad[:n]),
                     (g["dkb"], K.grad[n:]), (g["dv"], V.grad[:n]), (g["dvb"], V.grad[n:])):
        np.testing.assert_allclose(got, ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("name", list(HEADMAP_CASES))
def test_row_restricted_with_head_map_matches_dense(name):
    w = _headmap_case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w, grads=True))
    f = oracle.forward(p, t)
    g = oracle.backward(p, t, f)
    rows = list(range(p.Nq + p.Rb))
    O, L = oracle.forward_rows(p, t, rows)
    np.testing.assert_allclose(O, np.concatenate([f["o"], f["ob"]]), atol=1e-12)
    np.testing.assert_allclose(L, np.concatenate([f["lse"], f["lseb"]], axis=1), atol=1e-12)
    acc = {k: np.zeros_like(t[k[1:]]) for k in ("dk", "dv", "dkb", "dvb")}
    dQ = oracle.backward_rows(p, t, rows, acc)
    np.testing.assert_allclose(dQ, np.concatenate([g["dq"], g["dqb"]]), atol=1e-12)
    for k in acc:
        np.testing.assert_allclose(acc[k], g[k], atol=1e-12)


def _expand_kv(x, hq):
    """[K, Hkv, d] -> [Hq, K, d] with contiguous GQA groups."""
    rep = hq // x.shape[1]
    return torch.from_numpy(np.repeat(x, rep, axis=1).transpose(1, 0, 2).copy())


@pytest.mark.parametrize("name", list(TINY_CASES))
def test_forward_matches_torch_sdpa_with_mask(name):
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    f = oracle.forward(p, t)
    mask = torch.from_numpy(oracle.dense_mask(p))
    Q = torch.from_numpy(np.concatenate([t["q"], t["qb"]]).transpose(1, 0, 2).copy())
    K = _expand_kv(np.concatenate([t["k"], t["kb"]]), p.hq)
    V = _expand_kv(np.concatenate([t["v"], t["vb"]]), p.hq)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask).numpy()
    got = np.concatenate([f["o"], f["ob"]]).transpose(1, 0, 2)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_no_branches_reduces_to_per_sequence_causal_sdpa():
    w = _tiny("nb", hq=4, hkv=4, d=16, seqs=(7, 1, 12), anchors=(), lens=(), modes=())
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    f = oracle.forward(p, t)
    for s in range(len(w.cu_seqlens) - 1):
        lo, hi = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        Q = torch.from_numpy(t["q"][lo:hi].transpose(1, 0, 2).copy())
        K = torch.from_numpy(t["k"][lo:hi].transpose(1, 0, 2).copy())
        V = torch.from_numpy(t["v"][lo:hi].transpose(1, 0, 2).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True).numpy()
        np.testing.assert_allclose(f["o"][lo:hi].transpose(1, 0, 2), ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms

def _visible_count_closed_form(w, r):
    """n_r: t-cu[s]+1 (main), a-cu[s]+1+j (TTT query j), a-cu[s]+1+B (block of B)."""
    cu = w.cu_seqlens
    if r < w.Nq:
        t = int(w.q_pos[r]); s = int(np.searchsorted(cu, t, side="right") - 1)
        return t - int(cu[s]) + 1
    b = r - w.Nq
    m = int(np.searchsorted(w.cu_branch, b, side="right") - 1)
    a = int(w.anchors[m]); s = int(np.searchsorted(cu, a, side="right") - 1)
    L = int(w.cu_branch[m + 1] - w.cu_branch[m])
    j = b - int(w.cu_branch[m]) + 1
    return a - int(cu[s]) + 1 + (L if w.modes[m] == BLOCK else j)


@pytest.mark.parametrize("name", ["mixed", "single_tokens", "blocks"])
def test_zero_keys_closed_form(name):
    """K = 0: every score is 0, so LSE = ln n_r and O = mean of the visible V rows
    (computed here from prefix sums of V, not from a mask)."""
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    t["k"][:] = 0
    t["kb"][:] = 0
    f = oracle.forward(p, t)
    pre = np.concatenate([np.zeros((1,) + t["v"].shape[1:]), np.cumsum(t["v"], axis=0)])
    g = p.kv_head_of
    for r in range(p.Nq + p.Rb):
        n = _visible_count_closed_form(w, r)
        lse = f["lse"][:, r] if r < p.Nq else f["lseb"][:, r - p.Nq]
        np.testing.assert_allclose(lse, np.log(n), rtol=0, atol=1e-12)
        if r < p.Nq:
            t0 = int(w.q_pos[r]); s = int(np.searchsorted(w.cu_seqlens, t0, side="right") - 1)
            tot = pre[t0 + 1] - pre[int(w.cu_seqlens[s])]
            o = f["o"][r]
        else:
            b = r - p.Nq
            m = int(np.searchsorted(w.cu_branch, b, side="right") - 1)
            a = int(w.anchors[m]); s = int(np.searchsorted(w.cu_seqlens, a, side="right") - 1)
            first = int(w.cu_branch[m])
            last = int(w.cu_branch[m + 1]) if w.modes[m] == BLOCK else b + 1
            tot = pre[a + 1] - pre[int(w.cu_seqlens[s])] + t["vb"][first:last].sum(axis=0)
            o = f["ob"][b]
        np.testing.assert_allclose(o, tot[g] / n, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    w = _case("mixed")
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    t["v"][:] = 0.375
    t["vb"][:] = 0.375
    f = oracle.forward(p, t)
    np.testing.assert_allclose(f["o"], 0.375, rtol=0, atol=1e-13)
    np.testing.assert_allclose(f["ob"], 0.375, rtol=0, atol=1e-13)


def test_peaked_softmax_selects_the_matching_key():
    """q = 40 * k_u for one visible key u (and unit-norm keys): the softmax is a
    near one-hot at u, so O ~= V_u; a wrong scale, sign or mask boundary breaks it."""
    w = _tiny("pk", hq=2, hkv=1, d=16, seqs=(6, 6), anchors=(3, 8), lens=(2, 2), modes=(TTT, BLOCK))
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    for key in ("k", "kb"):
        t[key] /= np.linalg.norm(t[key], axis=-1, keepdims=True)
    # main row 5 (seq 0) aims at key 0 (its sequence start); branch row 1 of anchor 3 aims at branch key 1
    t["q"][5, :, :] = 40 * math.sqrt(16) * t["k"][0, 0]
    t["qb"][1, :, :] = 40 * math.sqrt(16) * t["kb"][1, 0]
    # block row 2 (anchor 8) aims at its own anchor's main key
    t["qb"][2, :, :] = 40 * math.sqrt(16) * t["k"][8, 0]
    f = oracle.forward(p, t)
    np.testing.assert_allclose(f["o"][5], np.broadcast_to(t["v"][0, 0], (2, 16)), atol=1e-6)
    np.testing.assert_allclose(f["ob"][1], np.broadcast_to(t["vb"][1, 0], (2, 16)), atol=1e-6)
    np.testing.assert_allclose(f["ob"][2], np.broadcast_to(t["v"][8, 0], (2, 16)), atol=1e-6)


# --------------------------------------------------------------------------
# the log-sum-exp merge

@pytest.mark.parametrize("name", list(TINY_CASES))
def test_split_then_merge_equals_union(name):
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    f = oracle.forward(p, t)
    merged, _ = oracle.split_forward(p, t)
    for k in ("o", "ob"):
        np.testing.assert_allclose(merged[k], f[k], rtol=0, atol=1e-12)
    for k in ("lse", "lseb"):
        np.testing.assert_allclose(merged[k], f[k], rtol=0, atol=1e-12)


def test_merge_identity_commutativity_and_empty():
    rng = np.random.default_rng(3)
    oa, ob = rng.standard_normal((5, 3, 4)), rng.standard_normal((5, 3, 4))
    la, lb = rng.standard_normal((3, 5)), rng.standard_normal((3, 5))
    empty_o, empty_l = np.zeros_like(oa), np.full_like(la, -np.inf)
    o, l = oracle.lse_merge(oa, la, empty_o, empty_l)
    np.testing.assert_array_equal(o, oa)
    np.testing.assert_array_equal(l, la)
    o1, l1 = oracle.lse_merge(oa, la, ob, lb)
    o2, l2 = oracle.lse_merge(ob, lb, oa, la)
    np.testing.assert_allclose(o1, o2, atol=1e-15)
    np.testing.assert_allclose(l1, l2, atol=1e-15)
    o3, l3 = oracle.lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(o3 == 0) and np.all(np.isneginf(l3))
    # closed form for equal LSEs: the plain average and L + ln 2
    o4, l4 = oracle.lse_merge(oa, la, ob, la)
    np.testing.assert_allclose(o4, 0.5 * (oa + ob), atol=1e-15)
    np.testing.assert_allclose(l4, la + math.log(2.0), atol=1e-15)


def test_three_way_split_matches_union():
    """Main keys split at an arbitrary position into two partials plus the branch
    partial: merging in either order reproduces the union softmax."""
    w = _tiny("ts", hq=2, hkv=1, d=8, seqs=(16,), anchors=(9, 13), lens=(3, 4), modes=(TTT, BLOCK))
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    f = oracle.forward(p, t)
    mask = oracle.dense_mask(p)[p.Nq:]
    Qb, cut = t["qb"], 6
    o1, l1 = oracle.attend(Qb, t["k"][:cut], t["v"][:cut], mask[:, :cut], p.kv_head_of, p.scale)
    o2, l2 = oracle.attend(Qb, t["k"][cut:], t["v"][cut:], mask[:, cut:p.N], p.kv_head_of, p.scale)
    o3, l3 = oracle.attend(Qb, t["kb"], t["vb"], mask[:, p.N:], p.kv_head_of, p.scale)
    oa, la = oracle.lse_merge(*oracle.lse_merge(o1, l1, o2, l2), o3, l3)
    ob, lb = oracle.lse_merge(o1, l1, *oracle.lse_merge(o3, l3, o2, l2))
    for o, l in ((oa, la), (ob, lb)):
        np.testing.assert_allclose(o, f["ob"], atol=1e-12)
        np.testing.assert_allclose(l, f["lseb"], atol=1e-12)


def _main_partials(p, t):
    _, part = oracle.split_forward(p, t)
    return (np.concatenate([part["o_main"], part["ob_main"]]),
            np.concatenate([part["lse_main"], part["lseb_main"]], axis=1))


@pytest.mark.parametrize("name", ["mixed", "blocks", "single_tokens"])
def test_ring_windows_merge_to_the_single_pass(name):
    """Key windows that tile [0, N), merged in any order (with empty windows and
    windows past N mixed in), give the main-key partial of every row."""
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    o_ref, l_ref = _main_partials(p, t)
    cuts = [0, 3, 4, 9, 10, p.N]
    wins = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if a < b]
    rng = np.random.default_rng(5)
    for order in (wins, wins[::-1], [wins[i] for i in rng.permutation(len(wins))]):
        o, l = oracle.ring_forward(p, t, list(order) + [(2, 2), (p.N, p.N + 7)])
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)


def test_ring_zigzag_steps_and_a_missing_window():
    """The zigzag layout of a CP=4 ring (8 chunks; rank r holds chunks r and 7-r)
    delivered to rank 1 in ring order reproduces the single pass; leaving one
    chunk out changes every row that sees it."""
    w = _tiny("zz", hq=2, hkv=1, d=8, seqs=(32,), q_pos=list(range(4, 8)) + list(range(24, 28)),
              anchors=(5, 24, 27), lens=(3, 2, 4), modes=(TTT, BLOCK, TTT))
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    o_ref, l_ref = _main_partials(p, t)
    steps = [(r, 7 - r) for r in (1, 0, 3, 2)]  # chunk pairs in the order the ring brings them
    wins = [(4 * c, 4 * c + 4) for pair in steps for c in pair]
    o, l = oracle.ring_forward(p, t, wins)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)
    o2, l2 = oracle.ring_forward(p, t, [x for x in wins if x != (8, 12)])
    sees = np.array([oracle.row_keys(p, r)[1] >= 8 for r in range(p.Nq + p.Rb)])
    assert sees.any()
    assert np.all(np.abs(l2 - l_ref)[:, sees] > 1e-6)
    np.testing.assert_allclose(l2[:, ~sees], l_ref[:, ~sees], atol=1e-12)


# --------------------------------------------------------------------------
# locality: branch rows depend only on their anchor's prefix and their own branch

def test_locality_of_branch_rows():
    w = _case("mixed")
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    base = oracle.forward(p, t)
    rng = np.random.default_rng(7)
    for m in range(p.A):
        a = int(p.anchors[m]); s = p.seq_of(a)
        rows = slice(int(p.cu_branch[m]), int(p.cu_branch[m + 1]))
        t2 = {k: v.copy() for k, v in t.items()}
        # main keys after the anchor and in other sequences
        far = np.ones(p.N, bool)
        far[int(p.cu[s]):a + 1] = False
        for key in ("k", "v"):
            t2[key][far] = rng.standard_normal(t2[key][far].shape) * 5
        # other anchors' branch keys
        other = np.ones(p.Rb, bool)
        other[rows] = False
        for key in ("kb", "vb"):
            t2[key][other] = rng.standard_normal(t2[key][other].shape) * 5
        pert = oracle.forward(p, t2)
        np.testing.assert_array_equal(pert["ob"][rows], base["ob"][rows])
        np.testing.assert_array_equal(pert["lseb"][:, rows], base["lseb"][:, rows])
    # the branch-key partial does not depend on main K/V at all
    _, part = oracle.split_forward(p, t)
    t3 = {k: v.copy() for k, v in t.items()}
    t3["k"] *= -3.0
    t3["v"] += 1.0
    _, part3 = oracle.split_forward(p, t3)
    np.testing.assert_array_equal(part3["ob_loc"], part["ob_loc"])
    np.testing.assert_array_equal(part3["lseb_loc"], part["lseb_loc"])


def test_main_rows_never_see_branch_keys():
    w = _case("mixed")
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w))
    base = oracle.forward(p, t)
    t["kb"] *= 7.0
    t["vb"] -= 2.0
    pert = oracle.forward(p, t)
    np.testing.assert_array_equal(pert["o"], base["o"])
    np.testing.assert_array_equal(pert["lse"], base["lse"])


# --------------------------------------------------------------------------
# backward

def _loss(p, t):
    f = oracle.forward(p, t)
    return float((f["o"] * t["do"]).sum() + (f["ob"] * t["dob"]).sum())


@pytest.mark.parametrize("q_pos", [None, [0, 2, 3, 5]], ids=["all_rows", "row_subset"])
def test_backward_matches_central_differences(q_pos):
    w = _tiny("fd", hq=2, hkv=1, d=4, seqs=(4, 3), q_pos=q_pos,
              anchors=(1, 3, 5), lens=(2, 2, 3), modes=(TTT, BLOCK, TTT))
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w, grads=True))
    f = oracle.forward(p, t)
    g = oracle.backward(p, t, f)
    eps = 1e-6
    for name_in, name_g in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("qb", "dqb"), ("kb", "dkb"), ("vb", "dvb")):
        x = t[name_in]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(p, t)
            x[idx] = old - eps
            lm = _loss(p, t)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[name_g], num, rtol=0, atol=1e-7, err_msg=name_g)


@pytest.mark.parametrize("name", ["mixed", "blocks", "single_tokens"])
def test_backward_matches_autograd(name):
    """torch autograd (fp64) of masked softmax attention with the dense mask."""
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w, grads=True))
    f = oracle.forward(p, t)
    g = oracle.backward(p, t, f)
    mask = torch.from_numpy(oracle.dense_mask(p))
    Q = torch.tensor(np.concatenate([t["q"], t["qb"]]), requires_grad=True)
    K = torch.tensor(np.concatenate([t["k"], t["kb"]]), requires_grad=True)
    V = torch.tensor(np.concatenate([t["v"], t["vb"]]), requires_grad=True)
    dO = torch.tensor(np.concatenate([t["do"], t["dob"]]))
    rep = p.hq // p.hkv
    Ke, Ve = K.repeat_interleave(rep, dim=1), V.repeat_interleave(rep, dim=1)
    S = torch.einsum("rhd,khd->hrk", Q, Ke) * p.scale
    S = S.masked_fill(~mask, float("-inf"))
    O = torch.einsum("hrk,khd->rhd", torch.softmax(S, dim=-1), Ve)
    (O * dO).sum().backward()
    nq, n = p.Nq, p.N
    np.testing.assert_allclose(g["dq"], Q.grad[:nq].numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dqb"], Q.grad[nq:].numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], K.grad[:n].numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dkb"], K.grad[n:].numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], V.grad[:n].numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dvb"], V.grad[n:].numpy(), atol=1e-12)


@pytest.mark.parametrize("name", list(TINY_CASES))
def test_gradient_sum_identities(name):
    """Per kv head: sum over all key rows of dK is 0 (every dS row sums to 0), and
    sum over all value rows of dV equals the sum of dO over the group's rows
    (every P row sums to 1)."""
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w, grads=True))
    g = oracle.backward(p, t, oracle.forward(p, t))
    sdk = g["dk"].sum(axis=0) + g["dkb"].sum(axis=0)
    np.testing.assert_allclose(sdk, 0.0, atol=1e-12)
    sdv = g["dv"].sum(axis=0) + g["dvb"].sum(axis=0)
    do_all = np.concatenate([t["do"], t["dob"]])
    for gi in range(p.hkv):
        heads = np.nonzero(p.kv_head_of == gi)[0]
        np.testing.assert_allclose(sdv[gi], do_all[:, heads].sum(axis=(0, 1)), atol=1e-12)


# --------------------------------------------------------------------------
# row-restricted evaluation (used at sizes the dense oracle cannot reach)

@pytest.mark.parametrize("name", ["mixed", "qsubset", "blocks"])
def test_row_restricted_matches_dense(name):
    w = _case(name)
    p = Problem.from_workload(w)
    t = _f64(make_inputs(w, grads=True))
    f = oracle.forward(p, t)
    g = oracle.backward(p, t, f)
    rows = list(range(p.Nq + p.Rb))
    O, L = oracle.forward_rows(p, t, rows)
    np.testing.assert_allclose(O, np.concatenate([f["o"], f["ob"]]), atol=1e-12)
    np.testing.assert_allclose(L, np.concatenate([f["lse"], f["lseb"]], axis=1), atol=1e-12)
    acc = {k: np.zeros_like(t[k[1:]]) for k in ("dk", "dv", "dkb", "dvb")}
    dQ = oracle.backward_rows(p, t, rows, acc)
    np.testing.assert_allclose(dQ, np.concatenate([g["dq"], g["dqb"]]), atol=1e-12)
    for k in acc:
        np.testing.assert_allclose(acc[k], g[k], atol=1e-12)


# --------------------------------------------------------------------------
# visible-pair counts of the named workloads, from closed-form sums

def _tri(a, b):
    """sum_{p=a}^{b-1} (p + 1 - a) for a sequence starting at a: b-a rows, 1..b-a keys."""
    n = b - a
    return n * (n + 1) // 2


def test_pair_counts_closed_forms():
    c = 16384
    # 256K share: one sequence from 0, queries at chunks 3 and 12; row at p sees p+1 keys
    main = sum(((b * (b + 1)) - (a * (a + 1))) // 2 for a, b in ((3 * c, 4 * c), (12 * c, 13 * c)))
    got = oracle.pair_counts(Problem.from_workload(W.get("ctx256k_rank3")))
    assert got == {"main": main, "branch_prefix": 7 * main, "branch_local": 2 * c * 28}
    assert main == 4_294_983_680
    # 16K packed, TTT 7 everywhere
    lens = [2048, 4096, 4096, 6144]
    main = sum(_tri(0, L) for L in lens)
    got = oracle.pair_counts(Problem.from_workload(W.get("qwen3_8b_16k")))
    assert got == {"main": main, "branch_prefix": 7 * main, "branch_local": 16384 * 28}
    # 64K blocks: anchors at 16m+15 see 16(m+1) main keys, 16 rows each
    n = 65536
    nb = n // 16
    got = oracle.pair_counts(Problem.from_workload(W.get("dflash_64k")))
    assert got == {"main": _tri(0, n), "branch_prefix": 16 * 16 * nb * (nb + 1) // 2, "branch_local": nb * 256}
    # the tiny fp32 case
    got = oracle.pair_counts(Problem.from_workload(W.get("tiny_f32")))
    assert got == {"main": _tri(0, 256), "branch_prefix": 3 * _tri(0, 256), "branch_local": 256 * 6}
