"""Shared helpers of the GPU parity tests: device transfer, tolerances, row sampling."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from workloads.inputs import to_f32

# Tolerances: float32 -- O and LSE max-abs 1e-5, gradients max-abs 1e-5 relative
# to the tensor's largest magnitude (gradients sum many fp32 terms); bf16 -- O
# max-abs 2e-2 and rel-L2 1e-2, LSE max-abs 1e-3, dQ/dK/dV rel-L2 2e-2 (over
# the whole tensor).
TOL = {
    "f32": {"o_abs": 1e-5, "lse_abs": 1e-5, "grad_abs": 1e-5},
    "bf16": {"o_abs": 2e-2, "o_rel": 1e-2, "lse_abs": 1e-3, "grad_rel": 2e-2},
}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    """Seeded host tensor -> GPU tensor (bf16 patterns become torch.bfloat16)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(a, b) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


class F32View:
    """Indexable float32 view over a seeded (possibly bf16-bit) array."""

    def __init__(self, a):
        self.a = a
        self.shape = a.shape

    def __getitem__(self, idx):
        return to_f32(self.a[idx])


def f32_views(t):
    return {k: F32View(v) for k, v in t.items()}


def f64_all(t):
    return {k: to_f32(v).astype(np.float64) for k, v in t.items()}


def check_out(name: str, got: np.ndarray, ref: np.ndarray, dtype: str, kind: str):
    """kind: 'o', 'lse' or 'grad'."""
    tol = TOL[dtype]
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = float(np.max(np.abs(got - ref)))
    rl = rel_l2(got, ref)
    say(f"  {name}: max_abs={err:.3e} rel_l2={rl:.3e}")
    if kind == "o":
        assert err <= tol["o_abs"], f"{name}: max-abs {err} > {tol['o_abs']}"
        if "o_rel" in tol:
            assert rl <= tol["o_rel"], f"{name}: rel-L2 {rl} > {tol['o_rel']}"
    elif kind == "lse":
        assert err <= tol["lse_abs"], f"{name}: max-abs {err} > {tol['lse_abs']}"
    else:
        if "grad_rel" in tol:
            assert rl <= tol["grad_rel"], f"{name}: rel-L2 {rl} > {tol['grad_rel']}"
        else:
            bound = tol["grad_abs"] * max(1.0, float(np.abs(ref).max()))
            assert err <= bound, f"{name}: max-abs {err} > {bound}"


def sample_rows(w, n_random: int = 16, seed: int = 0):
    """Combined row ids: first/last main rows of each sequence, branch rows of the
    first and last anchor of each sequence (depth 1 and the deepest), and uniform
    random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    Nq = w.Nq
    for s in range(w.num_seqs):
        lo, hi = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        q0, q1 = np.searchsorted(w.q_pos, [lo, hi])
        if q1 > q0:
            rows.update([int(q0), int(q1 - 1)])
        m0, m1 = np.searchsorted(w.anchors, [lo, hi])
        for m in {int(m0), int(m1 - 1)} if m1 > m0 else ():
            b0, b1 = int(w.cu_branch[m]), int(w.cu_branch[m + 1])
            if b1 > b0:
                rows.update([Nq + b0, Nq + b1 - 1])
    R = Nq + w.Rb
    rows.update(int(x) for x in rng.integers(0, R, size=n_random))
    return sorted(rows)


def gather_rows(o, ob, lse, lseb, rows, Nq):
    """Device outputs -> host arrays for the combined rows (O [n,H,d], LSE [H,n])."""
    rows = np.asarray(rows)
    mi, bi = rows[rows < Nq], rows[rows >= Nq] - Nq
    O = np.concatenate([host(o[torch.as_tensor(mi, device=o.device)]) if len(mi) else np.zeros((0,) + tuple(o.shape[1:])),
                        host(ob[torch.as_tensor(bi, device=ob.device)]) if len(bi) else np.zeros((0,) + tuple(ob.shape[1:]))])
    L = np.concatenate([host(lse[:, torch.as_tensor(mi, device=lse.device)]) if len(mi) else np.zeros((lse.shape[0], 0)),
                        host(lseb[:, torch.as_tensor(bi, device=lseb.device)]) if len(bi) else np.zeros((lseb.shape[0], 0))],
                       axis=1)
    return O, L


def oracle_rows(w, t, rows):
    p = oracle.Problem.from_workload(w)
    return oracle.forward_rows(p, f32_views(t), rows)
