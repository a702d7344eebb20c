"""Torch-tensor wrappers of the C ABI entry points: checks and pointer marshalling only."""
from __future__ import annotations

from typing import Optional

import torch

from ._abi import BA_BF16, BA_F32, Plan, check, lib

_DT = {BA_BF16: torch.bfloat16, BA_F32: torch.float32}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _p(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else t.data_ptr()


def _chk(t: torch.Tensor, name: str, dtype: torch.dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace(plan: Plan, pass_: int, device=None) -> torch.Tensor:
    """A device byte buffer of the size the library asks for (allocation by torch)."""
    n = max(plan.workspace_bytes(pass_), 256)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def _shapes(plan: Plan):
    return {"q": (plan.Nq, plan.hq, plan.d), "k": (plan.N, plan.hkv, plan.d),
            "qb": (plan.Rb, plan.hq, plan.d), "kb": (plan.Rb, plan.hkv, plan.d),
            "lse": (plan.hq, plan.Nq), "lseb": (plan.hq, plan.Rb)}


def branch_attn_fwd(plan: Plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, ws: torch.Tensor):
    dt, s = _DT[plan.dtype], _shapes(plan)
    for t, n, key in ((q, "q", "q"), (k, "k", "k"), (v, "v", "k"), (qb, "qb", "qb"), (kb, "kb", "kb"),
                      (vb, "vb", "kb"), (o, "o", "q"), (ob, "ob", "qb")):
        _chk(t, n, dt, s[key])
    _chk(lse, "lse", torch.float32, s["lse"])
    _chk(lseb, "lseb", torch.float32, s["lseb"])
    check(lib.branch_attn_fwd(plan.handle, _p(q), _p(k), _p(v), _p(qb), _p(kb), _p(vb), _p(o), _p(lse), _p(ob),
                              _p(lseb), _p(ws), ws.numel(), _stream()), "branch_attn_fwd")


def branch_attn_fwd_noalloc(plan: Plan, q, k, v, qb, kb, vb, o, lse, ob, lseb):
    """branch_attn_fwd on the library's fixed per-GPU scratch: no workspace, no allocation."""
    dt, s = _DT[plan.dtype], _shapes(plan)
    for t, n, key in ((q, "q", "q"), (k, "k", "k"), (v, "v", "k"), (qb, "qb", "qb"), (kb, "kb", "kb"),
                      (vb, "vb", "kb"), (o, "o", "q"), (ob, "ob", "qb")):
        _chk(t, n, dt, s[key])
    _chk(lse, "lse", torch.float32, s["lse"])
    _chk(lseb, "lseb", torch.float32, s["lseb"])
    check(lib.branch_attn_fwd_noalloc(plan.handle, _p(q), _p(k), _p(v), _p(qb), _p(kb), _p(vb), _p(o), _p(lse),
                                      _p(ob), _p(lseb), _stream()), "branch_attn_fwd_noalloc")


def fwd_noalloc_max_bytes() -> int:
    return int(lib.ba_fwd_noalloc_max_bytes())


def branch_attn_bwd(plan: Plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob, dq, dk, dv, dqb, dkb, dvb,
                    ws: torch.Tensor):
    dt, s = _DT[plan.dtype], _shapes(plan)
    for t, n, key in ((q, "q", "q"), (k, "k", "k"), (v, "v", "k"), (qb, "qb", "qb"), (kb, "kb", "kb"),
                      (vb, "vb", "kb"), (o, "o", "q"), (ob, "ob", "qb"), (do, "do", "q"), (dob, "dob", "qb"),
                      (dq, "dq", "q"), (dk, "dk", "k"), (dv, "dv", "k"), (dqb, "dqb", "qb"), (dkb, "dkb", "kb"),
                      (dvb, "dvb", "kb")):
        _chk(t, n, dt, s[key])
    _chk(lse, "lse", torch.float32, s["lse"])
    _chk(lseb, "lseb", torch.float32, s["lseb"])
    check(lib.branch_attn_bwd(plan.handle, _p(q), _p(k), _p(v), _p(qb), _p(kb), _p(vb), _p(o), _p(lse), _p(ob),
                              _p(lseb), _p(do), _p(dob), _p(dq), _p(dk), _p(dv), _p(dqb), _p(dkb), _p(dvb),
                              _p(ws), ws.numel(), _stream()), "branch_attn_bwd")


def lse_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out):
    """o_*: float32 [rows, heads, d]; lse_*: float32 [heads, rows]; o_out float32 or bfloat16."""
    rows, heads, d = o_a.shape
    for t, n in ((o_a, "o_a"), (o_b, "o_b")):
        _chk(t, n, torch.float32, (rows, heads, d))
    for t, n in ((lse_a, "lse_a"), (lse_b, "lse_b"), (lse_out, "lse_out")):
        _chk(t, n, torch.float32, (heads, rows))
    if o_out.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("o_out must be float32 or bfloat16")
    _chk(o_out, "o_out", o_out.dtype, (rows, heads, d))
    out_dt = BA_F32 if o_out.dtype == torch.float32 else BA_BF16
    check(lib.lse_merge(rows, heads, d, _p(o_a), _p(lse_a), _p(o_b), _p(lse_b), _p(o_out), out_dt, _p(lse_out),
                        _stream()), "lse_merge")


def ba_main_fwd(plan: Plan, q, qb, k, v, o, lse, o_pre, lse_pre, ws: torch.Tensor):
    dt, s = _DT[plan.dtype], _shapes(plan)
    for t, n, key in ((q, "q", "q"), (qb, "qb", "qb"), (k, "k", "k"), (v, "v", "k"), (o, "o", "q")):
        _chk(t, n, dt, s[key])
    _chk(lse, "lse", torch.float32, s["lse"])
    _chk(o_pre, "o_pre", torch.float32, s["qb"])
    _chk(lse_pre, "lse_pre", torch.float32, s["lseb"])
    check(lib.ba_main_fwd(plan.handle, _p(q), _p(qb), _p(k), _p(v), _p(o), _p(lse), _p(o_pre), _p(lse_pre), _p(ws),
                          ws.numel(), _stream()), "ba_main_fwd")


def ba_branch_local_fwd(plan: Plan, qb, kb, vb, o_loc, lse_loc, ws: torch.Tensor):
    dt, s = _DT[plan.dtype], _shapes(plan)
    for t, n, key in ((qb, "qb", "qb"), (kb, "kb", "kb"), (vb, "vb", "kb")):
        _chk(t, n, dt, s[key])
    _chk(o_loc, "o_loc", torch.float32, s["qb"])
    _chk(lse_loc, "lse_loc", torch.float32, s["lseb"])
    check(lib.ba_branch_local_fwd(plan.handle, _p(qb), _p(kb), _p(vb), _p(o_loc), _p(lse_loc), _p(ws), ws.numel(),
                                  _stream()), "ba_branch_local_fwd")


def ba_ring_step_fwd(plan: Plan, q, qb, k_win, v_win, win_lo: int, win_hi: int, o_run, lse_run, ws: torch.Tensor):
    """One ring step: every row against the main keys of its prefix in [win_lo, win_hi),
    merged into the running float32 (o_run [Nq+Rb, Hq, d], lse_run [Hq, Nq+Rb]) in place."""
    dt, s = _DT[plan.dtype], _shapes(plan)
    _chk(q, "q", dt, s["q"])
    _chk(qb, "qb", dt, s["qb"])
    win = (int(win_hi) - int(win_lo),) + tuple(s["k"][1:])
    _chk(k_win, "k_win", dt, win)
    _chk(v_win, "v_win", dt, win)
    rows = s["q"][0] + s["qb"][0]
    _chk(o_run, "o_run", torch.float32, (rows,) + tuple(s["q"][1:]))
    _chk(lse_run, "lse_run", torch.float32, (s["q"][1], rows))
    check(lib.ba_ring_step_fwd(plan.handle, _p(q), _p(qb), _p(k_win), _p(v_win), int(win_lo), int(win_hi), _p(o_run),
                               _p(lse_run), _p(ws), ws.numel(), _stream()), "ba_ring_step_fwd")


def fwd(plan: Plan, q, k, v, qb, kb, vb, ws: Optional[torch.Tensor] = None):
    """Allocating convenience form: returns (o, lse, ob, lseb)."""
    dev = q.device
    o = torch.empty_like(q)
    ob = torch.empty_like(qb)
    lse = torch.empty((plan.hq, plan.Nq), dtype=torch.float32, device=dev)
    lseb = torch.empty((plan.hq, plan.Rb), dtype=torch.float32, device=dev)
    ws = workspace(plan, 0, dev) if ws is None else ws
    branch_attn_fwd(plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, ws)
    return o, lse, ob, lseb


def bwd(plan: Plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob, ws: Optional[torch.Tensor] = None):
    """Allocating convenience form: returns (dq, dk, dv, dqb, dkb, dvb)."""
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dqb, dkb, dvb = torch.empty_like(qb), torch.empty_like(kb), torch.empty_like(vb)
    ws = workspace(plan, 1, q.device) if ws is None else ws
    branch_attn_bwd(plan, q, k, v, qb, kb, vb, o, lse, ob, lseb, do, dob, dq, dk, dv, dqb, dkb, dvb, ws)
    return dq, dk, dv, dqb, dkb, dvb
