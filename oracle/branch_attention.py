"""Plain CPU definition of speculative-draft branch attention (test infrastructure only).

Row and key axes
----------------
Query rows are the main-sequence rows ``0..Nq-1`` (row ``i`` sits at packed
position ``q_pos[i]``) followed by the branch rows ``Nq..Nq+Rb-1`` (branch row
``b`` belongs to the anchor ``m`` with ``cu_branch[m] <= b < cu_branch[m+1]``
and is that branch's query ``j = b - cu_branch[m] + 1``, 1-based).

Keys are the main keys ``0..N-1`` (packed positions) followed by the branch
keys ``N..N+Rb-1``; branch key ``b`` is the key/value of branch row ``b``.

Which keys a row sees (the mask)
--------------------------------
* main row at position t in sequence s: main keys u with cu[s] <= u <= t
  (packed causal attention: evolve.pub review, "Summary"; rcap.io explainer,
  results paragraph: the packed version does not pad variable-length batches);
* branch row j of anchor a in sequence s: main keys cu[s] <= u <= a (the
  causal main prefix) plus keys of its own branch only -- 1..j for a TTT
  branch, all of them for a block -- (rcap.io explainer, paragraph on branch
  attention under context parallelism: a branch query sees the causal prefix
  of the main sequence plus a small set of branch-local keys);
* main rows never see branch keys: a branch forks from its anchor and is never
  part of the main sequence, so no main query can reach it (cere-bro wiki,
  "Mechanism", paragraph on context parallelism).

Per head h (kv head g = kv_head_of[h]) over the row's visible keys:
  S = scale * q.k,  LSE = log(sum(exp(S))),  P = exp(S - LSE),  O = P V.
Backward (exact gradient of the above):
  D = rowsum(dO * O), dP = dO V^T, dS = P * (dP - D),
  dQ = scale dS K,  dK_g = scale sum_{h in g} dS^T Q,  dV_g = sum_{h in g} P^T dO.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

TTT = 0
BLOCK = 1


class Problem:
    """Structure of one packed batch (host arrays, any integer dtype)."""

    def __init__(self, num_q_heads, num_kv_heads, head_dim, cu_seqlens, q_pos, anchors,
                 cu_branch, modes, kv_head_of=None, scale=None):
        self.hq = int(num_q_heads)
        self.hkv = int(num_kv_heads)
        self.d = int(head_dim)
        self.cu = np.asarray(cu_seqlens, dtype=np.int64)
        self.q_pos = np.asarray(q_pos, dtype=np.int64)
        self.anchors = np.asarray(anchors, dtype=np.int64)
        self.cu_branch = np.asarray(cu_branch, dtype=np.int64)
        self.modes = np.asarray(modes, dtype=np.int64)
        if kv_head_of is None:
            kv_head_of = np.arange(self.hq) // (self.hq // self.hkv)
        self.kv_head_of = np.asarray(kv_head_of, dtype=np.int64)
        self.scale = 1.0 / math.sqrt(self.d) if not scale else float(scale)

    @classmethod
    def from_workload(cls, w, kv_head_of=None, scale=None) -> "Problem":
        if kv_head_of is None:
            kv_head_of = getattr(w, "kv_head_of", None)
        if scale is None:
            scale = getattr(w, "softmax_scale", None) or None
        return cls(w.num_q_heads, w.num_kv_heads, w.head_dim, w.cu_seqlens, w.q_pos, w.anchors,
                   w.cu_branch, w.modes, kv_head_of, scale)

    @property
    def N(self) -> int:
        return int(self.cu[-1])

    @property
    def Nq(self) -> int:
        return int(self.q_pos.shape[0])

    @property
    def A(self) -> int:
        return int(self.anchors.shape[0])

    @property
    def Rb(self) -> int:
        return int(self.cu_branch[-1])

    def seq_of(self, pos: int) -> int:
        return int(np.searchsorted(self.cu, pos, side="right") - 1)

    def anchor_of(self, b: int) -> int:
        """Anchor index owning branch row b."""
        return int(np.searchsorted(self.cu_branch, b, side="right") - 1)


def row_keys(p: Problem, r: int):
    """Keys visible to combined row r: (lo, hi, branch_keys).

    Main keys lo..hi inclusive (packed positions) and an int array of visible
    branch keys (branch row indices).
    """
    if r < p.Nq:
        t = int(p.q_pos[r])
        return int(p.cu[p.seq_of(t)]), t, np.zeros(0, dtype=np.int64)
    b = r - p.Nq
    m = p.anchor_of(b)
    a = int(p.anchors[m])
    first, last = int(p.cu_branch[m]), int(p.cu_branch[m + 1])
    j = b - first + 1
    if p.modes[m] == BLOCK:
        bk = np.arange(first, last, dtype=np.int64)
    else:
        bk = np.arange(first, first + j, dtype=np.int64)
    return int(p.cu[p.seq_of(a)]), a, bk


def dense_mask(p: Problem) -> np.ndarray:
    """Boolean mask [Nq+Rb, N+Rb] of the whole problem (small problems only)."""
    R, K = p.Nq + p.Rb, p.N + p.Rb
    mask = np.zeros((R, K), dtype=bool)
    for r in range(R):
        lo, hi, bk = row_keys(p, r)
        mask[r, lo:hi + 1] = True
        mask[r, p.N + bk] = True
    return mask


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: Optional[np.ndarray],
           kv_head_of: np.ndarray, scale: float, dtype=np.float64):
    """Masked softmax attention with one softmax per row over the masked-in keys.

    q [R, Hq, d]; k, v [K, Hkv, d]; mask [R, K] (None = all visible).
    Returns O [R, Hq, d] and LSE [Hq, R].  A row with no visible key gets O = 0
    and LSE = -inf.
    """
    R, hq, d = q.shape
    O = np.zeros((R, hq, d), dtype=dtype)
    LSE = np.full((hq, R), -np.inf, dtype=dtype)
    if R == 0:
        return O, LSE
    for h in range(hq):
        g = int(kv_head_of[h])
        qh = np.asarray(q[:, h, :], dtype=dtype)
        kg = np.asarray(k[:, g, :], dtype=dtype)
        vg = np.asarray(v[:, g, :], dtype=dtype)
        S = scale * (qh @ kg.T)
        if mask is not None:
            S = np.where(mask, S, -np.inf)
        m = S.max(axis=1) if S.shape[1] else np.full(R, -np.inf, dtype=dtype)
        alive = np.isfinite(m)
        m0 = np.where(alive, m, 0.0)
        with np.errstate(divide="ignore"):
            lse = m0 + np.log(np.exp(S - m0[:, None]).sum(axis=1))
        lse = np.where(alive, lse, -np.inf)
        P = np.exp(S - np.where(alive, lse, 0.0)[:, None])
        P[~alive] = 0.0
        O[:, h, :] = P @ vg
        LSE[h] = lse
    return O, LSE


def attend_bwd(q, k, v, o, lse, do, mask, kv_head_of, scale, dtype=np.float64):
    """Gradient of ``attend`` given its outputs (o, lse) and dO.

    Returns dQ [R, Hq, d], dK, dV [K, Hkv, d].
    """
    R, hq, d = q.shape
    dq = np.zeros((R, hq, d), dtype=dtype)
    dk = np.zeros(k.shape, dtype=dtype)
    dv = np.zeros(v.shape, dtype=dtype)
    for h in range(hq):
        g = int(kv_head_of[h])
        qh = np.asarray(q[:, h, :], dtype=dtype)
        kg = np.asarray(k[:, g, :], dtype=dtype)
        vg = np.asarray(v[:, g, :], dtype=dtype)
        doh = np.asarray(do[:, h, :], dtype=dtype)
        oh = np.asarray(o[:, h, :], dtype=dtype)
        lh = np.asarray(lse[h], dtype=dtype)
        S = scale * (qh @ kg.T)
        alive = np.isfinite(lh)
        P = np.exp(S - np.where(alive, lh, 0.0)[:, None])
        if mask is not None:
            P = np.where(mask, P, 0.0)
        P[~alive] = 0.0
        D = (doh * oh).sum(axis=1)
        dP = doh @ vg.T
        dS = P * (dP - D[:, None])
        dq[:, h, :] = scale * (dS @ kg)
        dk[:, g, :] += scale * (dS.T @ qh)
        dv[:, g, :] += P.T @ doh
    return dq, dk, dv


def _as(x, dtype):
    return np.asarray(x, dtype=dtype)


def _sequence_blocks(p: Problem):
    """Per sequence: (q row slice, anchor slice, branch row slice, main key slice).

    Cross-sequence mask entries are all False, so attending block by block is
    exact and avoids materialising the whole mask.
    """
    for s in range(len(p.cu) - 1):
        lo, hi = int(p.cu[s]), int(p.cu[s + 1])
        q0, q1 = np.searchsorted(p.q_pos, [lo, hi])
        m0, m1 = np.searchsorted(p.anchors, [lo, hi])
        b0, b1 = int(p.cu_branch[m0]), int(p.cu_branch[m1])
        yield slice(int(q0), int(q1)), slice(int(m0), int(m1)), slice(b0, b1), slice(lo, hi)


def _block_mask(p: Problem, qs: slice, bs: slice, ks: slice) -> np.ndarray:
    rows = list(range(qs.start, qs.stop)) + [p.Nq + b for b in range(bs.start, bs.stop)]
    nmain = ks.stop - ks.start
    mask = np.zeros((len(rows), nmain + bs.stop - bs.start), dtype=bool)
    for i, r in enumerate(rows):
        lo, hi, bk = row_keys(p, r)
        if hi >= lo:
            mask[i, lo - ks.start:hi - ks.start + 1] = True
        mask[i, nmain + (bk - bs.start)] = True
    return mask


def forward(p: Problem, t: Dict[str, np.ndarray], dtype=np.float64) -> Dict[str, np.ndarray]:
    """Union-softmax forward for every row. t holds q, k, v, qb, kb, vb.

    Returns o [Nq,Hq,d], lse [Hq,Nq], ob [Rb,Hq,d], lseb [Hq,Rb].
    """
    hq, d = p.hq, p.d
    out = {"o": np.zeros((p.Nq, hq, d), dtype), "lse": np.full((hq, p.Nq), -np.inf, dtype),
           "ob": np.zeros((p.Rb, hq, d), dtype), "lseb": np.full((hq, p.Rb), -np.inf, dtype)}
    for qs, _, bs, ks in _sequence_blocks(p):
        nq = qs.stop - qs.start
        if nq + bs.stop - bs.start == 0:
            continue
        Q = np.concatenate([_as(t["q"][qs], dtype), _as(t["qb"][bs], dtype)])
        K = np.concatenate([_as(t["k"][ks], dtype), _as(t["kb"][bs], dtype)])
        V = np.concatenate([_as(t["v"][ks], dtype), _as(t["vb"][bs], dtype)])
        O, L = attend(Q, K, V, _block_mask(p, qs, bs, ks), p.kv_head_of, p.scale, dtype)
        out["o"][qs], out["lse"][:, qs] = O[:nq], L[:, :nq]
        out["ob"][bs], out["lseb"][:, bs] = O[nq:], L[:, nq:]
    return out


def backward(p: Problem, t: Dict[str, np.ndarray], fwd: Dict[str, np.ndarray],
             dtype=np.float64) -> Dict[str, np.ndarray]:
    """Exact gradients of the union softmax. t holds the inputs plus do, dob;
    fwd is the output of ``forward``. Returns dq, dk, dv, dqb, dkb, dvb."""
    g = {"dq": np.zeros(t["q"].shape, dtype), "dk": np.zeros(t["k"].shape, dtype),
         "dv": np.zeros(t["v"].shape, dtype), "dqb": np.zeros(t["qb"].shape, dtype),
         "dkb": np.zeros(t["kb"].shape, dtype), "dvb": np.zeros(t["vb"].shape, dtype)}
    for qs, _, bs, ks in _sequence_blocks(p):
        nq = qs.stop - qs.start
        if nq + bs.stop - bs.start == 0:
            continue
        Q = np.concatenate([_as(t["q"][qs], dtype), _as(t["qb"][bs], dtype)])
        K = np.concatenate([_as(t["k"][ks], dtype), _as(t["kb"][bs], dtype)])
        V = np.concatenate([_as(t["v"][ks], dtype), _as(t["vb"][bs], dtype)])
        O = np.concatenate([fwd["o"][qs], fwd["ob"][bs]])
        L = np.concatenate([fwd["lse"][:, qs], fwd["lseb"][:, bs]], axis=1)
        dO = np.concatenate([_as(t["do"][qs], dtype), _as(t["dob"][bs], dtype)])
        dQ, dK, dV = attend_bwd(Q, K, V, O, L, dO, _block_mask(p, qs, bs, ks),
                                p.kv_head_of, p.scale, dtype)
        nk = ks.stop - ks.start
        g["dq"][qs], g["dqb"][bs] = dQ[:nq], dQ[nq:]
        g["dk"][ks], g["dkb"][bs] = dK[:nk], dK[nk:]
        g["dv"][ks], g["dvb"][bs] = dV[:nk], dV[nk:]
    return g


class _HeadMajor:
    """Per-kv-head contiguous copies of the key/value tensors, so a row's
    visible main keys are one contiguous slice."""

    def __init__(self, p: Problem, t: Dict[str, np.ndarray], dtype):
        self.k = [np.ascontiguousarray(t["k"][:, g, :], dtype=dtype) for g in range(p.hkv)]
        self.v = [np.ascontiguousarray(t["v"][:, g, :], dtype=dtype) for g in range(p.hkv)]
        self.kb, self.vb = t["kb"], t["vb"]


def _row_fwd(p: Problem, hm: _HeadMajor, q_row: np.ndarray, r: int, dtype):
    """One row, all heads: scores against its visible keys.

    Returns O [Hq,d], LSE [Hq], P [Hq, n_keys] and the key set (lo, hi, bk).
    The q heads of one kv group are scored together against that group's keys.
    """
    lo, hi, bk = row_keys(p, r)
    n = hi - lo + 1 + len(bk)
    O = np.zeros((p.hq, p.d), dtype)
    L = np.zeros(p.hq, dtype)
    P = np.zeros((p.hq, n), dtype)
    for g in range(p.hkv):
        heads = np.nonzero(p.kv_head_of == g)[0]
        if len(heads) == 0:
            continue
        qg = np.asarray(q_row[heads], dtype=dtype)                       # [G, d]
        kk = np.concatenate([hm.k[g][lo:hi + 1], _as(hm.kb[bk, g, :], dtype)])
        vv = np.concatenate([hm.v[g][lo:hi + 1], _as(hm.vb[bk, g, :], dtype)])
        S = p.scale * (qg @ kk.T)                                        # [G, n]
        m = S.max(axis=1)
        lse = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
        Pg = np.exp(S - lse[:, None])
        O[heads] = Pg @ vv
        L[heads] = lse
        P[heads] = Pg
    return O, L, P, (lo, hi, bk)


def forward_rows(p: Problem, t: Dict[str, np.ndarray], rows: Iterable[int], dtype=np.float64,
                 _hm: Optional[_HeadMajor] = None):
    """Union-softmax forward for selected combined rows only (any problem size).

    Returns O [n, Hq, d] and LSE [Hq, n] in the order of ``rows``.
    """
    rows = list(rows)
    hm = _hm or _HeadMajor(p, t, dtype)
    O = np.zeros((len(rows), p.hq, p.d), dtype)
    L = np.zeros((p.hq, len(rows)), dtype)
    for i, r in enumerate(rows):
        q_row = t["q"][r] if r < p.Nq else t["qb"][r - p.Nq]
        O[i], L[:, i], _, _ = _row_fwd(p, hm, q_row, r, dtype)
    return O, L


def backward_rows(p: Problem, t: Dict[str, np.ndarray], rows: Iterable[int], acc=None,
                  dtype=np.float64, _hm: Optional[_HeadMajor] = None):
    """Backward restricted to selected rows: their exact dQ, plus (if ``acc`` is
    a dict with dk, dv, dkb, dvb arrays) their contributions added into dK/dV.

    The full dK/dV is the sum of these contributions over all rows.
    Returns dQ [n, Hq, d] in the order of ``rows``.
    """
    rows = list(rows)
    hm = _hm or _HeadMajor(p, t, dtype)
    dQ = np.zeros((len(rows), p.hq, p.d), dtype)
    for i, r in enumerate(rows):
        main = r < p.Nq
        q_row = t["q"][r] if main else t["qb"][r - p.Nq]
        do_row = t["do"][r] if main else t["dob"][r - p.Nq]
        O, L, P, (lo, hi, bk) = _row_fwd(p, hm, q_row, r, dtype)
        nmain = hi - lo + 1
        for g in range(p.hkv):
            heads = np.nonzero(p.kv_head_of == g)[0]
            if len(heads) == 0:
                continue
            qg = np.asarray(q_row[heads], dtype=dtype)                   # [G, d]
            dog = np.asarray(do_row[heads], dtype=dtype)                 # [G, d]
            kk = np.concatenate([hm.k[g][lo:hi + 1], _as(hm.kb[bk, g, :], dtype)])
            vv = np.concatenate([hm.v[g][lo:hi + 1], _as(hm.vb[bk, g, :], dtype)])
            Pg = P[heads]                                                # [G, n]
            D = (dog * O[heads]).sum(axis=1)                             # [G]
            dS = Pg * (dog @ vv.T - D[:, None])                          # [G, n]
            dQ[i, heads] = p.scale * (dS @ kk)
            if acc is not None:
                dk_c = p.scale * (dS.T @ qg)                             # [n, d]
                dv_c = Pg.T @ dog                                        # [n, d]
                acc["dk"][lo:hi + 1, g] += dk_c[:nmain]
                acc["dv"][lo:hi + 1, g] += dv_c[:nmain]
                acc["dkb"][bk, g] += dk_c[nmain:]
                acc["dvb"][bk, g] += dv_c[nmain:]
    return dQ


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial softmax results over disjoint key sets (the online-softmax
    reduction, Eq. 2 of the paper as named in the evolve.pub review, "Scope & Claims";
    the same log-sum-exp step ring attention uses between ring steps, per the
    rcap.io explainer).

    o_* [R, H, d], lse_* [H, R].  L = M + log(e^{La-M} + e^{Lb-M}), M = max(La, Lb);
    O = e^{La-L} Oa + e^{Lb-L} Ob.  An empty partial (O=0, LSE=-inf) is the
    identity; two empty partials give (0, -inf).
    """
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    M = np.maximum(la, lb)
    M0 = np.where(np.isfinite(M), M, 0.0)
    wa, wb = np.exp(la - M0), np.exp(lb - M0)
    s = wa + wb
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.where(s > 0, M0 + np.log(np.where(s > 0, s, 1.0)), -np.inf)
        fa = np.where(s > 0, wa / np.where(s > 0, s, 1.0), 0.0)
        fb = np.where(s > 0, wb / np.where(s > 0, s, 1.0), 0.0)
    O = fa.T[:, :, None] * np.asarray(o_a, np.float64) + fb.T[:, :, None] * np.asarray(o_b, np.float64)
    return O, L


def split_forward(p: Problem, t: Dict[str, np.ndarray], dtype=np.float64):
    """The method's decomposition: a main-key partial for every row, a branch-key
    partial for branch rows, merged with ``lse_merge``.

    Returns (merged dict like ``forward``, partials dict with o_main, lse_main,
    ob_main, lseb_main, ob_loc, lseb_loc)."""
    hq, d = p.hq, p.d
    part = {"ob_main": np.zeros((p.Rb, hq, d), dtype), "lseb_main": np.full((hq, p.Rb), -np.inf, dtype),
            "ob_loc": np.zeros((p.Rb, hq, d), dtype), "lseb_loc": np.full((hq, p.Rb), -np.inf, dtype),
            "o_main": np.zeros((p.Nq, hq, d), dtype), "lse_main": np.full((hq, p.Nq), -np.inf, dtype)}
    for qs, _, bs, ks in _sequence_blocks(p):
        nq, nb = qs.stop - qs.start, bs.stop - bs.start
        if nq + nb == 0:
            continue
        mask = _block_mask(p, qs, bs, ks)
        nk = ks.stop - ks.start
        Q = np.concatenate([_as(t["q"][qs], dtype), _as(t["qb"][bs], dtype)])
        # main-key part, every row
        Om, Lm = attend(Q, _as(t["k"][ks], dtype), _as(t["v"][ks], dtype), mask[:, :nk],
                        p.kv_head_of, p.scale, dtype)
        # branch-key part, branch rows only
        Ob, Lb = attend(Q[nq:], _as(t["kb"][bs], dtype), _as(t["vb"][bs], dtype), mask[nq:, nk:],
                        p.kv_head_of, p.scale, dtype)
        part["o_main"][qs], part["lse_main"][:, qs] = Om[:nq], Lm[:, :nq]
        part["ob_main"][bs], part["lseb_main"][:, bs] = Om[nq:], Lm[:, nq:]
        part["ob_loc"][bs], part["lseb_loc"][:, bs] = Ob, Lb
    ob, lseb = lse_merge(part["ob_main"], part["lseb_main"], part["ob_loc"], part["lseb_loc"])
    merged = {"o": part["o_main"], "lse": part["lse_main"], "ob": ob, "lseb": lseb}
    return merged, part


def ring_forward(p: Problem, t: Dict[str, np.ndarray], windows, dtype=np.float64):
    """Main-key part of every row computed the way a context-parallel ring
    computes it: the main keys arrive in windows [lo, hi) of packed positions;
    for each window every row (main and branch) attends the keys of its causal
    main prefix that fall inside it, and that partial joins a running (O, LSE)
    through ``lse_merge``, in the order given (rcap.io explainer: ring attention
    passes K/V chunks between ranks and combines the partial results by the
    log-sum-exp step; evolve.pub review, section 3.2 and Eq. 2).

    Windows may be empty, overlap [0, N) only in part, or lie past N; when they
    tile [0, N) without overlap the result is the main-key partial of every row.
    Returns o_run [Nq+Rb, Hq, d] and lse_run [Hq, Nq+Rb] (rows: main, then branch).
    """
    R, N = p.Nq + p.Rb, p.N
    Q = np.concatenate([_as(t["q"], dtype), _as(t["qb"], dtype)])
    main_mask = np.zeros((R, N), dtype=bool)
    for r in range(R):
        lo, hi, _ = row_keys(p, r)
        main_mask[r, lo:hi + 1] = True
    o_run = np.zeros((R, p.hq, p.d), dtype)
    lse_run = np.full((p.hq, R), -np.inf, dtype)
    for lo, hi in windows:
        lo, hi = max(int(lo), 0), min(int(hi), N)
        if hi <= lo:
            continue
        o_w, l_w = attend(Q, _as(t["k"][lo:hi], dtype), _as(t["v"][lo:hi], dtype), main_mask[:, lo:hi],
                          p.kv_head_of, p.scale, dtype)
        o_run, lse_run = lse_merge(o_run, lse_run, o_w, l_w)
    return o_run, lse_run


def pair_counts(p: Problem) -> Dict[str, int]:
    """Visible (row, key) pairs per head: main rows x main keys, branch rows x
    main keys, branch rows x branch keys."""
    main = 0
    for t in p.q_pos:
        main += int(t) - int(p.cu[p.seq_of(int(t))]) + 1
    pre = loc = 0
    for m in range(p.A):
        a = int(p.anchors[m])
        L = int(p.cu_branch[m + 1] - p.cu_branch[m])
        pre += L * (a - int(p.cu[p.seq_of(a)]) + 1)
        loc += L * L if p.modes[m] == BLOCK else L * (L + 1) // 2
    return {"main": main, "branch_prefix": pre, "branch_local": loc}
