"""fp64 brute force, written independently of ``oracle/`` (pure Python loops).

Visible keys are found by walking: a row's main keys are collected by stepping
back from its prefix end one position at a time until the position leaves the
row's sequence (found by a linear scan of the sequence offsets), and its branch
keys are enumerated from the branch's mode.  Scores, the softmax and the output
use ``math.fsum``/``math.exp``/``math.log`` on Python floats.  For tiny inputs only.
"""
import math


def _seq_index(cu, pos):
    for s in range(len(cu) - 1):
        if cu[s] <= pos < cu[s + 1]:
            return s
    raise ValueError(pos)


def _walk_back(cu, end):
    s = _seq_index(cu, end)
    keys = []
    u = end
    while u >= 0 and _seq_index(cu, u) == s:
        keys.append(("main", u))
        u -= 1
        if u < cu[s]:
            break
    return keys


def visible_keys(cu, q_pos, anchors, cu_branch, modes, row):
    """List of ("main", position) / ("branch", branch_row) visible to combined row ``row``."""
    cu, q_pos, anchors = [int(x) for x in cu], [int(x) for x in q_pos], [int(x) for x in anchors]
    cub, modes = [int(x) for x in cu_branch], [int(x) for x in modes]
    nq = len(q_pos)
    if row < nq:
        return _walk_back(cu, q_pos[row])
    b = row - nq
    for m in range(len(anchors)):
        if cub[m] <= b < cub[m + 1]:
            j = b - cub[m] + 1                     # 1-based branch query index
            keys = _walk_back(cu, anchors[m])
            count = (cub[m + 1] - cub[m]) if modes[m] == 1 else j
            for jp in range(1, count + 1):
                keys.append(("branch", cub[m] + jp - 1))
            return keys
    raise ValueError(row)


def brute_forward(cu, q_pos, anchors, cu_branch, modes, q, k, v, qb, kb, vb, kv_group, scale):
    """Returns per combined row, per head: (O list, LSE float). Tensors are nested
    lists or arrays indexable as x[row][head][dim]. ``kv_group``: the group size G
    (q head h reads kv head h // G) or an explicit list, entry h = kv head of q head h."""
    nq = len(q_pos)
    rows = nq + int(cu_branch[-1])
    hq = len(q[0]) if nq else len(qb[0])
    d = len(k[0][0])
    out = []
    for r in range(rows):
        keys = visible_keys(cu, q_pos, anchors, cu_branch, modes, r)
        qrow = q[r] if r < nq else qb[r - nq]
        per_head = []
        for h in range(hq):
            g = h // kv_group if isinstance(kv_group, int) else int(kv_group[h])
            scores, vals = [], []
            for kind, idx in keys:
                kk = k[idx][g] if kind == "main" else kb[idx][g]
                vv = v[idx][g] if kind == "main" else vb[idx][g]
                scores.append(scale * math.fsum(float(qrow[h][e]) * float(kk[e]) for e in range(d)))
                vals.append([float(vv[e]) for e in range(d)])
            mx = max(scores)
            z = math.fsum(math.exp(s - mx) for s in scores)
            lse = mx + math.log(z)
            o = [math.fsum(math.exp(s - lse) * vals[i][e] for i, s in enumerate(scores)) for e in range(d)]
            per_head.append((o, lse))
        out.append(per_head)
    return out
