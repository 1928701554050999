"""Checks of a sampled-acceptance result that do not depend on how it was computed.

The GPU decides in fp32 what the oracle decides in fp64.  ``replay`` follows a given
result (path and tokens) through the rule in fp64 and reports whether every decision
on it is valid up to ``tol`` (a probability), and whether any of them lies within
``tol`` of its boundary (then either outcome is a correct result of the rule).
"""
from __future__ import annotations

import numpy as np

F32_MAX = float(np.finfo(np.float32).max)


def target_probs(row: np.ndarray, tau: float) -> np.ndarray:
    """Target distribution of one logits row in fp64: NaN and -inf give 0, +inf counts as
    the largest finite float, a row without a finite entry is all 0."""
    l = row.astype(np.float64)
    l = np.where(np.isnan(l), -np.inf, l)
    l = np.where(np.isposinf(l), F32_MAX, l)
    fin = np.isfinite(l)
    if not fin.any():
        return np.zeros_like(l)
    m = l[fin].max()
    e = np.where(fin, np.exp((np.where(fin, l, m) - m) / tau), 0.0)
    return e / e.sum()


def replay(lg, drf, par, ua, us, tau, L, nodes, toks, tol):
    """One sequence.  Returns (valid, ambiguous, reason)."""
    T, V = lg.shape
    if L < 1 or L > T or nodes[0] != 0:
        return False, False, f"bad length or root ({L}, {nodes[0]})"
    if np.any(nodes[L:] != -1) or np.any(toks[L:] != -1):
        return False, False, "tail not -1"
    amb = False
    v, j = 0, 0
    while True:
        p = target_probs(lg[v], tau)
        kids = [c for c in range(T) if par[c] == v and c > 0]
        nxt = int(nodes[j + 1]) if j + 1 < L else None
        if nxt is not None and nxt not in kids:
            return False, amb, f"node {nxt} is not a child of {v}"
        E, R = set(), 1.0
        moved = False
        for c in kids:
            x = int(drf[c])
            ok = 0 <= x < V and x not in E
            px = p[x] if ok else 0.0
            margin = px - ua[c] * R
            if ok and abs(margin) <= tol:
                amb = True
            if c == nxt:
                if margin <= -tol:
                    return False, amb, f"child {c} accepted with u*R {ua[c] * R} >= p {px}"
                if toks[j] != x:
                    return False, amb, f"token {toks[j]} for accepted child {c} (draft {x})"
                v, j, moved = c, j + 1, True
                break
            if margin >= tol:
                return False, amb, f"child {c} rejected with u*R {ua[c] * R} < p {px}"
            if ok:
                E.add(x)
                R -= px
        if moved:
            continue
        if nxt is not None:
            return False, amb, "path continues past a node whose children were all rejected"
        y = int(toks[j])
        if y in E or not (0 <= y < V):
            return False, amb, f"drawn token {y} excluded or out of range"
        q = p.copy()
        for x in E:
            q[x] = 0.0
        c = np.cumsum(q)
        target = us[v] * R
        if c[-1] <= tol:                 # no probability left: token 0
            return (y == 0), amb or c[-1] > 0.0, "no mass left"
        before = c[y - 1] if y > 0 else 0.0
        if abs(c[y] - target) <= tol or abs(before - target) <= tol:
            amb = True
        if not (before <= target + tol and c[y] >= target - tol and q[y] > 0.0):
            return False, amb, f"drawn token {y}: cumulative [{before}, {c[y]}] vs {target}"
        return True, amb, ""


def compare_sampled(g, o, lg, drf, par, ua, us, tau, tol=5e-5):
    """g, o: (L, nodes, toks) of the GPU and the oracle.  Sequences must agree exactly,
    except where the oracle's own path holds a decision within tol of its boundary;
    there the GPU's result must be a valid outcome of the rule.  Returns the number
    of such sequences."""
    gL, gn, gt = g
    oL, on, ot = o
    n_amb = 0
    for b in range(len(oL)):
        same = (gL[b] == oL[b] and np.array_equal(gn[b], on[b]) and np.array_equal(gt[b], ot[b]))
        if oL[b] == 0:
            assert same, (b, gL[b], oL[b])
            continue
        if same:
            continue
        ok_o, amb_o, _ = replay(lg[b], drf[b], par[b], ua[b], us[b], tau, oL[b], on[b], ot[b], tol)
        ok_g, amb_g, why = replay(lg[b], drf[b], par[b], ua[b], us[b], tau, gL[b], gn[b], gt[b], tol)
        assert ok_o, f"sequence {b}: the oracle's own result fails the replay"
        assert ok_g, f"sequence {b}: GPU result invalid: {why}"
        assert amb_o or amb_g, (f"sequence {b}: GPU and oracle differ with no decision near "
                                f"its boundary: {gL[b]} {gn[b][:gL[b]]} {gt[b][:gL[b]]} vs "
                                f"{oL[b]} {on[b][:oL[b]]} {ot[b][:oL[b]]}")
        n_amb += 1
    return n_amb
