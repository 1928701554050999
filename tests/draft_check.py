"""Comparison of a draft tree built on the GPU with the oracle's.

The GPU evaluates each row's log-sum-exp in fp64 in a different order than the
oracle, so its log-probs differ from the oracle's by about 1e-15 relative.  Two
pending candidates whose keys are that close may be admitted in either order.
Outside such near-ties the two trees must be identical; where they differ, the
GPU's tree must be a valid best-first expansion under the oracle's own log-probs
with that tolerance, and the oracle's expansion must hold a near-tie.
"""
from __future__ import annotations

import numpy as np

TOL = 1e-9


def _replay(orc, rows, root, par, tok, K, max_levels, tol):
    """Replays one sequence's admissions with the oracle's top-K lists; returns the
    cumulative log-probs along it and the smallest gap between the admitted key and
    the best other pending key.  Raises AssertionError if an admission was invalid."""
    T = len(par)
    lists, nxt, level, cum = {}, {}, [1], [0.0]
    min_gap = np.inf

    def offer(i):
        if i < T - 1 and level[i] < max_levels:
            t, lp = orc.topk_logprobs(rows[i][None], K)
            lists[i] = (t[0], lp[0])
            nxt[i] = 0

    assert par[0] == -1 and tok[0] == root
    offer(0)
    for n in range(1, T):
        keys = {j: cum[j] + lists[j][1][nxt[j]] for j in lists if nxt[j] < K}
        assert keys, "no pending candidate"
        p = int(par[n])
        assert p in keys, f"node {n}: parent {p} has no pending child"
        assert int(tok[n]) == int(lists[p][0][nxt[p]]), f"node {n}: not its parent's next child"
        best = max(keys.values())
        assert keys[p] >= best - tol * max(1.0, abs(best)), f"node {n}: key below the best"
        others = [v for j, v in keys.items() if j != p]
        if others:
            min_gap = min(min_gap, abs(keys[p] - max(others)))
        cum.append(keys[p])
        level.append(level[p] + 1)
        nxt[p] += 1
        offer(n)
    return np.array(cum), min_gap


def compare_draft(orc, g, o, rows, roots, K, max_levels, tol=TOL) -> int:
    """g, o: (parents, tokens, cum) of the GPU and of the oracle; rows float32 [B, T, V].
    Returns the number of sequences that differ (each within the tolerance)."""
    gp, gt, gc = g
    op, ot, oc = o
    n_diff = 0
    for b in range(gp.shape[0]):
        if np.array_equal(gp[b], op[b]) and np.array_equal(gt[b], ot[b]):
            assert np.allclose(gc[b], oc[b], rtol=1e-13, atol=1e-12), (b, gc[b], oc[b])
            continue
        n_diff += 1
        cum, _ = _replay(orc, rows[b], int(roots[b]), gp[b], gt[b], K, max_levels, tol)
        assert np.allclose(gc[b], cum, rtol=1e-13, atol=1e-12)
        _, gap = _replay(orc, rows[b], int(roots[b]), op[b], ot[b], K, max_levels, 0.0)
        assert gap <= tol * max(1.0, float(np.abs(oc[b]).max())), \
            f"sequence {b}: trees differ without a near-tie (smallest gap {gap})"
    return n_diff
