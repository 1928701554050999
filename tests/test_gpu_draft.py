"""GPU parity of the draft-tree builder: sv_topk_logprobs and sv_draft_tree through the C
ABI against the oracle on the same seeded inputs.

Top-K tokens must be identical and log-probs within 1e-12.  Trees must be identical
(parents, tokens) with cumulative log-probs within 1e-12, except where two pending keys
lie within 1e-9 of each other (see draft_check.py).
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import tree_masked_verify_amd as sv
from _support import to_np
from draft_check import compare_draft
from tree_masked_verify_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def orc():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return O.Oracle()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_topk(logits: torch.Tensor, K: int):
    shape = logits.shape[:-1]
    tok = torch.full((*shape, K), -7, dtype=torch.int32, device=DEV)
    lp = torch.full((*shape, K), 7.0, dtype=torch.float64, device=DEV)
    sv.sv_topk_logprobs(logits, K, tok, lp)
    torch.cuda.synchronize()
    return to_np(tok), to_np(lp)


def check_topk(orc, x: np.ndarray, K: int, label=""):
    _say(f"[case] topk {label} rows={x.shape[0]} V={x.shape[-1]} K={K}")
    gt, gl = gpu_topk(_dev(x), K)
    ot, ol = orc.topk_logprobs(x, K)
    assert np.array_equal(gt, ot), (label, np.argwhere(gt != ot)[:5])
    inf = np.isinf(ol)
    assert np.array_equal(np.isinf(gl), inf) and np.all(gl[inf] == ol[inf])
    assert np.allclose(gl[~inf], ol[~inf], rtol=1e-14, atol=1e-12), \
        float(np.abs(gl[~inf] - ol[~inf]).max())


def gpu_draft(dl: torch.Tensor, roots: torch.Tensor, K: int, max_levels: int):
    B, T, _ = dl.shape
    par = torch.full((B, T), -7, dtype=torch.int32, device=DEV)
    tok = torch.full((B, T), -7, dtype=torch.int32, device=DEV)
    cum = torch.full((B, T), 7.0, dtype=torch.float64, device=DEV)
    ws = sv.workspace(sv.sv_draft_tree_workspace_size(B, T, K), DEV)
    sv.sv_draft_tree(dl, roots, K, max_levels, par, tok, cum, ws)
    torch.cuda.synchronize()
    return to_np(par), to_np(tok), to_np(cum)


def check_draft(orc, rows: np.ndarray, roots: np.ndarray, K: int, max_levels: int, label=""):
    B, T, V = rows.shape
    _say(f"[case] draft {label} B={B} T={T} V={V} K={K} max_levels={max_levels}")
    g = gpu_draft(_dev(rows), _dev(roots.astype(np.int32)), K, max_levels)
    o = orc.draft_tree(rows, roots, K, max_levels)
    n = compare_draft(orc, g, o, rows, roots, K, max_levels)
    depth = np.zeros((B, T), np.int64)
    for i in range(1, T):
        depth[:, i] = depth[np.arange(B), g[0][:, i]] + 1
    _say(f"       depth max {depth.max()}, {n} sequence(s) decided within tolerance of a tie")
    return g


# ------------------------------------------------------------------------------ top-K
@pytest.mark.parametrize("R,V,K", [(7, 1000, 8), (3, 5, 5), (5, 70001, 16), (4, 131073, 64),
                                   (2, 1, 1), (3, 257, 33), (9, 151936, 8), (1, 3, 2)])
def test_topk_random(orc, R, V, K):
    rng = np.random.default_rng(R * 1000 + K)
    # a coarse grid makes ties common
    x = (np.round(rng.normal(0, 2, size=(R, V)) * 8) / 8).astype(np.float32)
    check_topk(orc, x, K, label="random")


@pytest.mark.parametrize("loc,std", [(0.0, 50.0), (1000.0, 3.0), (-500.0, 3.0), (60.0, 4.0),
                                     (-62.0, 3.0), (30.0, 2.0), (-31.0, 1.0), (0.0, 1e-3)])
def test_topk_wide_range(orc, loc, std):
    """Logits beyond the small-range path (|x| >= 31.5) alone and mixed with small ones:
    far above and far below zero, straddling +-31.5 and +-64, the values at the edge of the
    range's tables, and tightly packed."""
    rng = np.random.default_rng(int(abs(loc)) + 7)
    x = (loc + std * rng.normal(size=(6, 20011))).astype(np.float32)
    x[1, ::97] = np.float32(loc + 200.0)           # a few far larger entries
    x[2, :] = np.where(rng.random(20011) < 0.5, x[2, :], np.float32(-70.0))
    edge = np.float32(31.5)
    below = np.nextafter(edge, np.float32(0))
    x[3, ::53] = edge                              # just outside the small range
    x[3, 1::53] = -edge
    x[3, 2::53] = below                            # the largest logits inside it
    x[3, 3::53] = -below
    check_topk(orc, x, 16, label=f"loc {loc} std {std}")


def test_topk_special_rows(orc):
    V = 3000
    rng = np.random.default_rng(5)
    rows = [rng.normal(0, 2, V).astype(np.float32) for _ in range(12)]
    rows[0][::7] = np.nan
    rows[1][[5, 900, 2999]] = np.inf
    rows[2][:] = -np.inf
    rows[3][:] = np.nan
    rows[4][:] = 1.5                                   # every token tied
    rows[5][:] = 0.0
    rows[5][1::2] = -0.0                               # the two zeros are equal
    rows[6] = np.sort(rows[6])                         # ascending: the best at the end
    rows[7] = np.sort(rows[7])[::-1].copy()            # descending
    rows[8][:3] = [0.0, -3e38, -2e38]
    rows[8][3:] = -np.inf
    rows[9][:] = -np.inf
    rows[9][[2990, 10, 2999]] = [1.0, 1.0, 2.0]        # fewer finite entries than K
    rows[10][:] = np.float32(-3.4028235e38)            # every entry -FLT_MAX
    rows[11][100:] = -np.inf
    x = np.stack(rows)
    for K in (1, 8, 64):
        check_topk(orc, x, K, label="special")


def test_topk_unaligned_rows(orc):
    """A row pointer that is not 16-byte aligned (an offset view)."""
    rng = np.random.default_rng(9)
    base = rng.normal(0, 2, size=4 * 5003 + 3).astype(np.float32)
    d = _dev(base)
    for off in (1, 2, 3):
        view = d[off: off + 4 * 5003].view(4, 5003)
        gt, gl = gpu_topk(view, 12)
        ot, ol = orc.topk_logprobs(base[off: off + 4 * 5003].reshape(4, 5003), 12)
        assert np.array_equal(gt, ot)
        assert np.allclose(gl, ol, rtol=1e-14, atol=1e-12)


# ------------------------------------------------------------------------ draft tree
@pytest.mark.parametrize("K,levels,T", [(1, 16, 16), (3, 4, 16), (8, 16, 16), (4, 2, 5),
                                        (2, 6, 40), (8, 6, 64), (64, 3, 64), (2, 64, 64)])
def test_draft_tree_random(orc, K, levels, T):
    rng = np.random.default_rng(K * 100 + levels)
    B, V = 5, 700
    rows = rng.normal(0, 2, size=(B, T, V)).astype(np.float32)
    roots = rng.integers(0, V, size=B).astype(np.int32)
    check_draft(orc, rows, roots, K, levels, label="random")


def test_draft_tree_ties(orc):
    """Identical rows (equal keys through different paths), rows where every token ties,
    and rows with a single finite entry (log-prob 0)."""
    rng = np.random.default_rng(41)
    B, T, V = 4, 32, 300
    rows = np.empty((B, T, V), np.float32)
    rows[0] = rng.normal(0, 1, size=V).astype(np.float32)[None]
    rows[1] = 0.25
    rows[2] = -np.inf
    rows[2][:, 7] = 3.0
    rows[3] = (np.round(rng.normal(0, 1, size=(T, V)) * 2) / 2).astype(np.float32)
    roots = np.array([1, 2, 3, 4], np.int32)
    check_draft(orc, rows, roots, 4, 6, label="ties")
    check_draft(orc, rows, roots, 3, 32, label="ties")


def test_draft_tree_edges(orc):
    rng = np.random.default_rng(43)
    rows = rng.normal(0, 2, size=(3, 1, 100)).astype(np.float32)
    g = check_draft(orc, rows, np.array([5, 6, 7], np.int32), 4, 3, label="T=1")
    assert g[0].tolist() == [[-1]] * 3 and g[1][:, 0].tolist() == [5, 6, 7]
    rows = rng.normal(0, 2, size=(2, 7, 3)).astype(np.float32)
    check_draft(orc, rows, np.array([0, 1], np.int32), 3, 3, label="K=V")
    rows = rng.normal(0, 2, size=(2, 4, 50)).astype(np.float32)
    check_draft(orc, rows, np.array([0, 1], np.int32), 3, 2, label="star")
    rows[1, 0, :] = np.nan                                   # root row without a finite entry
    check_draft(orc, rows, np.array([0, 1], np.int32), 2, 4, label="empty root row")


def test_draft_tree_full_size(orc):
    """The batched 8K shape: 32 sequences, a 64-node tree of 6 levels, top-8 expansion over
    151936-token drafter rows; the tree then passes the mask builder."""
    w = wl.WORKLOADS["batched8k"]
    dl, roots = wl.make_drafter_inputs(w, seed=1, device=DEV)
    rows, r = to_np(dl), to_np(roots)
    g = check_draft(orc, rows, r, w.topk, w.max_levels, label="batched8k")
    mask = torch.empty((w.B, w.T, 1), dtype=torch.int64, device=DEV)
    depth = torch.empty((w.B, w.T), dtype=torch.int32, device=DEV)
    err = torch.full((w.B,), -7, dtype=torch.int32, device=DEV)
    sv.sv_build_tree_mask(_dev(g[0]), mask, depth, err)
    torch.cuda.synchronize()
    assert np.all(to_np(err) == 0) and to_np(depth).max() <= w.max_levels - 1
