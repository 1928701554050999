"""Pins of the oracle against facts that do not come from the oracle itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with: values printed on the pages (golden files), hand-derived worked
examples, closed forms, library routines that compute a special case (torch
scaled_dot_product_attention in fp64, numpy argmax / nanargmax), brute force on
tiny inputs, or invariants.  ``tests/test_oracle_pins.py`` runs them against the
real oracle; ``tests/test_oracle_mutants.py`` runs them against deliberately
broken copies of it, each of which must fail at least one pin.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from _support import as_f64, gather_prefix, to_np
import oracle as O
from tree_masked_verify_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# =========================================================================== helpers
def closure_mask(parents: np.ndarray) -> np.ndarray:
    """Ancestor-or-self relation by transitive closure of the parent relation
    (boolean matrix powers), as bool [T, T]: R[i, j] = j is i or an ancestor of i."""
    T = len(parents)
    A = np.zeros((T, T), dtype=bool)
    for i, p in enumerate(parents):
        if p >= 0:
            A[i, p] = True
    R = np.eye(T, dtype=bool) | A
    for _ in range(int(math.ceil(math.log2(max(T, 2)))) + 1):
        R = R | ((R.astype(np.int64) @ R.astype(np.int64)) > 0)
    return R


def bits_of(mask_row: np.ndarray, T: int) -> np.ndarray:
    out = np.zeros(T, dtype=bool)
    for j in range(T):
        out[j] = (int(mask_row[j // 64]) >> (j % 64)) & 1
    return out


def small_inputs(name: str, seed: int, **kw) -> wl.Inputs:
    w = wl.scaled(wl.WORKLOADS[name], **kw)
    return wl.make_inputs(w, seed=seed, device="cpu")


def contiguous_cache(kc: np.ndarray, vc: np.ndarray, dtype: int) -> O.Cache:
    """kc, vc [B, Hkv, cap, D] -> Cache with one block per sequence."""
    B, Hkv, cap, D = kc.shape
    table = np.arange(B, dtype=np.int32).reshape(B, 1)
    return O.Cache(k=np.ascontiguousarray(kc), v=np.ascontiguousarray(vc), table=table,
                   block_size=cap, block_stride=Hkv * cap * D, head_stride=cap * D,
                   row_stride=D, num_blocks=B, dtype=dtype)


def sdpa_reference(q, kp, vp, kt, vt, allowed, scale):
    """fp64 torch SDPA for one sequence.  q [Hq,T,D]; kp/vp [Hkv,P,D] prefix;
    kt/vt [Hkv,T,D] tree; allowed bool [T,T] (tree visibility).  -> [T,Hq,D]."""
    Hq, T, D = q.shape
    P = kp.shape[1]
    k = torch.cat([torch.from_numpy(kp), torch.from_numpy(kt)], dim=1)[None]
    v = torch.cat([torch.from_numpy(vp), torch.from_numpy(vt)], dim=1)[None]
    m = torch.cat([torch.ones(T, P, dtype=torch.bool), torch.from_numpy(allowed)], dim=1)
    o = F.scaled_dot_product_attention(torch.from_numpy(q)[None], k, v, attn_mask=m,
                                       scale=scale, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()   # [T, Hq, D]


def run_attention(orc: O.Oracle, inp: wl.Inputs, mask=None, scale=None, cache=None,
                  prefix=None):
    if mask is None:
        mask, _, _ = orc.build_tree_mask(to_np(inp.parents))
    cache = cache or _cache(inp)
    return orc.tree_verify_attention(
        to_np(inp.q), to_np(inp.k_tree), to_np(inp.v_tree), cache,
        to_np(inp.prefix_len) if prefix is None else prefix, inp.max_prefix_len, mask,
        inp.scale if scale is None else scale)


def _cache(inp):
    from _support import oracle_cache
    return oracle_cache(inp)


def check_vs_sdpa(orc, inp, scale=None, atol=2e-6, rtol=2e-6):
    scale = inp.scale if scale is None else scale
    out = run_attention(orc, inp, scale=scale)
    cache = _cache(inp)
    dt = cache.dtype
    parents = to_np(inp.parents)
    P = to_np(inp.prefix_len)
    q, kt, vt = to_np(inp.q), to_np(inp.k_tree), to_np(inp.v_tree)
    for b in range(inp.w.B):
        Hkv = inp.w.Hkv
        kp = np.stack([gather_prefix(cache, b, h, int(P[b]), "k") for h in range(Hkv)])
        vp = np.stack([gather_prefix(cache, b, h, int(P[b]), "v") for h in range(Hkv)])
        ref = sdpa_reference(as_f64(q[b], dt), kp, vp, as_f64(kt[b], dt), as_f64(vt[b], dt),
                             closure_mask(parents[b]), scale)
        np.testing.assert_allclose(out[b].astype(np.float64), ref, rtol=rtol, atol=atol)


# =========================================================================== mask pins
def pin_mask_worked_example(orc):
    with open(os.path.join(GOLDEN, "mask_worked_example.txt")) as f:
        lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    parents = np.array([int(x) for x in lines[0][1:]], dtype=np.int32)[None]
    want_mask = [int(l[1], 16) for l in lines[1:]]
    want_depth = [int(l[2]) for l in lines[1:]]
    mask, depth, err = orc.build_tree_mask(parents)
    assert err[0] == O.TREE_OK
    assert [int(x) for x in mask[0, :, 0]] == want_mask, mask[0, :, 0]
    assert list(depth[0]) == want_depth


def pin_mask_closed_forms(orc):
    for T in (1, 2, 7, 63, 64):
        chain = np.array([wl.chain_tree(T)], dtype=np.int32)
        mask, depth, err = orc.build_tree_mask(chain)
        assert err[0] == 0
        for i in range(T):  # causal: lower triangle including the diagonal
            assert int(mask[0, i, 0]) == (1 << (i + 1)) - 1, (T, i)
            assert depth[0, i] == i
        star = np.array([[-1] + [0] * (T - 1)], dtype=np.int32)
        mask, depth, err = orc.build_tree_mask(star)
        assert int(mask[0, 0, 0]) == 1
        for i in range(1, T):
            assert int(mask[0, i, 0]) == 1 | (1 << i)
            assert depth[0, i] == 1


def pin_mask_bruteforce(orc):
    rng = np.random.Generator(np.random.PCG64(11))
    trees = []
    for T, lv, ch in ((8, 4, 3), (60, 8, 4), (64, 6, 8), (64, 64, 1), (100, 10, 3)):
        trees.append(np.array(wl.random_tree(rng, T, lv, ch), dtype=np.int32))
    trees.append(np.array(wl.eagle2_tree(rng, 64, 6, 8), dtype=np.int32))
    for par in trees:
        T = len(par)
        mask, depth, err = orc.build_tree_mask(par[None])
        assert err[0] == 0
        R = closure_mask(par)
        for i in range(T):
            assert np.array_equal(bits_of(mask[0, i], T), R[i]), (T, i)
            assert depth[0, i] == R[i].sum() - 1


def pin_mask_invalid(orc):
    cases = [([0, 0, 1], O.TREE_BAD_ROOT), ([-1, 1, 0], O.TREE_BAD_PARENT),
             ([-1, 0, 2], O.TREE_BAD_PARENT), ([-1, 0, -1], O.TREE_BAD_PARENT),
             ([-1, -2, 0], O.TREE_BAD_PARENT), ([-1, 0, 5], O.TREE_BAD_PARENT),
             ([3, 0, 9], O.TREE_BAD_ROOT)]
    for par, code in cases:
        mask, depth, err = orc.build_tree_mask(np.array([par], dtype=np.int32))
        assert err[0] == code, (par, err)
        for i in range(3):
            assert int(mask[0, i, 0]) == 1 << i and depth[0, i] == 0
    # a bad sequence does not disturb its neighbours
    par = np.array([[-1, 0, 1], [-1, 2, 0], [-1, 0, 0]], dtype=np.int32)
    mask, depth, err = orc.build_tree_mask(par)
    assert list(err) == [0, O.TREE_BAD_PARENT, 0]
    assert [int(x) for x in mask[0, :, 0]] == [1, 3, 7]
    assert [int(x) for x in mask[2, :, 0]] == [1, 3, 5]


# =========================================================================== attention pins
def pin_attn_decode_T1(orc):
    """Tree of one node = ordinary single-token decode over prefix + self."""
    inp = small_inputs("parity512", 3, T=1, tree="chain", prefix=(37, 37), capacity=64)
    check_vs_sdpa(orc, inp)


def pin_attn_chain_causal(orc):
    """Chain = causal attention over prefix + chain (torch tril mask)."""
    inp = small_inputs("parity512", 4, T=8, tree="chain", prefix=(45, 45), capacity=64)
    out = run_attention(orc, inp)
    cache = _cache(inp)
    P = int(inp.max_prefix_len)
    kp = np.stack([gather_prefix(cache, 0, h, P, "k") for h in range(2)])
    vp = np.stack([gather_prefix(cache, 0, h, P, "v") for h in range(2)])
    k = torch.cat([torch.from_numpy(kp), torch.from_numpy(as_f64(to_np(inp.k_tree)[0], 1))], 1)
    v = torch.cat([torch.from_numpy(vp), torch.from_numpy(as_f64(to_np(inp.v_tree)[0], 1))], 1)
    causal = torch.ones(8, P + 8, dtype=torch.bool).tril(diagonal=P)
    q = torch.from_numpy(as_f64(to_np(inp.q)[0], 1))
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=causal,
                                         enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out[0].astype(np.float64), ref, rtol=2e-6, atol=2e-6)


def pin_attn_tree_vs_sdpa(orc):
    """Random trees, GQA, paged shuffled cache, explicit scale; fp32 and bf16."""
    check_vs_sdpa(orc, small_inputs("parity512", 5, prefix=(0, 90), B=3))
    check_vs_sdpa(orc, small_inputs("long32k", 6, B=2, prefix=(33, 70), T=21, Hq=8, Hkv=2, V=1000,
                                    max_levels=5), scale=0.3)
    check_vs_sdpa(orc, small_inputs("tiny", 7, Hq=4, Hkv=2, D=64))
    check_vs_sdpa(orc, small_inputs("chain2k", 8, prefix=(20, 20), capacity=32, D=96, V=1000))


def pin_attn_prefix_zero(orc):
    check_vs_sdpa(orc, small_inputs("parity512", 9, prefix=(0, 0), capacity=16))


def pin_attn_closed_forms(orc):
    """Constant V -> O = V; equal keys -> O = mean of the visible V rows, which
    also fixes the [node, head, dim] output layout and the head -> kv-head map."""
    inp = small_inputs("long32k", 12, B=2, prefix=(5, 19), T=9, Hq=6, Hkv=3, D=32,
                       max_levels=4, dtype="f32", block_size=4)
    w = inp.w
    parents = to_np(inp.parents)
    cache = _cache(inp)
    P = to_np(inp.prefix_len)
    q = to_np(inp.q)
    kt = np.zeros_like(to_np(inp.k_tree))
    # V rows encode (kv head, position): cache row p of kv head h -> 1000*h + p, tree
    # row j -> 1000*h + 500 + j, repeated along D.
    vt = np.zeros_like(kt)
    for b in range(w.B):
        for h in range(w.Hkv):
            vt[b, h, :, :] = (1000 * h + 500 + np.arange(w.T))[:, None]
    kpool = np.zeros_like(cache.k)
    vpool = np.zeros_like(cache.v)
    for b in range(w.B):
        for p in range(int(P[b]) + w.T):
            blk = cache.table[b, p // cache.block_size]
            for h in range(w.Hkv):
                vpool[blk, h, p % cache.block_size, :] = 1000 * h + p
    c2 = O.Cache(k=kpool, v=vpool, table=cache.table, block_size=cache.block_size,
                 block_stride=cache.block_stride, head_stride=cache.head_stride,
                 row_stride=cache.row_stride, num_blocks=cache.num_blocks, dtype=O.F32)
    mask, _, _ = orc.build_tree_mask(parents)
    out = orc.tree_verify_attention(q, kt, vt, c2, P, inp.max_prefix_len, mask, 0.7)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        R = closure_mask(parents[b])
        for i in range(w.T):
            for h in range(w.Hq):
                kvh = h // G
                vals = [1000 * kvh + p for p in range(int(P[b]))]
                vals += [1000 * kvh + 500 + j for j in range(w.T) if R[i, j]]
                want = np.float32(np.mean(np.array(vals, dtype=np.float64)))
                assert np.all(out[b, i, h] == want), (b, i, h, out[b, i, h, 0], want)
    # constant V: output equals that constant whatever Q and K are
    out = orc.tree_verify_attention(q, to_np(inp.k_tree), np.full_like(vt, 2.5), O.Cache(
        k=cache.k, v=np.full_like(cache.v, 2.5), table=cache.table,
        block_size=cache.block_size, block_stride=cache.block_stride,
        head_stride=cache.head_stride, row_stride=cache.row_stride,
        num_blocks=cache.num_blocks, dtype=O.F32), P, inp.max_prefix_len, mask, inp.scale)
    np.testing.assert_allclose(out, 2.5, rtol=1e-6)


def pin_attn_paged_equals_contiguous(orc):
    """The same rows laid out paged (shuffled blocks) or contiguous give identical bits."""
    inp = small_inputs("batched8k", 13, B=3, prefix=(10, 77), T=12, Hq=4, Hkv=2, D=64)
    paged = _cache(inp)
    P = to_np(inp.prefix_len)
    cap = int(P.max()) + inp.w.T
    B, Hkv, D = inp.w.B, inp.w.Hkv, inp.w.D
    kc = np.zeros((B, Hkv, cap, D), dtype=paged.k.dtype)
    vc = np.zeros_like(kc)
    pool4k = paged.k.reshape(paged.num_blocks, Hkv, paged.block_size, D)
    pool4v = paged.v.reshape(paged.num_blocks, Hkv, paged.block_size, D)
    for b in range(B):
        for p in range(int(P[b])):
            blk = paged.table[b, p // paged.block_size]
            kc[b, :, p] = pool4k[blk, :, p % paged.block_size]
            vc[b, :, p] = pool4v[blk, :, p % paged.block_size]
    a = run_attention(orc, inp)
    c = run_attention(orc, inp, cache=contiguous_cache(kc, vc, paged.dtype))
    assert np.array_equal(a, c)


def pin_attn_bad_block_entry(orc):
    """A prefix block whose table entry is out of range drops exactly its rows."""
    inp = small_inputs("batched8k", 14, B=1, prefix=(70, 70), T=5, Hq=2, Hkv=1, D=32,
                       max_levels=3)
    cache = _cache(inp)
    table = cache.table.copy()
    table[0, 2] = -1                       # positions 32..47
    c_bad = O.Cache(**{**cache.__dict__, "table": table})
    out = run_attention(orc, inp, cache=c_bad)
    keep = [p for p in range(70) if not (32 <= p < 48)]
    kp = np.stack([gather_prefix(cache, 0, 0, 70, "k")[keep]])
    vp = np.stack([gather_prefix(cache, 0, 0, 70, "v")[keep]])
    ref = sdpa_reference(as_f64(to_np(inp.q)[0], 1), kp, vp, as_f64(to_np(inp.k_tree)[0], 1),
                         as_f64(to_np(inp.v_tree)[0], 1), closure_mask(to_np(inp.parents)[0]),
                         inp.scale)
    np.testing.assert_allclose(out[0].astype(np.float64), ref, rtol=2e-6, atol=2e-6)


def pin_attn_chain_equals_serial(orc):
    """A chain verified as one tree equals T serial one-node verifies, each followed
    by a commit of its root (bit for bit: the same keys in the same order)."""
    inp = small_inputs("chain2k", 15, prefix=(50, 50), capacity=64, D=64, Hq=4)
    w = inp.w
    chain = run_attention(orc, inp)
    cache = _cache(inp)
    q, kt, vt = to_np(inp.q), to_np(inp.k_tree), to_np(inp.v_tree)
    P = to_np(inp.prefix_len).copy()
    one = np.array([[-1]], dtype=np.int32)
    m1, _, e1 = orc.build_tree_mask(one)
    for i in range(w.T):
        qi = np.ascontiguousarray(q[:, :, i:i + 1])
        ki = np.ascontiguousarray(kt[:, :, i:i + 1])
        vi = np.ascontiguousarray(vt[:, :, i:i + 1])
        o = orc.tree_verify_attention(qi, ki, vi, cache, P, int(P.max()), m1, inp.scale)
        assert np.array_equal(o[0, 0], chain[0, i]), i
        P = orc.kv_commit(ki, vi, np.array([1], np.int32), np.array([[0]], np.int32), e1, cache,
                          P, int(P.max()))


# =========================================================================== argmax pins
def pin_argmax_numpy(orc):
    rng = np.random.Generator(np.random.PCG64(21))
    x = rng.standard_normal((64, 1000)).astype(np.float32)
    assert np.array_equal(orc.argmax(x), np.argmax(x, axis=1))
    # ties: small integer-valued rows have repeated maxima; numpy returns the first
    y = rng.integers(0, 5, size=(200, 37)).astype(np.float32)
    assert np.array_equal(orc.argmax(y), np.argmax(y, axis=1))


def pin_argmax_special_values(orc):
    rng = np.random.Generator(np.random.PCG64(22))
    x = rng.integers(-3, 3, size=(300, 50)).astype(np.float32)
    x[rng.random(x.shape) < 0.2] = np.nan
    x[5, :] = np.nan
    want = np.array([np.nanargmax(r) if not np.all(np.isnan(r)) else 0 for r in x])
    assert np.array_equal(orc.argmax(x), want)
    z = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0], [-np.inf, -np.inf, -np.inf],
                  [np.nan, np.inf, np.inf], [np.nan, -np.inf, np.nan]], dtype=np.float32)
    assert list(orc.argmax(z)) == [0, 0, 0, 1, 1]


def pin_argmax_planted(orc):
    """The generator draws each row's maximum position first; the oracle finds it."""
    gen = torch.Generator().manual_seed(5)
    x, pos = wl.planted_max_logits(40, 5000, 2.0, gen, torch.device("cpu"))
    assert np.array_equal(orc.argmax(x.numpy()), pos.numpy())


# =========================================================================== accept pins
def brute_force_accept(logits, draft, parents):
    """Enumerate every root path; keep those whose every edge matches; the longest
    wins, ties to the smallest end node."""
    T = len(parents)
    a = np.argmax(logits, axis=1)
    best = None
    for end in range(T):
        path, n = [], end
        while n != -1:
            path.append(n)
            n = parents[n]
        path = path[::-1]
        if all(draft[path[k]] == a[path[k - 1]] for k in range(1, len(path))):
            if best is None or len(path) > len(best):
                best = path
    return a, best


def pin_accept_bruteforce(orc):
    rng = np.random.Generator(np.random.PCG64(31))
    for trial in range(60):
        T = int(rng.integers(1, 20))
        V = int(rng.integers(2, 6))
        # random recursive tree: node i picks any earlier node as parent
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)], dtype=np.int32)
        logits = rng.standard_normal((T, V)).astype(np.float32)
        draft = rng.integers(0, V, size=T).astype(np.int32)
        am, L, nodes, toks = orc.accept_longest_path(logits[None], draft[None], par[None])
        a, path = brute_force_accept(logits, draft, par)
        assert np.array_equal(am[0], a)
        assert L[0] == len(path), (trial, L[0], path)
        assert list(nodes[0, :L[0]]) == path
        assert list(toks[0, :L[0]]) == [a[n] for n in path]
        assert np.all(nodes[0, L[0]:] == -1) and np.all(toks[0, L[0]:] == -1)


def pin_accept_edge_cases(orc):
    T, V = 6, 10
    par = np.array([wl.chain_tree(T)], dtype=np.int32)
    logits = np.zeros((1, T, V), np.float32)
    for i in range(T):
        logits[0, i, (3 * i + 1) % V] = 1.0          # argmax of row i = (3i+1) % V
    a = [(3 * i + 1) % V for i in range(T)]
    full = np.array([[7] + [a[i - 1] for i in range(1, T)]], np.int32)
    _, L, nodes, toks = orc.accept_longest_path(logits, full, par)
    assert L[0] == T and list(nodes[0]) == list(range(T)) and list(toks[0]) == a
    none = full.copy()
    none[0, 1] = (a[0] + 1) % V
    _, L, nodes, toks = orc.accept_longest_path(logits, none, par)
    assert L[0] == 1 and nodes[0, 0] == 0 and toks[0, 0] == a[0]
    assert np.all(nodes[0, 1:] == -1)
    # the anchor's own draft token is never read
    for d0 in (0, 5, -9, 10 ** 6):
        f2 = full.copy()
        f2[0, 0] = d0
        assert orc.accept_longest_path(logits, f2, par)[1][0] == T
    # invalid tree (given or detected) accepts nothing
    _, L, nodes, toks = orc.accept_longest_path(logits, full, par, np.array([2], np.int32))
    assert L[0] == 0 and np.all(nodes == -1) and np.all(toks == -1)
    bad = par.copy()
    bad[0, 3] = 4
    _, L, _, _ = orc.accept_longest_path(logits, full, bad)
    assert L[0] == 0
    # duplicate sibling tokens: the longest matching path wins, not the first match
    par = np.array([[-1, 0, 0, 2]], np.int32)
    lg = np.zeros((1, 4, 4), np.float32)
    lg[0, :, 1] = 1.0                                 # every argmax is 1
    drf = np.array([[0, 1, 1, 1]], np.int32)
    _, L, nodes, _ = orc.accept_longest_path(lg, drf, par)
    assert L[0] == 3 and list(nodes[0, :3]) == [0, 2, 3]
    # T = 1: the root alone, its argmax is the bonus token
    _, L, nodes, toks = orc.accept_longest_path(lg[:, :1], drf[:, :1], par[:, :1])
    assert L[0] == 1 and nodes[0, 0] == 0 and toks[0, 0] == 1


def _monte_carlo_chain(orc, K, p, n, seed):
    """Chain of K drafts; each draft equals its parent's argmax with probability
    exactly p (else one of the other V-1 tokens)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, V = K + 1, 4
    top = rng.integers(0, V, size=(n, T))
    logits = np.zeros((n, T, V), np.float32)
    logits[np.arange(n)[:, None], np.arange(T)[None], top] = 1.0
    hit = rng.random((n, T)) < p
    other = (top + rng.integers(1, V, size=(n, T))) % V
    draft = np.zeros((n, T), np.int32)
    draft[:, 1:] = np.where(hit[:, 1:], top[:, :-1], other[:, :-1])
    par = np.tile(np.array(wl.chain_tree(T), np.int32), (n, 1))
    _, L, _, _ = orc.accept_longest_path(logits, draft, par)
    return L.astype(np.float64)


def pin_accept_expected_tokens_golden(orc):
    with open(os.path.join(GOLDEN, "expected_tokens_per_burst.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for K, p, printed in rows:
        K, p, printed = int(K), float(p), float(printed)
        L = _monte_carlo_chain(orc, K, p, 400_000, seed=int(p * 100))
        sigma = L.std() / math.sqrt(len(L))
        assert abs(L.mean() - printed) <= 0.005 + 5 * sigma, (K, p, L.mean(), printed)


def pin_accept_expected_tokens_closed_form(orc):
    """Generalised chain: E[L] = sum_{k=0..K} p^k (K=7, p=0.5 -> 1.9921875)."""
    for K, p in ((7, 0.5), (1, 0.8), (5, 0.9)):
        L = _monte_carlo_chain(orc, K, p, 200_000, seed=K * 7 + int(10 * p))
        want = sum(p ** k for k in range(K + 1))
        sigma = L.std() / math.sqrt(len(L))
        assert abs(L.mean() - want) <= 5 * sigma + 1e-9, (K, p, L.mean(), want)


# =========================================================================== sampled accept pins
def _p64(row, tau):
    """Target distribution of one logits row in fp64 (numpy; -inf entries give 0)."""
    l = np.asarray(row, np.float64) / tau
    e = np.exp(l - l.max())
    return e / e.sum()


def pin_sampled_worked_examples(orc):
    """Hand-derived cases of the rule: proposals tried in node order, a rejected
    token is excluded and the rest renormalised, strict comparison u * R < p."""
    lg = np.log(np.array([[0.5, 0.3, 0.2], [1, 1, 1], [1, 1, 1], [0.1, 0.1, 0.8]],
                         np.float32))[None]
    par = np.array([[-1, 0, 0, 0]], np.int32)
    drf = np.array([[0, 0, 0, 1]], np.int32)
    us = np.array([[0.0, 0.0, 0.0, 0.15]], np.float32)
    # node 1 (token 0): 0.6 >= 0.5, rejected, R = 0.5; node 2 repeats token 0: p = 0;
    # node 3 (token 1): 0.59 * 0.5 < 0.3, accepted; leaf: cumulative 0.1, 0.2 > 0.15
    L, nodes, toks = orc.accept_sampled(lg, drf, par, np.array([[0, 0.6, 0.0, 0.59]], np.float32),
                                        us, 1.0)
    assert L[0] == 2 and list(nodes[0]) == [0, 3, -1, -1] and list(toks[0]) == [1, 1, -1, -1]
    # 0.61 * 0.5 >= 0.3: every proposal rejected, E = {0, 1}, R = 0.2; only token 2 is left
    us2 = np.array([[0.99, 0.0, 0.0, 0.15]], np.float32)
    L, nodes, toks = orc.accept_sampled(lg, drf, par, np.array([[0, 0.6, 0.0, 0.61]], np.float32),
                                        us2, 1.0)
    assert L[0] == 1 and nodes[0, 0] == 0 and toks[0, 0] == 2 and np.all(toks[0, 1:] == -1)
    # equal logits give p = 0.5 exactly: u = 0.5 rejects (strict), the next float below accepts
    lg2 = np.zeros((1, 2, 2), np.float32)
    par2 = np.array([[-1, 0]], np.int32)
    drf2 = np.array([[0, 0]], np.int32)
    half = np.float32(0.5)
    L, _, toks = orc.accept_sampled(lg2, drf2, par2, np.array([[0, half]], np.float32),
                                    np.array([[0.3, 0.3]], np.float32), 1.0)
    assert L[0] == 1 and toks[0, 0] == 1            # token 0 excluded: token 1 is drawn
    below = np.nextafter(half, np.float32(0))
    L, _, toks = orc.accept_sampled(lg2, drf2, par2, np.array([[0, below]], np.float32),
                                    np.array([[0.3, 0.3]], np.float32), 1.0)
    assert L[0] == 2 and list(toks[0]) == [0, 0]     # row 1: cumulative 0.5 > 0.3 at token 0
    # temperature: logits (0, ln 3) give p = (1/4, 3/4) at tau 1 and (1/10, 9/10) at tau 1/2
    lg3 = np.zeros((1, 2, 2), np.float32)
    lg3[0, :, 1] = np.float32(math.log(3.0))
    ua = np.array([[0, 0.2]], np.float32)
    assert orc.accept_sampled(lg3, drf2, par2, ua, np.array([[0.5, 0.5]], np.float32), 1.0)[0][0] == 2
    assert orc.accept_sampled(lg3, drf2, par2, ua, np.array([[0.5, 0.5]], np.float32), 0.5)[0][0] == 1
    # a row with no finite logit: every proposal has p = 0 and token 0 is emitted
    lg4 = np.full((1, 2, 3), -np.inf, np.float32)
    L, _, toks = orc.accept_sampled(lg4, np.array([[0, 2]], np.int32), par2,
                                    np.array([[0, 0.0]], np.float32),
                                    np.array([[0.7, 0.7]], np.float32), 1.0)
    assert L[0] == 1 and toks[0, 0] == 0
    # NaN entries have probability 0: row (NaN, 0, 0) is (0, 1/2, 1/2)
    lg5 = np.zeros((1, 2, 3), np.float32)
    lg5[0, 0, 0] = np.nan
    L, _, toks = orc.accept_sampled(lg5, np.array([[0, 0]], np.int32), par2,
                                    np.array([[0, 0.0]], np.float32),
                                    np.array([[0.6, 0.6]], np.float32), 1.0)
    assert L[0] == 1 and toks[0, 0] == 2
    # an invalid tree accepts nothing
    L, nodes, toks = orc.accept_sampled(lg, drf, par, np.zeros((1, 4), np.float32), us, 1.0,
                                        np.array([1], np.int32))
    assert L[0] == 0 and np.all(nodes == -1) and np.all(toks == -1)


def pin_sampled_expected_tokens_golden(orc):
    """A K-draft chain whose every row gives its child's draft token probability p:
    each position is accepted with probability p, so the mean burst length is the
    pages' 1 + p + p^2 + p^3 (K = 3: 1.42 at 30%, 1.88 at 50%)."""
    with open(os.path.join(GOLDEN, "expected_tokens_per_burst.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for K, p, printed in rows:
        K, p, printed = int(K), float(p), float(printed)
        n, T, V = 200_000, K + 1, 4
        rng = np.random.Generator(np.random.PCG64(int(p * 1000) + 17))
        tok = rng.integers(0, V, size=(n, T)).astype(np.int32)   # draft token of each node
        lg = np.full((n, T, V), np.float32(math.log((1 - p) / (V - 1))), np.float32)
        nxt = np.concatenate([tok[:, 1:], tok[:, :1]], axis=1)      # row i favours node i+1's token
        lg[np.arange(n)[:, None], np.arange(T)[None], nxt] = np.float32(math.log(p))
        par = np.tile(np.array(wl.chain_tree(T), np.int32), (n, 1))
        ua, us = wl.make_uniforms(n, T, seed=K)
        L, _, _ = orc.accept_sampled(lg, tok, par, ua, us, 1.0)
        L = L.astype(np.float64)
        sigma = L.std() / math.sqrt(n)
        assert abs(L.mean() - printed) <= 0.005 + 5 * sigma, (K, p, L.mean(), printed)


def pin_sampled_preserves_target(orc):
    """Monte Carlo: the first emitted token follows the root's target distribution,
    and after an accepted child the next one follows that child's (the property the
    rule exists for).  Node 2 repeats node 1's token, so it is never accepted."""
    rng = np.random.Generator(np.random.PCG64(77))
    par1 = np.array([-1, 0, 0, 0, 1, 1, 3], np.int32)
    drf1 = np.array([0, 2, 2, 4, 0, 3, 1], np.int32)
    T, V, tau, n = len(par1), 5, 0.7, 60_000
    rows = rng.normal(0.0, 1.0, size=(T, V)).astype(np.float32)
    lg = np.tile(rows[None], (n, 1, 1))
    par = np.tile(par1[None], (n, 1))
    drf = np.tile(drf1[None], (n, 1))
    ua, us = wl.make_uniforms(n, T, seed=99)
    L, nodes, toks = orc.accept_sampled(lg, drf, par, ua, us, tau)

    def check(sel, want, what):
        m = int(sel.sum())
        assert m > 2000, (what, m)
        got = np.bincount(toks[sel, 0 if what == "root" else 1], minlength=V)[:V] / m
        sig = np.sqrt(want * (1 - want) / m)
        assert np.all(np.abs(got - want) <= 5 * sig + 1e-12), (what, got, want)
    check(np.ones(n, bool), _p64(rows[0], tau), "root")
    # after child 1 (token 2) is accepted the next token follows row 1; after child 3
    # (token 4) row 3
    for c in (1, 3):
        sel = (L >= 2) & (nodes[:, 1] == c)
        m = int(sel.sum())
        assert m > 2000, (c, m)
        got = np.bincount(toks[sel, 1], minlength=V)[:V] / m
        want = _p64(rows[c], tau)
        sig = np.sqrt(want * (1 - want) / m)
        assert np.all(np.abs(got - want) <= 5 * sig + 1e-12), (c, got, want)
    assert not np.any(nodes == 2)
    # acceptance rates: node 1 with p_root(2); node 3 after both token-2 proposals fail
    p0 = _p64(rows[0], tau)
    r1 = np.mean(nodes[:, 1] == 1)
    assert abs(r1 - p0[2]) <= 5 * math.sqrt(p0[2] * (1 - p0[2]) / n)


def pin_sampled_low_temperature_is_greedy(orc):
    """As the temperature goes to 0 the target distribution is the argmax: with
    distinct sibling tokens and well-separated maxima the sampled rule accepts
    exactly the greedy longest matching path and emits the same tokens."""
    rng = np.random.Generator(np.random.PCG64(41))
    for trial in range(40):
        T = int(rng.integers(1, 24))
        V = int(rng.integers(4, 40))
        par = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, T)], np.int32)
        top = rng.integers(0, V, size=T)
        lg = rng.uniform(-1.0, 0.0, size=(T, V)).astype(np.float32)
        lg[np.arange(T), top] = 1.0                      # maxima 1 apart from the rest
        drf = np.zeros(T, np.int32)
        kids_of = [[c for c in range(T) if par[c] == v] for v in range(T)]
        if max(len(k) for k in kids_of) > V:
            continue
        for v in range(T):
            toks = rng.permutation(V)[:len(kids_of[v])]          # distinct sibling tokens
            if len(toks) and top[v] not in toks and rng.random() < 0.7:
                toks[0] = top[v]                                 # one child proposes the argmax
            for c, t in zip(kids_of[v], toks):
                drf[c] = t
        ua, us = wl.make_uniforms(1, T, seed=trial)
        _, Lg, ng, tg = orc.accept_longest_path(lg[None], drf[None], par[None])
        Ls, ns, ts = orc.accept_sampled(lg[None], drf[None], par[None], ua, us, 1e-3)
        assert Ls[0] == Lg[0] and np.array_equal(ns, ng) and np.array_equal(ts, tg), trial


def pin_sampled_invariants(orc):
    """On workload-shaped inputs: the path is a root path, the emitted tokens are the
    accepted children's draft tokens then one drawn token, and the drawn token is
    none of the final node's children's tokens (all of them were rejected)."""
    for name, seed in (("tiny", 3), ("parity512", 4), ("batched8k", 5)):
        kw = {"V": 2048} if name == "batched8k" else {}
        if name == "batched8k":
            kw.update(B=3, prefix=(16, 32))
        inp = small_inputs(name, seed, **kw)
        lg, drf, par = to_np(inp.logits), to_np(inp.draft), to_np(inp.parents)
        B, T = par.shape
        ua, us = wl.make_uniforms(B, T, seed)
        L, nodes, toks = orc.accept_sampled(lg, drf, par, ua, us, inp.w.temperature)
        for b in range(B):
            assert 1 <= L[b] <= T
            path = list(nodes[b, :L[b]])
            assert path[0] == 0 and np.all(nodes[b, L[b]:] == -1) and np.all(toks[b, L[b]:] == -1)
            for j in range(1, L[b]):
                assert par[b, path[j]] == path[j - 1] and toks[b, j - 1] == drf[b, path[j]]
            last = path[-1]
            rejected = {int(drf[b, c]) for c in range(T) if par[b, c] == last}
            assert int(toks[b, L[b] - 1]) not in rejected
            assert 0 <= toks[b, L[b] - 1] < lg.shape[-1]


# =========================================================================== RoPE pins
def _bf16_to_f64(a):
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_rope_worked_examples(orc):
    """D = 4, theta = 100: frequencies 1 and 100^(-1/2) = 0.1 (hand-derived); position
    = prefix + depth; position 0 leaves the vector unchanged bit for bit."""
    q = np.zeros((1, 1, 3, 4), np.float32)
    q[0, 0, :, 0] = 1.0                                   # e0 on every node
    k = np.zeros((1, 1, 3, 4), np.float32)
    k[0, 0, :, 1] = 2.0                                   # 2 e1
    depth = np.array([[0, 1, 2]], np.int32)
    qo, ko = orc.rope_tree(q, k, np.array([5], np.int32), depth, 100.0, O.F32)
    for i, pos in enumerate((5, 6, 7)):
        want_q = [math.cos(pos), 0.0, math.sin(pos), 0.0]
        want_k = [0.0, 2 * math.cos(0.1 * pos), 0.0, 2 * math.sin(0.1 * pos)]
        assert np.allclose(qo[0, 0, i], want_q, atol=1e-7), (i, qo[0, 0, i], want_q)
        assert np.allclose(ko[0, 0, i], want_k, atol=2e-7), (i, ko[0, 0, i], want_k)
    rng = np.random.Generator(np.random.PCG64(3))
    x = rng.standard_normal((2, 3, 4, 8)).astype(np.float32)
    y = rng.standard_normal((2, 1, 4, 8)).astype(np.float32)
    x0, y0 = orc.rope_tree(x, y, np.zeros(2, np.int32), np.zeros((2, 4), np.int32), 1e4, O.F32)
    assert np.array_equal(x0, x) and np.array_equal(y0, y)


def pin_rope_relative_position(orc):
    """Rotary embeddings make <R(q, m), R(k, n)> depend on m - n only: shifting every
    position by the same amount (through the prefix) keeps all query-key dot products."""
    rng = np.random.Generator(np.random.PCG64(4))
    B, Hq, Hkv, T, D = 1, 2, 1, 6, 64
    q = rng.standard_normal((B, Hq, T, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    depth = np.array([[0, 1, 1, 2, 3, 2]], np.int32)
    dots = []
    for P in (0, 37, 1000):
        qo, ko = orc.rope_tree(q, k, np.array([P], np.int32), depth, 1e4, O.F32)
        dots.append(np.einsum("hid,jd->hij", qo[0].astype(np.float64), ko[0, 0].astype(np.float64)))
    assert np.allclose(dots[0], dots[1], atol=2e-4) and np.allclose(dots[0], dots[2], atol=2e-4)
    # while rotating one side only does change them
    qo, _ = orc.rope_tree(q, k, np.array([37], np.int32), depth, 1e4, O.F32)
    plain = np.einsum("hid,jd->hij", qo[0].astype(np.float64), k[0, 0].astype(np.float64))
    assert not np.allclose(plain, dots[0], atol=1e-2)


def pin_rope_pairs_and_tree(orc):
    """NeoX pairs (j, j + D/2) keep their norms; a tree node is rotated like the chain
    node at its depth (position = prefix + depth), so siblings with equal inputs agree."""
    rng = np.random.Generator(np.random.PCG64(6))
    T, D = 7, 16
    v = rng.standard_normal(D).astype(np.float32)
    q = np.tile(v, (1, 1, T, 1)).astype(np.float32)
    k = np.tile(v, (1, 2, T, 1)).astype(np.float32)
    tree_depth = np.array([[0, 1, 1, 2, 2, 3, 1]], np.int32)
    chain_depth = np.arange(T, dtype=np.int32)[None]
    qt, kt = orc.rope_tree(q, k, np.array([100], np.int32), tree_depth, 500.0, O.F32)
    qc, _ = orc.rope_tree(q, k, np.array([100], np.int32), chain_depth, 500.0, O.F32)
    for i in range(T):
        assert np.array_equal(qt[0, 0, i], qc[0, 0, tree_depth[0, i]]), i
        assert np.array_equal(kt[0, 1, i], qt[0, 0, i]), i
    n_in = v[:D // 2].astype(np.float64) ** 2 + v[D // 2:].astype(np.float64) ** 2
    for i in range(T):
        r = qt[0, 0, i].astype(np.float64)
        n_out = r[:D // 2] ** 2 + r[D // 2:] ** 2
        assert np.allclose(n_out, n_in, rtol=1e-6, atol=1e-7), i


def pin_rope_bf16_rounding(orc):
    """bf16 tensors: the result is the fp32 result rounded to nearest-even bf16 (the bits
    of the fp32 value's top half, rounded), checked against numpy's own rounding."""
    rng = np.random.Generator(np.random.PCG64(9))
    B, Hq, Hkv, T, D = 2, 2, 1, 5, 32
    qf = rng.standard_normal((B, Hq, T, D)).astype(np.float32)
    kf = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)   # exact: bf16 inputs
    qb = to_bits(qf)
    kb = to_bits(kf)
    P = np.array([3, 900], np.int32)
    depth = np.array([[0, 1, 1, 2, 3], [0, 1, 2, 3, 4]], np.int32)
    q32, k32 = orc.rope_tree(_bf16_to_f64(qb).astype(np.float32), _bf16_to_f64(kb).astype(np.float32),
                             P, depth, 1e4, O.F32)
    qo, ko = orc.rope_tree(qb, kb, P, depth, 1e4, O.BF16)
    t = torch.from_numpy(q32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(qo, t)
    t = torch.from_numpy(k32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ko, t)


# =========================================================================== commit pins
def _commit_case(orc, name, seed, **kw):
    inp = small_inputs(name, seed, **kw)
    parents = to_np(inp.parents)
    mask, _, err = orc.build_tree_mask(parents)
    _, L, nodes, _ = orc.accept_longest_path(to_np(inp.logits), to_np(inp.draft), parents, err)
    return inp, err, L, nodes


def check_commit_invariants(orc, inp, err, L, nodes):
    cache = _cache(inp)
    k0, v0 = cache.k.copy(), cache.v.copy()
    P = to_np(inp.prefix_len)
    npl = orc.kv_commit(to_np(inp.k_tree), to_np(inp.v_tree), L, nodes, err, cache, P,
                        inp.max_prefix_len)
    w = inp.w
    bs = cache.block_size
    kt, vt = to_np(inp.k_tree), to_np(inp.v_tree)
    k4 = lambda a: a.reshape(cache.num_blocks, w.Hkv, bs, w.D)
    expect_k, expect_v = k4(k0.copy()), k4(v0.copy())
    for b in range(w.B):
        if err[b] != 0:
            assert npl[b] == P[b]
            continue
        assert npl[b] == P[b] + L[b]
        for j in range(L[b]):
            pos = P[b] + j
            blk = cache.table[b, pos // bs]
            expect_k[blk, :, pos % bs] = kt[b, :, nodes[b, j]]
            expect_v[blk, :, pos % bs] = vt[b, :, nodes[b, j]]
    assert np.array_equal(k4(cache.k), expect_k)
    assert np.array_equal(k4(cache.v), expect_v)
    changed = np.any(k4(cache.k) != k4(k0), axis=-1).sum()
    assert changed <= int(sum(L[b] for b in range(w.B) if err[b] == 0)) * w.Hkv
    return cache, npl


def pin_commit_invariants(orc):
    inp, err, L, nodes = _commit_case(orc, "batched8k", 41, B=4, prefix=(3, 60), T=20,
                                      Hq=4, Hkv=2, D=32, V=50, max_levels=5)
    assert L.max() > 1                     # something beyond the root was accepted
    check_commit_invariants(orc, inp, err, L, nodes)
    inp, err, L, nodes = _commit_case(orc, "tiny", 42, D=16)
    check_commit_invariants(orc, inp, err, L, nodes)


def pin_commit_single_root(orc):
    inp, err, L, nodes = _commit_case(orc, "parity512", 43, T=1, tree="chain", D=16,
                                      prefix=(9, 9), capacity=16)
    assert L[0] == 1
    cache, npl = check_commit_invariants(orc, inp, err, L, nodes)
    assert npl[0] == 10


def pin_commit_refusals(orc):
    inp, err, L, nodes = _commit_case(orc, "parity512", 44, D=16, B=3, prefix=(5, 9),
                                      capacity=24)
    cache = _cache(inp)
    k0 = cache.k.copy()
    P = to_np(inp.prefix_len)
    bad_err = np.array([1, 0, 0], np.int32)
    L2 = L.copy()
    L2[1] = inp.w.T + 1                    # more rows than tree nodes
    nodes2 = nodes.copy()
    npl = orc.kv_commit(to_np(inp.k_tree), to_np(inp.v_tree), L2, nodes2, bad_err, cache, P,
                        inp.max_prefix_len)
    assert npl[0] == P[0] and npl[1] == P[1] and npl[2] == P[2] + L[2]
    k4 = cache.k.reshape(3, 2, -1, 16)
    k04 = k0.reshape(3, 2, -1, 16)
    assert np.array_equal(k4[0], k04[0]) and np.array_equal(k4[1], k04[1])
    # prefix beyond the declared bound: refused
    cache = _cache(inp)
    npl = orc.kv_commit(to_np(inp.k_tree), to_np(inp.v_tree), L, nodes, err, cache, P,
                        int(P.min()) - 1)
    assert np.array_equal(npl, P) and np.array_equal(cache.k, k0)


def pin_commit_chain_equals_serial(orc):
    """Full accept of a chain leaves the same cache bytes as T serial root commits."""
    inp = small_inputs("chain2k", 45, prefix=(30, 30), capacity=48, D=32, Hq=2, draft_p=1.0,
                       V=64)
    parents = to_np(inp.parents)
    _, _, err = orc.build_tree_mask(parents)
    _, L, nodes, _ = orc.accept_longest_path(to_np(inp.logits), to_np(inp.draft), parents, err)
    assert L[0] == inp.w.T
    c1 = _cache(inp)
    P = to_np(inp.prefix_len)
    orc.kv_commit(to_np(inp.k_tree), to_np(inp.v_tree), L, nodes, err, c1, P, int(P.max()))
    c2 = _cache(inp)
    kt, vt = to_np(inp.k_tree), to_np(inp.v_tree)
    Pi = P.copy()
    for i in range(inp.w.T):
        Pi = orc.kv_commit(np.ascontiguousarray(kt[:, :, i:i + 1]),
                           np.ascontiguousarray(vt[:, :, i:i + 1]), np.array([1], np.int32),
                           np.array([[0]], np.int32), None, c2, Pi, int(Pi.max()))
    assert np.array_equal(c1.k, c2.k) and np.array_equal(c1.v, c2.v)



# ======================================================= top-K and best-first expansion
F32MAX = float(np.finfo(np.float32).max)


def pin_topk_worked_examples(orc):
    """Hand-derived rows: the pages' ordering case [0, -3e38, -2e38] (ADR-037 row
    E4b.10a: choosing on clamped values would merge the two tails), ties to the smaller
    token, NaN / +inf / -inf handling, a row without a finite entry, and K = V."""
    tok, lp = orc.topk_logprobs(np.array([[0.0, -3e38, -2e38]], np.float32), 3)
    assert tok[0].tolist() == [0, 2, 1]
    assert lp[0, 0] == 0.0 and lp[0, 1] == float(np.float32(-2e38))
    assert lp[0, 2] == float(np.float32(-3e38))
    # three tokens at 7, two at 5: p(7) = 1 / (3 + 2 e^-2)
    tok, lp = orc.topk_logprobs(np.array([[5, 7, 7, 5, 7]], np.float32), 4)
    assert tok[0].tolist() == [1, 2, 4, 0]
    top = -math.log(3.0 + 2.0 * math.exp(-2.0))
    assert np.allclose(lp[0], [top, top, top, top - 2.0], rtol=0, atol=1e-15)
    # NaN and -inf have probability 0; +inf counts as the largest finite float
    tok, lp = orc.topk_logprobs(
        np.array([[np.nan, 1.0, np.inf, -np.inf, np.inf]], np.float32), 5)
    assert tok[0].tolist() == [2, 4, 1, 0, 3]
    assert lp[0, 0] == lp[0, 1] and abs(lp[0, 0] + math.log(2.0)) < 1e-15
    assert abs(lp[0, 2] - ((1.0 - F32MAX) - math.log(2.0))) <= 1e-15 * F32MAX
    assert lp[0, 3] == -np.inf and lp[0, 4] == -np.inf
    # no finite entry: every log-probability is -inf, the smallest tokens come first
    tok, lp = orc.topk_logprobs(np.array([[np.nan, -np.inf, np.nan, -np.inf]], np.float32), 3)
    assert tok[0].tolist() == [0, 1, 2] and np.all(lp == -np.inf)
    # K = V: a permutation whose probabilities sum to 1
    row = np.random.default_rng(3).normal(0, 3, size=(1, 40)).astype(np.float32)
    tok, lp = orc.topk_logprobs(row, 40)
    assert sorted(tok[0].tolist()) == list(range(40))
    assert abs(math.fsum(np.exp(lp[0]).tolist()) - 1.0) < 1e-14
    assert np.all(np.diff(lp[0]) <= 0)


def pin_topk_vs_library(orc):
    """Random rows (on a coarse grid, so that ties occur) against scipy's log_softmax in
    fp64 and a stable descending argsort (ties keep the smaller index)."""
    from scipy.special import log_softmax
    rng = np.random.default_rng(17)
    for V, K in ((1000, 8), (37, 37), (5000, 1), (300, 64)):
        x = (np.round(rng.normal(0, 2, size=(6, V)) * 4) / 4).astype(np.float32)
        tok, lp = orc.topk_logprobs(x, K)
        ref = log_softmax(x.astype(np.float64), axis=-1)
        for r in range(x.shape[0]):
            order = np.argsort(-x[r].astype(np.float64), kind="stable")[:K]
            assert tok[r].tolist() == order.tolist()
            assert np.allclose(lp[r], ref[r, order], rtol=0, atol=1e-12)


def _draft_rows():
    """Rows of the worked best-first example (V = 3, K = 2)."""
    ninf = -np.inf
    return np.array([[[0.0, -0.375, ninf],    # node 0 (root)
                      [-2.0, ninf, 0.0],      # node 1
                      [0.0, 0.0, ninf],       # node 2
                      [-1.0, 0.0, 1.0],       # node 3
                      [-9.0, -9.0, -9.0],     # node 4
                      [np.nan] * 3]],         # node 5 completes the tree: never read
                    np.float32)


def pin_draft_tree_worked_example(orc):
    """Global best-first expansion worked by hand (ADR-037 row E4a: a grandchild of A
    is admitted before a sibling of A when its cumulative log-probability is higher).

    Root offers token 0 (c1 = -log(1 + e^-0.375)) and token 1 (c3 = -0.375 + c1).  Node 1
    (token 0) offers token 2 at c1 - log(1 + e^-2), which beats the root's token 1, so
    node 2 is that grandchild.  Node 2 offers tokens 0 and 1 at c2 - log 2 (a tie).
    Node 3 is the root's token 1; it offers token 2 at c3 + 1 - log(e^-1 + 1 + e), which
    beats the tie, so node 4 is that; node 5 is the first-offered side of the tie."""
    rows = _draft_rows()
    par, tok, cum = orc.draft_tree(rows, np.array([77], np.int32), K=2, max_levels=4)
    assert par[0].tolist() == [-1, 0, 1, 0, 3, 2]
    assert tok[0].tolist() == [77, 0, 2, 1, 2, 0]
    c1 = -math.log1p(math.exp(-0.375))
    c2 = c1 - math.log1p(math.exp(-2.0))
    c3 = -0.375 + c1
    c4 = c3 + 1.0 - math.log(math.exp(-1.0) + 1.0 + math.exp(1.0))
    c5 = c2 - math.log(2.0)
    assert np.allclose(cum[0], [0.0, c1, c2, c3, c4, c5], rtol=0, atol=1e-14)
    # a level limit of 2: only the root offers candidates, three nodes at most
    par, tok, _ = orc.draft_tree(rows[:, :3], np.array([5], np.int32), K=2, max_levels=2)
    assert par[0].tolist() == [-1, 0, 0] and tok[0].tolist() == [5, 0, 1]
    for T, K, lv in ((4, 2, 2), (2, 4, 3), (2, 1, 1)):
        try:
            orc.draft_tree(np.zeros((1, T, 3), np.float32), np.zeros(1, np.int32), K=K,
                           max_levels=lv)
        except ValueError:
            continue
        raise AssertionError(f"T={T} K={K} max_levels={lv} must be refused")


def pin_draft_tree_bruteforce(orc):
    """With every drafter row the same the candidate tree is fixed, and best-first
    admits exactly its T - 1 best non-root nodes (brute force over all rank sequences
    with scipy's log-softmax); admission order never raises the cumulative log-prob."""
    from itertools import product
    from scipy.special import log_softmax
    rng = np.random.default_rng(23)
    V, K, levels = 6, 3, 4
    for trial in range(4):
        row = rng.normal(0, 1.5, size=V).astype(np.float32)
        lp = log_softmax(row.astype(np.float64))
        order = np.argsort(-row.astype(np.float64), kind="stable")[:K]
        paths = []
        for d in range(1, levels):
            for seq in product(range(K), repeat=d):
                paths.append((sum(lp[order[r]] for r in seq),
                              tuple(int(order[r]) for r in seq)))
        paths.sort(key=lambda t: -t[0])
        # a budget whose cut is not inside a group of (near-)equal sums
        cuts = [n for n in range(4, len(paths)) if paths[n - 1][0] - paths[n][0] > 1e-9]
        n = cuts[trial]
        T = n + 1
        rows = np.tile(row[None, None], (1, T, 1))
        par, tok, cum = orc.draft_tree(rows, np.array([9], np.int32), K=K, max_levels=levels)
        got = set()
        for i in range(1, T):
            seq, j = [], i
            while j > 0:
                seq.append(int(tok[0, j]))
                j = par[0, j]
            got.add(tuple(reversed(seq)))
        assert got == {p for _, p in paths[:n]}
        assert np.all(np.diff(cum[0, 1:]) <= 0)
        sums = {p: c for c, p in paths}
        for i in range(1, T):
            seq, j = [], i
            while j > 0:
                seq.append(int(tok[0, j]))
                j = par[0, j]
            assert abs(cum[0, i] - sums[tuple(reversed(seq))]) < 1e-12


def pin_draft_tree_structure(orc):
    """K = 1 gives a chain of each row's argmax (numpy); a two-level limit gives a star
    of the root row's top-K (stable argsort); T = 1 reads no row; every child comes
    from the top-K of the row of its parent's admission index, and keys never rise."""
    rng = np.random.default_rng(31)
    rows = rng.normal(0, 2, size=(2, 12, 50)).astype(np.float32)
    roots = np.array([4, 8], np.int32)
    par, tok, _ = orc.draft_tree(rows, roots, K=1, max_levels=12)
    for b in range(2):
        assert par[b].tolist() == [-1] + list(range(11))
        assert tok[b, 1:].tolist() == [int(np.argmax(rows[b, i])) for i in range(11)]
    par, tok, _ = orc.draft_tree(rows[:, :5], roots, K=4, max_levels=2)
    for b in range(2):
        assert par[b].tolist() == [-1, 0, 0, 0, 0]
        assert tok[b, 1:].tolist() == np.argsort(-rows[b, 0], kind="stable")[:4].tolist()
    par, tok, cum = orc.draft_tree(np.full((2, 1, 50), np.nan, np.float32), roots, K=3,
                                   max_levels=3)
    assert par.tolist() == [[-1], [-1]] and tok[:, 0].tolist() == [4, 8] and np.all(cum == 0)
    par, tok, cum = orc.draft_tree(rows, roots, K=5, max_levels=4)
    for b in range(2):
        assert par[b, 0] == -1 and tok[b, 0] == roots[b] and cum[b, 0] == 0.0
        assert np.all(np.diff(cum[b, 1:]) <= 0)
        depth = [0] * 12
        for c in range(1, 12):
            p = int(par[b, c])
            assert 0 <= p < c
            depth[c] = depth[p] + 1
            assert depth[c] <= 3
            top = np.argsort(-rows[b, p], kind="stable")[:5].tolist()
            assert int(tok[b, c]) in top
        # no token offered twice by one parent
        pairs = [(int(par[b, c]), int(tok[b, c])) for c in range(1, 12)]
        assert len(set(pairs)) == len(pairs)


# ============================================= write-before-accept (in-cache) variant
def gather_at(cache: O.Cache, b: int, h: int, pos, which: str = "k") -> np.ndarray:
    """Rows at the given positions of sequence b, kv head h, float64 [n, D] (numpy
    indexing over the block table, independent of the oracle's addressing)."""
    pool = cache.k if which == "k" else cache.v
    D = cache.row_stride
    pool4 = pool.reshape(pool.shape[0], -1, cache.block_size, D)
    pos = np.asarray(pos)
    rows = pool4[cache.table[b, pos // cache.block_size], h, pos % cache.block_size, :]
    return as_f64(rows, cache.dtype)


def pin_incache_append_and_attention(orc):
    """Append puts tree row i at position P + i and touches nothing else; attention over
    the cache-resident tree equals attention over the tree buffers (bit for bit) and the
    fp64 SDPA reference; sequences that cannot be appended are refused whole."""
    inp = small_inputs("batched8k", 51, B=3, prefix=(10, 77), T=12, Hq=4, Hkv=2, D=64)
    w = inp.w
    cache = _cache(inp)
    k0, v0 = cache.k.copy(), cache.v.copy()
    P = to_np(inp.prefix_len)
    kt, vt, q = to_np(inp.k_tree), to_np(inp.v_tree), to_np(inp.q)
    err = orc.kv_append(kt, vt, None, cache, P, inp.max_prefix_len)
    assert np.all(err == 0)
    changed = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            pos = int(P[b]) + np.arange(w.T)
            assert np.array_equal(gather_at(cache, b, h, pos, "k"), as_f64(kt[b, h], cache.dtype))
            assert np.array_equal(gather_at(cache, b, h, pos, "v"), as_f64(vt[b, h], cache.dtype))
            changed += w.T
    D = w.D
    diff_rows = np.any(cache.k.reshape(-1, D) != k0.reshape(-1, D), axis=1).sum()
    assert diff_rows <= changed and np.array_equal(
        cache.k.reshape(-1, D)[np.all(cache.k.reshape(-1, D) == k0.reshape(-1, D), axis=1)],
        k0.reshape(-1, D)[np.all(cache.k.reshape(-1, D) == k0.reshape(-1, D), axis=1)])
    mask, _, _ = orc.build_tree_mask(to_np(inp.parents))
    a = orc.tree_verify_attention(q, None, None, cache, P, inp.max_prefix_len, mask, inp.scale)
    c = run_attention(orc, inp)
    assert np.array_equal(a, c)
    for b in range(w.B):
        kp = np.stack([gather_prefix(cache, b, h, int(P[b]), "k") for h in range(w.Hkv)])
        vp = np.stack([gather_prefix(cache, b, h, int(P[b]), "v") for h in range(w.Hkv)])
        pos = int(P[b]) + np.arange(w.T)
        kk = np.stack([gather_at(cache, b, h, pos, "k") for h in range(w.Hkv)])
        vv = np.stack([gather_at(cache, b, h, pos, "v") for h in range(w.Hkv)])
        ref = sdpa_reference(as_f64(q[b], cache.dtype), kp, vp, kk, vv,
                             closure_mask(to_np(inp.parents)[b]), inp.scale)
        np.testing.assert_allclose(a[b].astype(np.float64), ref, rtol=2e-6, atol=2e-6)
    # refusals: a sequence already invalid, a prefix past max_prefix_len, a block entry
    # out of range inside [P, P + T); each leaves its sequence untouched
    cache = _cache(inp)
    table = cache.table.copy()
    blk = (int(P[2]) + 3) // cache.block_size
    table[2, blk] = -1
    cache = O.Cache(**{**cache.__dict__, "table": table})
    Pbad = P.copy()
    Pbad[1] = inp.max_prefix_len + 1
    k0 = cache.k.copy()
    err = orc.kv_append(kt, vt, np.array([5, 0, 0], np.int32), cache, Pbad, inp.max_prefix_len)
    assert err.tolist() == [5, 3, 3] and np.array_equal(cache.k, k0)


def pin_incache_compaction(orc):
    """Append then compaction leaves the cache rows [0, P + L) and the new prefix lengths
    of delayed write-through, each row P + j holding tree row nodes[j] (numpy); a path
    whose rows overlap their destinations, L = 0 and invalid requests behave as stated."""
    inp = small_inputs("batched8k", 52, B=4, prefix=(20, 90), T=16, Hq=4, Hkv=2, D=32,
                       draft_p=0.9)
    w = inp.w
    P = to_np(inp.prefix_len)
    kt, vt = to_np(inp.k_tree), to_np(inp.v_tree)
    parents = to_np(inp.parents)
    _, _, err = orc.build_tree_mask(parents)
    _, L, nodes, _ = orc.accept_longest_path(to_np(inp.logits), to_np(inp.draft), parents, err)
    assert L.max() > 2
    ca = _cache(inp)
    orc.kv_append(kt, vt, err, ca, P, inp.max_prefix_len)
    npl_a = orc.kv_compact(L, nodes, err, ca, P, inp.max_prefix_len, w.Hkv, w.T, w.D)
    cb = _cache(inp)
    npl_b = orc.kv_commit(kt, vt, L, nodes, err, cb, P, inp.max_prefix_len)
    assert np.array_equal(npl_a, npl_b) and np.array_equal(npl_a, P + L)
    for b in range(w.B):
        for h in range(w.Hkv):
            pos = np.arange(int(P[b] + L[b]))
            for which, src in (("k", kt), ("v", vt)):
                ra, rb = gather_at(ca, b, h, pos, which), gather_at(cb, b, h, pos, which)
                assert np.array_equal(ra, rb)
                for j in range(int(L[b])):
                    assert np.array_equal(ra[P[b] + j], as_f64(src[b, h, nodes[b, j]], ca.dtype))
    # a path whose sources are later destinations: nodes [0, 2, 3]
    cc = _cache(inp)
    orc.kv_append(kt, vt, None, cc, P, inp.max_prefix_len)
    before = [gather_at(cc, 0, h, int(P[0]) + np.arange(w.T), "k") for h in range(w.Hkv)]
    Lx = np.array([3, 0, 2, 2], np.int32)
    nx = np.zeros((w.B, w.T), np.int32)
    nx[0, :3] = [0, 2, 3]
    nx[2, :2] = [0, w.T]            # a node index out of range: refused
    nx[3, :2] = [0, 1]
    ex = np.array([0, 0, 0, 4], np.int32)       # sequence 3 invalid
    snap = [cc.k.copy(), cc.v.copy()]
    npl = orc.kv_compact(Lx, nx, ex, cc, P, inp.max_prefix_len, w.Hkv, w.T, w.D)
    assert npl.tolist() == [P[0] + 3, P[1], P[2], P[3]]
    for h in range(w.Hkv):
        after = gather_at(cc, 0, h, int(P[0]) + np.arange(w.T), "k")
        assert np.array_equal(after[:3], before[h][[0, 2, 3]])
        assert np.array_equal(after[3:], before[h][3:])
    for b in (1, 2, 3):
        for h in range(w.Hkv):
            pos = np.arange(int(P[b]) + w.T)
            cc_only = O.Cache(**{**cc.__dict__, "k": snap[0], "v": snap[1]})
            assert np.array_equal(gather_at(cc, b, h, pos, "k"), gather_at(cc_only, b, h, pos, "k"))

ALL_PINS = [
    pin_mask_worked_example, pin_mask_closed_forms, pin_mask_bruteforce, pin_mask_invalid,
    pin_attn_decode_T1, pin_attn_chain_causal, pin_attn_tree_vs_sdpa, pin_attn_prefix_zero,
    pin_attn_closed_forms, pin_attn_paged_equals_contiguous, pin_attn_bad_block_entry,
    pin_attn_chain_equals_serial,
    pin_argmax_numpy, pin_argmax_special_values, pin_argmax_planted,
    pin_accept_bruteforce, pin_accept_edge_cases, pin_accept_expected_tokens_golden,
    pin_accept_expected_tokens_closed_form,
    pin_sampled_worked_examples, pin_sampled_expected_tokens_golden, pin_sampled_preserves_target,
    pin_sampled_low_temperature_is_greedy, pin_sampled_invariants,
    pin_rope_worked_examples, pin_rope_relative_position, pin_rope_pairs_and_tree,
    pin_rope_bf16_rounding,
    pin_topk_worked_examples, pin_topk_vs_library, pin_draft_tree_worked_example,
    pin_draft_tree_bruteforce, pin_draft_tree_structure,
    pin_incache_append_and_attention, pin_incache_compaction,
    pin_commit_invariants, pin_commit_single_root, pin_commit_refusals,
    pin_commit_chain_equals_serial,
]
