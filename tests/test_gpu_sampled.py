"""GPU parity of sampled acceptance: sv_accept_sampled through the C ABI against the
oracle on the same seeded inputs and uniforms.

Accepted lengths, nodes and tokens must be identical, except in a sequence whose
oracle path holds a decision within 5e-5 (a probability) of its boundary: the GPU
decides in fp32 what the oracle decides in fp64, so there either outcome is a correct
result of the rule, and the GPU's must pass the fp64 replay in sampled_check.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import tree_masked_verify_amd as sv
from _support import oracle_cache, to_np
from sampled_check import compare_sampled
from tree_masked_verify_amd import workloads as wl
from tree_masked_verify_amd.step import VerifyStep

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


def gpu_sampled(lg, drf, par, ua, us, tau, tree_err=None):
    """lg, drf, par: device tensors; ua, us: host float32 arrays."""
    B, T = par.shape
    V = lg.shape[-1]
    L = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nodes = torch.full((B, T), -7, dtype=torch.int32, device=DEV)
    toks = torch.full((B, T), -7, dtype=torch.int32, device=DEV)
    ws = sv.workspace(sv.sv_accept_sampled_workspace_size(B, T, V), DEV)
    sv.sv_accept_sampled(lg, drf, par, tree_err, _dev(ua), _dev(us), tau, L, nodes, toks, ws)
    torch.cuda.synchronize()
    return to_np(L), to_np(nodes), to_np(toks)


def run(orc, lg, drf, par, tau, seed, tree_err=None, uniforms=None, label=""):
    B, T = par.shape
    ua, us = wl.make_uniforms(B, T, seed) if uniforms is None else uniforms
    _say(f"[case] sampled {label} B={B} T={T} V={lg.shape[-1]} tau={tau} seed={seed}")
    g = gpu_sampled(lg, drf, par, ua, us, tau, None if tree_err is None else _dev(tree_err))
    hl, hd, hp = to_np(lg), to_np(drf), to_np(par)
    o = orc.accept_sampled(hl, hd, hp, ua, us, tau, tree_err)
    n_amb = compare_sampled(g, o, hl, hd, hp, ua, us, tau)
    _say(f"       accepted {list(g[0][:8])}, mean L {g[0].mean():.2f}, "
         f"{n_amb} sequence(s) decided within tolerance of a boundary")
    return g, o


# --------------------------------------------------------------- the workload shapes
@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("tiny", 2), ("parity512", 0),
                                       ("parity512", 1), ("parity512", 2), ("chain2k", 0),
                                       ("chain2k", 1)])
def test_small_workloads(orc, name, seed):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, seed=seed, device=DEV)
    run(orc, inp.logits, inp.draft, inp.parents, w.temperature, seed, label=name)


@pytest.mark.parametrize("name", ["batched8k", "long32k"])
def test_full_size_workloads(orc, name):
    """The two large configurations at full size (B x T rows of 151936 logits)."""
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, seed=3, device=DEV)
    g, _ = run(orc, inp.logits, inp.draft, inp.parents, w.temperature, 3, label=name)
    assert g[0].min() >= 1 and g[0].max() > 1          # valid trees; some drafts accepted


@pytest.mark.parametrize("tau", [0.05, 0.3, 1.0, 4.0])
def test_temperatures(orc, tau):
    w = wl.WORKLOADS["parity512"]
    inp = wl.make_inputs(wl.scaled(w, B=8), seed=11, device=DEV)
    run(orc, inp.logits, inp.draft, inp.parents, tau, 11, label=f"parity512 x8")


def test_many_copies_of_one_tree(orc):
    """4096 sequences with the same small tree and rows, different uniforms: every
    outcome of the rule appears, each must be the oracle's."""
    rng = np.random.Generator(np.random.PCG64(5))
    par1 = np.array([-1, 0, 0, 0, 1, 1, 3, 6], np.int32)
    drf1 = np.array([0, 2, 2, 4, 0, 3, 1, 6], np.int32)
    T, V, n = len(par1), 7, 4096
    rows = rng.normal(0.0, 1.5, size=(T, V)).astype(np.float32)
    lg = _dev(np.tile(rows[None], (n, 1, 1)))
    g, _ = run(orc, lg, _dev(np.tile(drf1[None], (n, 1))), _dev(np.tile(par1[None], (n, 1))), 0.8,
               21, label="copies")
    assert len(set(g[0].tolist())) >= 3 and len(set(g[2][:, 0].tolist())) >= 5


def test_odd_vocabulary_and_chunks(orc):
    """V odd (rows not 16-byte aligned), over several 16384-element chunks, and rows of
    more than 16 chunks (the walk merges a row's chunk pairs sixteen at a time): 524288 =
    32 chunks, 600001 = 37."""
    for V in (70001, 131073, 5, 524288, 600001):
        w = wl.scaled(wl.WORKLOADS["parity512"], V=V, B=4)
        inp = wl.make_inputs(w, seed=V % 97, device=DEV)
        run(orc, inp.logits, inp.draft, inp.parents, 0.3, V % 97, label=f"V={V}")


def test_special_values(orc):
    """Rows with no finite logit, NaN and +inf entries, draft tokens outside the
    vocabulary, repeated sibling tokens, a single node, invalid trees."""
    rng = np.random.Generator(np.random.PCG64(8))
    T, V, B = 8, 1000, 6
    par = np.array([[-1, 0, 0, 0, 1, 1, 2, 4]] * B, np.int32)
    lg = (rng.normal(0, 2.0, size=(B, T, V)) ).astype(np.float32)
    drf = rng.integers(0, V, size=(B, T)).astype(np.int32)
    top = lg.argmax(-1)
    for b in range(B):
        for c in range(1, T):
            drf[b, c] = top[b, par[b, c]]                # proposals that are likely accepted
    lg[0, 0, :] = -np.inf                                # root row without a finite entry
    lg[1, 0, ::3] = np.nan                               # NaN entries have probability 0
    lg[2, 0, 17] = np.inf                                # +inf dominates
    drf[2, 1] = 17
    drf[3, 1] = -1                                       # outside the vocabulary
    drf[3, 2] = V + 5
    drf[4, 2] = drf[4, 1]                                # repeated sibling token
    lg[5, :, :] = -np.inf                                # every row empty
    lg[5, :, 3] = 0.0                                    # except token 3: probability 1
    drf[5, :] = 3
    run(orc, _dev(lg), _dev(drf), _dev(par), 0.5, 2, label="special")
    # u = 0 accepts any proposal with probability > 0; u just below 1 rejects most
    ua = np.zeros((B, T), np.float32)
    us = np.full((B, T), np.nextafter(np.float32(1), np.float32(0)), np.float32)
    run(orc, _dev(lg), _dev(drf), _dev(par), 0.5, 2, uniforms=(ua, us), label="u extremes")
    run(orc, _dev(lg), _dev(drf), _dev(par), 0.5, 2, uniforms=(us.copy(), ua.copy()),
        label="u extremes swapped")
    # T = 1: the root alone draws the emitted token
    run(orc, _dev(lg[:, :1]), _dev(drf[:, :1]), _dev(par[:, :1]), 0.5, 4, label="T=1")
    # invalid trees: tree_err given, or a malformed parent array
    err = np.array([0, 3, 0, 0, 1, 0], np.int32)
    bad = par.copy()
    bad[2, 5] = 6
    g, _ = run(orc, _dev(lg), _dev(drf), _dev(bad), 0.5, 6, tree_err=err, label="invalid")
    assert list(g[0][[1, 2, 4]]) == [0, 0, 0] and np.all(g[1][[1, 2, 4]] == -1)


def test_then_commit(orc):
    """Sampled acceptance feeds the delayed write-through exactly as greedy does."""
    w = wl.WORKLOADS["parity512"]
    inp = wl.make_inputs(wl.scaled(w, B=4), seed=13, device=DEV)
    cache = oracle_cache(inp)
    h = dict(parents=to_np(inp.parents), k_tree=to_np(inp.k_tree), v_tree=to_np(inp.v_tree),
             prefix=to_np(inp.prefix_len), logits=to_np(inp.logits), draft=to_np(inp.draft))
    ua, us = wl.make_uniforms(4, w.T, 13)
    st = VerifyStep.from_inputs(inp)
    st.build_mask()
    st.accept_sampled(_dev(ua), _dev(us), w.temperature)
    st.commit()
    torch.cuda.synchronize()
    _, _, err = orc.build_tree_mask(h["parents"])
    L, nodes, toks = orc.accept_sampled(h["logits"], h["draft"], h["parents"], ua, us,
                                        w.temperature, err)
    assert np.array_equal(to_np(st.accepted_len), L) and np.array_equal(to_np(st.accepted_nodes), nodes)
    assert np.array_equal(to_np(st.out_tokens), toks)
    npl = orc.kv_commit(h["k_tree"], h["v_tree"], L, nodes, err, cache, h["prefix"],
                        inp.max_prefix_len)
    assert np.array_equal(to_np(st.new_prefix_len), npl)
    assert np.array_equal(to_np(inp.k_pool), cache.k) and np.array_equal(to_np(inp.v_pool), cache.v)
