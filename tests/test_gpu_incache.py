"""GPU parity of the write-before-accept variant through the C ABI: sv_kv_append, the
attention over the cache-resident tree (NULL tree buffers) and sv_kv_compact.

Against the oracle on the same seeded inputs: tree status, accepted paths, new prefix
lengths and both cache pools bit for bit, attention within the step tolerance.  Against
the delayed write-through path on the GPU: attention outputs bit for bit (the same
kernels read the same bytes) and the same cache rows [0, P + L).
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from _support import oracle_cache, to_np
from parity import compare, host_copy, oracle_in_cache, sample_rows, step_result
from tree_masked_verify_amd import make_cache, sv_kv_append, sv_kv_compact
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


def committed_rows(inp, pool, P, L, b):
    """Rows [0, P + L) of sequence b (all kv heads) from a host pool, via the table."""
    table = to_np(inp.block_table)
    bs = inp.block_size
    pos = np.arange(int(P[b] + L[b]))
    p4 = pool.reshape(pool.shape[0], inp.w.Hkv, bs, inp.w.D)
    return p4[table[b, pos // bs], :, pos % bs, :]


def run_case(orc, w, seed, rows=None, num_splits=0, also_write_through=True):
    _say(f"[case] in-cache {w.name} seed={seed} B={w.B} T={w.T} D={w.D} splits={num_splits}")
    inp = wl.make_inputs(w, seed=seed, device=DEV)
    h = host_copy(inp)
    st = VerifyStep.from_inputs(inp, num_splits=num_splits)
    st.run_in_cache()
    g = step_result(st, inp)
    o = oracle_in_cache(orc, inp, h, rows=rows)
    err = compare(g, o, rows=rows)
    _say(f"       attention max-abs {err['max_abs']:.3e}, accepted {list(g['L'][:8])}")
    if also_write_through:
        inp2 = wl.make_inputs(w, seed=seed, device=DEV)
        st2 = VerifyStep.from_inputs(inp2, num_splits=num_splits)
        st2.run()
        g2 = step_result(st2, inp2)
        assert np.array_equal(g["out"], g2["out"]), "attention differs from the buffer path"
        assert np.array_equal(g["L"], g2["L"]) and np.array_equal(g["npl"], g2["npl"])
        P = h["prefix"]
        for b in range(w.B):
            for a, c in ((g["k_pool"], g2["k_pool"]), (g["v_pool"], g2["v_pool"])):
                assert np.array_equal(committed_rows(inp, a, P, g["L"], b),
                                      committed_rows(inp, c, P, g["L"], b))
    return inp, g, o


@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("parity512", 0),
                                       ("parity512", 1), ("chain2k", 0)])
def test_small_workloads(orc, name, seed):
    run_case(orc, wl.WORKLOADS[name], seed)


@pytest.mark.parametrize("name", ["batched8k", "long32k", "long32k_d128"])
def test_scaled_paged(orc, name):
    """The paged shapes (shuffled blocks) at reduced batch and prefix."""
    w = wl.scaled(wl.WORKLOADS[name], B=3, prefix=(100, 700))
    run_case(orc, w, 7)
    run_case(orc, w, 8, num_splits=3)


def test_long32k_full_size(orc):
    """The 32K shape at full size: sampled attention rows against the oracle, every pool
    byte after the compaction, and the buffer path's outputs and committed rows."""
    w = wl.WORKLOADS["long32k"]
    run_case(orc, w, 5, rows=sample_rows(w, 24, 5))


def test_refused_sequence(orc):
    """A block-table entry out of range inside [P, P + T): the append refuses that
    sequence (status 3), which then accepts and compacts nothing; the others proceed."""
    w = wl.scaled(wl.WORKLOADS["batched8k"], B=3, prefix=(200, 300), T=16)
    inp = wl.make_inputs(w, seed=9, device=DEV)
    P = to_np(inp.prefix_len)
    blk = (int(P[1]) + 5) // inp.block_size
    inp.block_table[1, blk] = -1
    h = host_copy(inp)
    st = VerifyStep.from_inputs(inp)
    st.run_in_cache()
    g = step_result(st, inp)
    o = oracle_in_cache(orc, inp, h)
    assert g["tree_err"].tolist() == [0, 3, 0] and o["tree_err"].tolist() == [0, 3, 0]
    assert g["L"][1] == 0 and g["npl"][1] == P[1]
    # the refused sequence's attention read stand-in rows: compare the others only
    keep = [0, 2]
    g["out"], o["out"] = g["out"][keep], o["out"][keep]
    compare(g, o)


def test_compact_direct(orc):
    """sv_kv_compact on hand-made paths: one whose sources are later destinations
    (nodes 0, 2, 3), the identity, L = 0, a node out of range and an invalid tree."""
    w = wl.scaled(wl.WORKLOADS["batched8k"], B=6, prefix=(50, 400), T=16, D=256)
    inp = wl.make_inputs(w, seed=11, device=DEV)
    cache = make_cache(inp.k_pool, inp.v_pool, inp.block_table)
    err = torch.zeros((w.B,), dtype=torch.int32, device=DEV)
    sv_kv_append(inp.k_tree, inp.v_tree, err, cache, inp.prefix_len, inp.max_prefix_len)
    torch.cuda.synchronize()
    hc = oracle_cache(inp)
    L = np.array([3, 4, 0, 2, 5, 16], np.int32)
    nodes = np.zeros((w.B, w.T), np.int32)
    nodes[0, :3] = [0, 2, 3]
    nodes[1, :4] = [0, 1, 2, 3]
    nodes[3, :2] = [0, w.T]                       # out of range: refused
    nodes[4, :5] = [0, 1, 5, 9, 15]
    nodes[5, :] = np.arange(w.T)[::-1]            # every row moves (not a tree path)
    terr = np.array([0, 0, 0, 0, 2, 0], np.int32)  # sequence 4: invalid tree
    dev = lambda a: torch.from_numpy(a).to(DEV)
    npl = torch.full((w.B,), -7, dtype=torch.int32, device=DEV)
    sv_kv_compact(dev(L), dev(nodes), dev(terr), cache, inp.prefix_len, inp.max_prefix_len, npl,
                  w.Hkv, w.D)
    torch.cuda.synchronize()
    onpl = orc.kv_compact(L, nodes, terr, hc, to_np(inp.prefix_len), inp.max_prefix_len, w.Hkv,
                          w.T, w.D)
    assert np.array_equal(to_np(npl), onpl)
    assert np.array_equal(to_np(inp.k_pool), hc.k) and np.array_equal(to_np(inp.v_pool), hc.v)
