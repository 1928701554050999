"""GPU edge cases against the oracle: malformed trees, ties / NaN / infinities in the
logits, out-of-range block-table entries, determinism across runs and across
synchronised vs back-to-back dispatch, and a chain verified at once vs node by node."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from _support import to_np
from parity import ATOL, attention_error, compare, gpu_step, host_copy, oracle_step
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


def _check(orc, inp):
    h = host_copy(inp)
    g = gpu_step(inp)
    o = oracle_step(orc, inp, h)
    compare(g, o)
    return g, o


def test_invalid_trees(orc):
    _say("[case] invalid trees")
    w = wl.scaled(wl.WORKLOADS["parity512"], name="bad", B=4, V=777)
    inp = wl.make_inputs(w, seed=21, device=DEV)
    inp.parents[1, 5] = 6          # parent after child
    inp.parents[2, 0] = 0          # root with a parent
    inp.parents[3, 3] = -1         # a second root
    g, o = _check(orc, inp)
    assert list(g["tree_err"]) == [0, O.TREE_BAD_PARENT, O.TREE_BAD_ROOT, O.TREE_BAD_PARENT]
    assert list(g["L"][1:]) == [0, 0, 0]


def test_logit_ties_nan_inf(orc):
    _say("[case] logits with ties, NaN, infinities")
    w = wl.scaled(wl.WORKLOADS["parity512"], name="nan", B=2, V=40000)
    inp = wl.make_inputs(w, seed=22, device=DEV)
    lg = inp.logits
    lg[0, 1, :] = 0.5                               # all tied -> index 0
    lg[0, 2, 17] = float("nan")
    lg[0, 2, 39999] = float("inf")
    lg[0, 2, 123] = float("inf")                    # first +inf wins
    lg[0, 3, :] = float("nan")                      # all NaN -> 0
    lg[0, 4, :] = float("-inf")                     # all -inf -> 0
    lg[0, 5, ::7] = float("nan")
    row = lg[1, 6]
    top = int(torch.argmax(torch.nan_to_num(row, nan=-1e30)))
    row[top + 1:] = torch.where(torch.arange(row.numel() - top - 1, device=DEV) % 5 == 0,
                                row[top], row[top + 1:])   # later copies of the maximum
    lg[1, 7, 1000:1016] = 1e30                      # a tie inside one 16-byte vector run
    _check(orc, inp)


def test_bad_block_entries(orc):
    _say("[case] out-of-range block-table entries")
    w = wl.scaled(wl.WORKLOADS["batched8k"], name="badblk", B=3, prefix=(200, 400), V=999)
    inp = wl.make_inputs(w, seed=23, device=DEV)
    P = to_np(inp.prefix_len)
    inp.block_table[0, 3] = -1                      # prefix rows 48..63 of sequence 0 dropped
    inp.block_table[1, 1] = inp.num_blocks + 7      # prefix rows 16..31 of sequence 1 dropped
    inp.block_table[2, int(P[2]) // 16] = -5        # the commit target of sequence 2: refused
    g, o = _check(orc, inp)
    assert g["npl"][2] == P[2]


def test_determinism_and_serial_dispatch(orc):
    _say("[case] determinism")
    w = wl.scaled(wl.WORKLOADS["long32k"], name="det", B=2, prefix=(2000, 3000), V=3000)
    inp = wl.make_inputs(w, seed=24, device=DEV)
    st = VerifyStep.from_inputs(inp)
    outs = []
    for rep in range(5):
        if rep % 2 == 0:
            st.run()
        else:  # serial control arm: wait for each call before the next
            st.build_mask(); torch.cuda.synchronize()
            st.attention(); torch.cuda.synchronize()
            st.accept(); torch.cuda.synchronize()
            st.commit()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (st.mask, st.out, st.argmax, st.accepted_len,
                                          st.accepted_nodes, st.out_tokens, st.new_prefix_len)])
    for rep in outs[1:]:
        for a, b in zip(outs[0], rep):
            assert torch.equal(a, b)


def test_chain_at_once_equals_node_by_node(orc):
    """A chain verified as one tree vs T single-node verifies with a commit after each:
    the same tokens and the same cache bytes; attention rows agree within tolerance."""
    _say("[case] chain vs serial single-node verifies")
    w = wl.WORKLOADS["chain2k"]
    inp = wl.make_inputs(w, seed=25, device=DEV)
    kp0, vp0 = inp.k_pool.clone(), inp.v_pool.clone()
    chain = VerifyStep.from_inputs(inp)
    chain.run()
    torch.cuda.synchronize()
    L = int(chain.accepted_len[0])
    _say(f"       chain accepted {L}")

    # node-by-node: fresh copy of the cache, one-node trees, commit each root
    kp, vp = kp0.clone(), vp0.clone()
    prefix = inp.prefix_len.clone()
    outs, toks = [], []
    for i in range(w.T):
        sl = lambda t: t[:, :, i:i + 1].contiguous()
        one = VerifyStep(sl(inp.q), sl(inp.k_tree), sl(inp.v_tree), kp, vp, inp.block_table,
                         prefix, int(inp.max_prefix_len) + i,
                         torch.full((1, 1), -1, dtype=torch.int32, device=DEV),
                         inp.logits[:, i:i + 1].contiguous(), inp.draft[:, i:i + 1].contiguous(),
                         inp.scale, new_prefix_len=prefix)
        one.run()
        torch.cuda.synchronize()
        outs.append(one.out[0, 0].clone())
        toks.append(int(one.out_tokens[0, 0]))
    # the chain's emitted tokens are the argmax of its rows along the accepted path
    assert toks[:L] == [int(x) for x in chain.out_tokens[0, :L]]
    # the chain committed L rows; the serial path committed all T: compare the first L
    P0 = int(inp.max_prefix_len)
    cap = inp.k_pool.shape[2]
    for j in range(L):
        assert torch.equal(inp.k_pool[0, :, P0 + j], kp[0, :, P0 + j])
        assert torch.equal(inp.v_pool[0, :, P0 + j], vp[0, :, P0 + j])
    # everything outside the committed rows is untouched in both
    assert torch.equal(inp.k_pool[0, :, :P0], kp0[0, :, :P0])
    assert torch.equal(inp.k_pool[0, :, P0 + L:cap], kp0[0, :, P0 + L:cap])
    for i in range(w.T):
        mx, _ = attention_error(to_np(outs[i]), to_np(chain.out[0, i]))
        assert mx <= ATOL, (i, mx)
