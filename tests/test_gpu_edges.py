"""GPU edge cases against the oracle: malformed trees, ties / NaN / infinities in the
logits, out-of-range block-table entries, determinism across runs and across
synchronised vs back-to-back dispatch, and a chain verified at once vs node by node."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from _support import oracle_cache, to_np
from parity import ATOL, REL_RMS, attention_error, compare, gpu_step, host_copy, oracle_step
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
    # each single-node verify against the oracle, on the cache as it stood for that call:
    # rows P0 .. P0 + i - 1 committed by the calls before it (the final pools hold them;
    # rows from P0 + i on are not read)
    cache = oracle_cache(inp, k_pool=to_np(kp), v_pool=to_np(vp))
    one = np.ones((1, 1, 1), dtype=np.uint64)
    for i in range(w.T):
        sl = lambda t: to_np(t[:, :, i:i + 1].contiguous())
        ref = orc.tree_verify_attention(sl(inp.q), sl(inp.k_tree), sl(inp.v_tree), cache,
                                        np.array([P0 + i], dtype=np.int32), P0 + i, one,
                                        inp.scale)
        got = to_np(outs[i])
        assert np.all(np.isfinite(got))
        mx, rel = attention_error(got, ref[0, 0])
        assert mx <= ATOL and rel <= REL_RMS, (i, mx, rel)


def _poison_unattended(inp, value=float("nan")):
    """Fill every cache row no query attends to with `value`: rows at or past each
    sequence's prefix length inside its blocks, and two extra pool blocks that no
    block-table entry reaches (appended to both pools)."""
    P = to_np(inp.prefix_len)
    bs = inp.block_size
    tbl = to_np(inp.block_table)
    for pool in (inp.k_pool, inp.v_pool):
        for b in range(inp.w.B):
            for pos in range(int(P[b]), int((tbl[b] >= 0).sum()) * bs):
                blk = int(tbl[b, pos // bs])
                if 0 <= blk < pool.shape[0]:
                    pool[blk, :, pos % bs, :] = value
    extra = torch.full((2, *inp.k_pool.shape[1:]), value, dtype=inp.k_pool.dtype,
                       device=inp.k_pool.device)
    inp.k_pool = torch.cat([inp.k_pool, extra])
    inp.v_pool = torch.cat([inp.v_pool, extra])


@pytest.mark.parametrize("case", ["d256", "d128", "d512", "f32", "t1"])
def test_unattended_cache_rows_may_be_nonfinite(orc, case):
    """Cache rows that no query attends to may hold anything: with NaN (or infinity)
    there -- past every prefix (ragged tile ends), in blocks no table entry reaches, and
    behind an out-of-range table entry -- the outputs still equal the oracle's, which
    never reads those rows.  Covers the matrix-core kernels at head_dim 128, 256 and
    512 and the vector-ALU kernel (fp32, and single-node bf16)."""
    _say(f"[case] non-finite unattended rows {case}")
    base = wl.WORKLOADS["batched8k"]
    if case == "d512":
        w = wl.scaled(wl.WORKLOADS["chain2k"], name="nan512", B=3, Hq=16, Hkv=2, T=8,
                      tree="random", max_levels=4, max_children=3, block_size=16,
                      shuffled=True, prefix=(100, 700), V=999)
    elif case == "f32":
        w = wl.scaled(wl.WORKLOADS["tiny"], name="nanf32", B=3, Hq=4, Hkv=2, block_size=16,
                      shuffled=True, prefix=(40, 300), V=999)
    elif case == "t1":
        w = wl.scaled(base, name="nant1", B=3, T=1, tree="chain", Hq=8, Hkv=1,
                      prefix=(100, 700), V=999)
    else:
        w = wl.scaled(base, name=f"nan{case}", B=3, D=int(case[1:]), prefix=(100, 700),
                      V=999)
    inp = wl.make_inputs(w, seed=26, device=DEV, prefix_override=[333, 517, 130])
    _poison_unattended(inp, float("nan") if case != "d128" else float("inf"))
    inp.block_table[1, 2] = inp.num_blocks + 5   # keys 32..47 of sequence 1 left out
    _check(orc, inp)
    # the cache-resident variant reads the tree rows at P + j; the rows after them stay
    # poisoned
    if case in ("d256", "d512"):
        from parity import oracle_in_cache, step_result
        inp = wl.make_inputs(w, seed=27, device=DEV, prefix_override=[333, 517, 130])
        _poison_unattended(inp)
        h = host_copy(inp)
        st = VerifyStep.from_inputs(inp)
        st.run_in_cache()
        torch.cuda.synchronize()
        compare(step_result(st, inp), oracle_in_cache(orc, inp, h))


def test_attended_nan_stays_in_its_rows(orc):
    """A NaN in a value row that queries do attend to (prefix row 100 of sequence 1, kv
    head 0) makes exactly the outputs of that sequence's kv-head-0 query heads
    non-finite, as in the oracle; every other output matches the oracle."""
    _say("[case] attended NaN")
    w = wl.scaled(wl.WORKLOADS["batched8k"], name="nanvis", B=3, prefix=(300, 700), V=999)
    inp = wl.make_inputs(w, seed=28, device=DEV)
    blk = int(inp.block_table[1, 100 // inp.block_size])
    inp.v_pool[blk, 0, 100 % inp.block_size, 7] = float("nan")
    h = host_copy(inp)
    g = gpu_step(inp)
    o = oracle_step(orc, inp, h)
    G = w.Hq // w.Hkv
    bad = np.zeros(g["out"].shape, dtype=bool)
    bad[1, :, :G, :] = True
    assert not np.any(np.isfinite(g["out"][bad].reshape(-1, w.D)).all(axis=1))
    assert not np.any(np.isfinite(o["out"][bad].reshape(-1, w.D)).all(axis=1))
    mx, rel = attention_error(g["out"][~bad], o["out"][~bad])
    assert mx <= ATOL and rel <= REL_RMS, (mx, rel)
    for key in ("mask", "argmax", "L", "nodes", "toks", "npl"):
        assert np.array_equal(g[key], o[key]), key


@pytest.mark.parametrize("name", ["batched8k", "long32k"])
def test_determinism_soak_full_size(name):
    """Full-size soak: two input sets of one workload (different prefix lengths, so
    different chunk plans) verified alternately, 200 steps back to back on one stream
    sharing one attention workspace, then 10 steps with a synchronisation after every
    call.  Every step's outputs (mask, attention, argmax, acceptance, new prefix
    lengths) must equal, byte for byte, those of the first synchronised run of the same
    inputs; the checks stop at the first mismatch."""
    w = wl.WORKLOADS[name]
    _say(f"[case] determinism soak {name}")
    steps = [VerifyStep.from_inputs(wl.make_inputs(w, seed=s, device=DEV)) for s in (40, 41)]
    big = max(steps, key=lambda st: st.attn_ws.numel()).attn_ws
    for st in steps:
        st.attn_ws = big
    outs = lambda st: (st.mask, st.out, st.argmax, st.accepted_len, st.accepted_nodes,
                       st.out_tokens, st.new_prefix_len)
    ref = []
    for st in steps:
        st.run()
        torch.cuda.synchronize()
        ref.append([t.clone() for t in outs(st)])
    for chunk in range(10):                        # 10 x 20 back-to-back steps
        snap = []
        for k in range(20):
            st = steps[k % 2]
            st.run()
            snap.append([t.clone() for t in outs(st)])
        torch.cuda.synchronize()
        for k, got in enumerate(snap):
            for a, b in zip(ref[k % 2], got):
                assert torch.equal(a, b), f"step {chunk * 20 + k} differs"
    for k in range(10):                            # serial dispatch control arm
        st = steps[k % 2]
        for call in (st.build_mask, st.attention, st.accept, st.commit):
            call()
            torch.cuda.synchronize()
        for a, b in zip(ref[k % 2], outs(st)):
            assert torch.equal(a, b), f"serial step {k} differs"


def test_concurrent_streams():
    """The library keeps no state between calls: two different steps, each with its own
    workspaces, enqueued on two streams with no ordering between them (ten rounds), give
    byte for byte the outputs each gives alone.  One merges several chunks per sequence
    inside the attention kernel (arrival counters in its workspace), the other is fp32."""
    shapes = [wl.scaled(wl.WORKLOADS["long32k"], name="cs-a", B=6, prefix=(1200, 2000), V=300),
              wl.scaled(wl.WORKLOADS["tiny"], name="cs-b", B=5, Hq=4, Hkv=2, prefix=(100, 600),
                        block_size=16, shuffled=True)]
    inps = [wl.make_inputs(w, seed=19 + j, device=DEV) for j, w in enumerate(shapes)]
    steps = [VerifyStep.from_inputs(inp) for inp in inps]
    pools0 = [(inp.k_pool.clone(), inp.v_pool.clone()) for inp in inps]
    alone = []
    for st in steps:
        st.run()
        torch.cuda.synchronize()
        alone.append((st.out.clone(), st.accepted_len.clone(), st.new_prefix_len.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rnd in range(10):
        _say(f"[case] concurrent streams round {rnd}")
        for st, (k0, v0), inp in zip(steps, pools0, inps):
            inp.k_pool.copy_(k0)
            inp.v_pool.copy_(v0)
            st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        for st, s in zip(steps, streams):
            st.run(stream=s)
        torch.cuda.synchronize()
        for st, (o, L, npl) in zip(steps, alone):
            assert torch.equal(st.out, o), f"round {rnd}: attention output differs"
            assert torch.equal(st.accepted_len, L) and torch.equal(st.new_prefix_len, npl)
