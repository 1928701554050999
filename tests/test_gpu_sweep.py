"""A seeded sweep of verify-step shapes against the oracle, through the C ABI.

The fixed cases elsewhere follow the workloads of the pages and their edges one at a time;
here 120 shapes are drawn from one fixed generator so that the combinations meet: bf16
and fp32, head_dim 128 / 256 / 512, GQA groups of 1 to 8 query heads (up to 512 query rows
per kv head, i.e. two row groups), trees of 1 to 64 nodes (chains, random trees, EAGLE-2
trees), ragged prefixes from 0 to 4200 keys, contiguous and paged caches (block sizes 16
to 256, in order or shuffled), automatic and explicit chunk counts, vocabularies from 1 to
32000 and draft tokens that match their parent's argmax never, sometimes or always.

Every case runs the whole step (mask, attention, greedy acceptance, commit) and compares
it with the oracle as the parity tests do: bit for bit except the attention outputs, which
are held to max-abs 1e-2 and relative RMS 2^-6 on every row.  Every other case then runs
the write-before-accept step on fresh inputs from the same seed (append, attention over
the cache-resident tree, acceptance, compaction) against the oracle's, the same way.  The
oracle's work per case is bounded, so the sweep takes well under a minute of host time.

Two more sweeps of 60 cases each cover the other stages the same way: sampled acceptance
(temperatures from 0.05 to 2, vocabularies from 1 to 151936, trees and draft-match rates
as above), held to the sampled tests' rule (identical results except a decision within
5e-5 of its boundary, which must pass the fp64 replay); and the draft tree (top-K of every
drafter row, then the best-first expansion; K from 1 to 64, level limits, logits from
narrow to wide and on coarse grids that make ties common), held to the draft tests' rule.
A last sweep of 40 cases covers the tree-position RoPE (even head_dims from 2 to 1024, bf16
and fp32, theta from 100 to 10^6, positions up to 2^20), held to the RoPE tests' rules.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from parity import compare, gpu_step, host_copy, oracle_in_cache, oracle_step, step_result
from tree_masked_verify_amd import workloads as wl
from tree_masked_verify_amd.step import VerifyStep
from test_gpu_draft import check_draft, check_topk
from test_gpu_rope import check as check_rope
from test_gpu_sampled import run as run_sampled

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 120
ORACLE_BUDGET = 4e8          # B * Hq * T * (max prefix + T) * D per case
N_STAGE_CASES = 60
LOGIT_BUDGET = 2e7           # B * T * V per case of the sampled and draft sweeps


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tree_ok(w: wl.Workload, seed: int) -> bool:
    """Whether make_inputs can draw this tree with this seed (the tree is the first draw
    of the input generator, so the same seed gives the same attempt)."""
    try:
        wl.make_trees(w, np.random.Generator(np.random.PCG64(seed)))
        return True
    except (RuntimeError, IndexError):
        return False


def _tree_kind(rng: np.random.Generator, T: int):
    """A tree kind for T nodes and its parameters (random trees get enough levels and
    children per node for T nodes to fit)."""
    kind = str(rng.choice(["chain", "random", "eagle2"])) if T > 1 else "chain"
    levels, children, topk = 0, 0, 0
    if kind == "random":
        children = int(rng.integers(2, 5))
        need = 1
        while sum(children ** j for j in range(need)) < T:
            need += 1
        levels = int(rng.integers(need, max(need, min(T, 8)) + 1))
    elif kind == "eagle2":
        topk = int(rng.integers(2, 9))
        levels = int(rng.integers(3, 9))
    return kind, levels, children, topk


def _draw(rng: np.random.Generator, i: int):
    while True:
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        D = int(rng.choice([128, 256, 512]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 31, 32, 33, 48, 63, 64]))
        B = int(rng.integers(1, 7))
        hi = int(rng.choice([0, 1, 15, 16, 17, 63, 64, 65, 100, 500, 1000, 2100, 4200]))
        lo = int(rng.integers(0, hi + 1))
        bs = int(rng.choice([0, 16, 32, 64, 128, 256]))
        splits = int(rng.choice([0, 0, 0, 1, 2, 3, 7]))
        V = int(rng.choice([1, 7, 100, 1000, 5000, 32000]))
        std = float(rng.choice([0.5, 1.0, 2.0]))
        draft_p = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
        kind, levels, children, topk = _tree_kind(rng, T)
        if B * Hkv * G * T * (hi + T) * D > ORACLE_BUDGET:
            continue
        w = wl.Workload(name=f"sweep{i:02d}", B=B, Hq=Hkv * G, Hkv=Hkv, D=D, dtype=dtype,
                        prefix=(lo, hi), T=T, tree=kind, V=V, logit_std=2.0, draft_p=draft_p,
                        block_size=bs, shuffled=bool(rng.random() < 0.5), max_levels=levels,
                        max_children=children, topk=topk, qkv_std=std)
        seed = 1000 + i
        if _tree_ok(w, seed):
            return w, seed, splits


def _cases():
    rng = np.random.Generator(np.random.PCG64(20261202))
    return [_draw(rng, i) for i in range(N_CASES)]


CASES = _cases()


VOCABS = [1, 2, 7, 100, 1000, 17000, 65537, 151936]
TREE_SIZES = [1, 2, 3, 5, 8, 13, 16, 17, 31, 32, 33, 48, 63, 64]


def _draw_sampled(rng: np.random.Generator, i: int):
    while True:
        B = int(rng.integers(1, 9))
        T = int(rng.choice(TREE_SIZES))
        V = int(rng.choice(VOCABS))
        if B * T * V > LOGIT_BUDGET:
            continue
        kind, levels, children, topk = _tree_kind(rng, T)
        w = wl.Workload(name=f"sampled{i:02d}", B=B, Hq=1, Hkv=1, D=128, dtype="bf16",
                        prefix=(0, 0), T=T, tree=kind, V=V,
                        logit_std=float(rng.choice([0.5, 2.0, 8.0])),
                        draft_p=float(rng.choice([0.0, 0.5, 0.9, 1.0])), block_size=0,
                        max_levels=levels, max_children=children, topk=topk,
                        temperature=float(rng.choice([0.05, 0.3, 1.0, 2.0])))
        seed = 2000 + i
        if _tree_ok(w, seed):
            return w, seed


def _tree_capacity(K: int, levels: int) -> int:
    return sum(min(K ** j, 65) for j in range(levels))


def _draw_draft(rng: np.random.Generator, i: int):
    while True:
        B = int(rng.integers(1, 9))
        T = int(rng.choice(TREE_SIZES))
        V = int(rng.choice(VOCABS))
        if B * T * V > LOGIT_BUDGET:
            continue
        K = int(rng.integers(1, min(64, V) + 1))
        levels = int(rng.integers(1, 9))
        if _tree_capacity(K, levels) < T:
            continue
        return dict(name=f"draft{i:02d}", B=B, T=T, V=V, K=K, levels=levels,
                    std=float(rng.choice([0.5, 2.0, 8.0, 40.0])),
                    grid=bool(rng.random() < 0.3), seed=3000 + i)


def _draw_rope(rng: np.random.Generator, i: int):
    while True:
        B = int(rng.integers(1, 9))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.choice(TREE_SIZES))
        D = int(rng.choice([2, 4, 6, 32, 64, 96, 128, 256, 512, 1024]))
        kind, levels, children, topk = _tree_kind(rng, T)
        w = wl.Workload(name=f"rope{i:02d}", B=B, Hq=Hkv * G, Hkv=Hkv, D=D,
                        dtype=str(rng.choice(["bf16", "f32"])), prefix=(0, 0), T=T, tree=kind,
                        V=1, logit_std=1.0, draft_p=0.0, block_size=0, max_levels=levels,
                        max_children=children, topk=topk)
        prefix = rng.integers(0, int(rng.choice([64, 4096, 65536, 1 << 20])) + 1, size=B)
        theta = float(rng.choice([100.0, 10000.0, 500000.0, 1000000.0]))
        seed = 4000 + i
        if _tree_ok(w, seed):
            return w, seed, [int(v) for v in prefix], theta


SAMPLED_CASES = [_draw_sampled(np.random.Generator(np.random.PCG64([20261202, 1, i])), i)
                 for i in range(N_STAGE_CASES)]
DRAFT_CASES = [_draw_draft(np.random.Generator(np.random.PCG64([20261202, 2, i])), i)
               for i in range(N_STAGE_CASES)]
ROPE_CASES = [_draw_rope(np.random.Generator(np.random.PCG64([20261202, 3, i])), i)
              for i in range(40)]


@pytest.fixture(scope="module")
def orc():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return O.Oracle()


@pytest.mark.parametrize("case", range(N_CASES), ids=[c[0].name for c in CASES])
def test_sweep(orc, case):
    w, seed, splits = CASES[case]
    _say(f"[case] {w.name} seed={seed} {w.dtype} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
         f"T={w.T} tree={w.tree} prefix={w.prefix} block={w.block_size}"
         f"{' shuffled' if w.shuffled else ''} V={w.V} splits={splits}")
    inp = wl.make_inputs(w, seed=seed, device=DEV)
    h = host_copy(inp)
    g = gpu_step(inp, num_splits=splits)
    o = oracle_step(orc, inp, h)
    err = compare(g, o)
    _say(f"       attention max-abs {err['max_abs']:.3e} rel-rms {err['rel_rms']:.3e}, "
         f"accepted {list(g['L'])}")
    if case % 2:
        inp = wl.make_inputs(w, seed=seed, device=DEV)
        h = host_copy(inp)
        st = VerifyStep.from_inputs(inp, num_splits=splits)
        st.run_in_cache()
        err = compare(step_result(st, inp), oracle_in_cache(orc, inp, h))
        _say(f"       write-before-accept: attention max-abs {err['max_abs']:.3e}")


@pytest.mark.parametrize("case", range(N_STAGE_CASES), ids=[c[0].name for c in SAMPLED_CASES])
def test_sweep_sampled(orc, case):
    w, seed = SAMPLED_CASES[case]
    inp = wl.make_inputs(w, seed=seed, device=DEV)
    run_sampled(orc, inp.logits, inp.draft, inp.parents, w.temperature, seed,
                label=f"{w.name} {w.tree} std={w.logit_std} draft_p={w.draft_p}")


@pytest.mark.parametrize("case", range(N_STAGE_CASES), ids=[c["name"] for c in DRAFT_CASES])
def test_sweep_draft(orc, case):
    c = DRAFT_CASES[case]
    rng = np.random.default_rng(c["seed"])
    x = rng.normal(0.0, c["std"], size=(c["B"], c["T"], c["V"]))
    if c["grid"]:  # a coarse grid: many tied logits
        x = np.round(x * 4.0) / 4.0
    x = x.astype(np.float32)
    roots = rng.integers(0, c["V"], size=c["B"]).astype(np.int32)
    label = f"{c['name']} std={c['std']}{' grid' if c['grid'] else ''}"
    check_topk(orc, x.reshape(-1, c["V"]), c["K"], label=label)
    check_draft(orc, x, roots, c["K"], c["levels"], label=label)


@pytest.mark.parametrize("case", range(len(ROPE_CASES)), ids=[c[0].name for c in ROPE_CASES])
def test_sweep_rope(orc, case):
    w, seed, prefix, theta = ROPE_CASES[case]
    inp = wl.make_inputs(w, seed=seed, device=DEV, with_logits=False)
    # beyond 2^16 a last-bit difference of a frequency can flip more roundings than the
    # ordinary rule allows: there the RoPE tests' absolute rule applies
    check_rope(orc, inp, theta, prefix=prefix, label=f"{w.name} {w.tree} P<={max(prefix)}",
               large=max(prefix) > 65536)
