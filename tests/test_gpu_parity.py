"""GPU parity: the HIP path through the C ABI against the oracle, same seeded inputs.

Bit-exact: masks, depths, tree errors, argmax, accepted lengths / nodes / tokens, new
prefix lengths and every byte of both cache pools after the commit.  Attention
outputs: max-abs <= 1e-2 and relative RMS <= 2^-6.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from parity import compare, gpu_step, host_copy, oracle_step, sample_rows
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


def run_case(orc, w, seed, num_splits=0, rows=None, mutate=None, **mk):
    _say(f"[case] {w.name} seed={seed} splits={num_splits} B={w.B} T={w.T} D={w.D}")
    inp = wl.make_inputs(w, seed=seed, device=DEV, **mk)
    if mutate is not None:
        mutate(inp)
    h = host_copy(inp)
    g = gpu_step(inp, num_splits=num_splits)
    o = oracle_step(orc, inp, h, rows=rows)
    err = compare(g, o, rows=rows)
    _say(f"       attention max-abs {err['max_abs']:.3e} rel-rms {err['rel_rms']:.3e}, "
         f"accepted {list(g['L'][:8])}")
    return inp, g, o


# ----------------------------------------------------------------- the five workload shapes
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny(orc, seed):
    run_case(orc, wl.WORKLOADS["tiny"], seed)


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_parity512(orc, seed):
    run_case(orc, wl.WORKLOADS["parity512"], seed)


@pytest.mark.parametrize("seed", [0, 1])
def test_chain2k(orc, seed):
    run_case(orc, wl.WORKLOADS["chain2k"], seed)


def test_batched8k_full_size(orc):
    """Every output row of the full batched workload (32 sequences, prefixes 4096-8192,
    chunks cut from the actual lengths, merged inside the attention kernel)."""
    run_case(orc, wl.WORKLOADS["batched8k"], 0)


def test_long32k_full_size(orc):
    """Every output row of the full 32K workload (16 x 32 heads x 60 nodes)."""
    run_case(orc, wl.WORKLOADS["long32k"], 0)


# ----------------------------------------------------------------- reduced shapes, every row
@pytest.mark.parametrize("seed", [0, 1])
def test_batched_reduced_ragged(orc, seed):
    w = wl.scaled(wl.WORKLOADS["batched8k"], name="batched_small", B=4, prefix=(290, 1111),
                  V=5003)
    run_case(orc, w, seed)


@pytest.mark.parametrize("splits", [0, 1, 3, 7])
def test_long_reduced_splits(orc, splits):
    w = wl.scaled(wl.WORKLOADS["long32k"], name="long_small", B=2, prefix=(1501, 1501), V=4096)
    run_case(orc, w, 3, num_splits=splits)


def _rows_every_sequence(w):
    """Two (b, h, i) rows of every sequence."""
    return np.array(sorted({(b, (7 * b) % w.Hq, (3 * b) % w.T) for b in range(w.B)} |
                           {(b, (7 * b + 19) % w.Hq, (5 * b + 1) % w.T) for b in range(w.B)}),
                    dtype=np.int32)


@pytest.mark.parametrize("B,splits", [(8, 0), (12, 0), (32, 0), (32, 2), (70, 0)])
def test_varied_prefix_chunking(orc, B, splits):
    """The batched shape's heads with prefix lengths from 0 to 3000, some on either side of
    a chunk boundary.  Automatic chunking at B = 8 and 12 (the grid needs several chunks per
    sequence) cuts the chunks from the actual lengths, starts the largest first and merges
    them inside the attention kernel; at B = 32 and 70 one chunk per sequence fills the
    grid and each workgroup writes its rows' output directly; an explicit split count keeps
    the plan's uniform chunks.  Two rows of every sequence."""
    rng = np.random.default_rng(B)
    P = [3000, 0, 2999, 1, 2016, 2015, 2017, 32, 31, 33, 2000, 1500][:B]
    P += [int(v) for v in rng.integers(1500, 3001, B - len(P))]
    w = wl.scaled(wl.WORKLOADS["batched8k"], name=f"varied{B}", B=B, prefix=(0, 3000), V=1000)
    run_case(orc, w, 5, num_splits=splits, rows=_rows_every_sequence(w), prefix_override=P)


@pytest.mark.parametrize("bs", [32, 48, 64, 256])
def test_block_sizes(orc, bs):
    # cache blocks larger than a 16-key group: both groups of a tile often share a block
    w = wl.scaled(wl.WORKLOADS["long32k"], name=f"bs{bs}", B=2, prefix=(1501, 2000), V=2048,
                  block_size=bs)
    run_case(orc, w, 5)


def test_chunk_beyond_staged_table(orc):
    # one chunk of 40000 keys in 16-key blocks touches 2500 table entries, more than
    # the kernel stages in LDS, so its tiles read the block table directly
    w = wl.scaled(wl.WORKLOADS["long32k"], name="chunk40k", B=1, Hq=8, Hkv=2,
                  prefix=(40000, 40000), V=2048)
    run_case(orc, w, 6, num_splits=1, rows=sample_rows(w, 32, 3))


def test_peaked_attention(orc):
    """Sharp softmax (Q, K with std 3): outputs of order one, so 1e-2 is tight."""
    w = wl.scaled(wl.WORKLOADS["long32k"], name="peaked", B=2, prefix=(700, 900), V=2048,
                  qkv_std=3.0)
    run_case(orc, w, 5)
    w = wl.scaled(wl.WORKLOADS["parity512"], name="peaked512", qkv_std=3.0)
    run_case(orc, w, 6)


def test_prefix_zero_and_single_node(orc):
    run_case(orc, wl.scaled(wl.WORKLOADS["parity512"], name="p0", prefix=(0, 0), capacity=16), 7)
    run_case(orc, wl.scaled(wl.WORKLOADS["parity512"], name="t1", T=1, tree="chain",
                            prefix=(333, 333), capacity=352), 8)
    run_case(orc, wl.scaled(wl.WORKLOADS["tiny"], name="t1f", T=1, tree="chain",
                            parents=(-1,)), 9)


def test_fp32_gqa(orc):
    run_case(orc, wl.scaled(wl.WORKLOADS["tiny"], name="f32gqa", Hq=8, Hkv=2, prefix=(40, 90),
                            B=3, tree="random", max_levels=4, max_children=3, capacity=160,
                            block_size=0), 10)


def test_unaligned_vocab(orc):
    run_case(orc, wl.scaled(wl.WORKLOADS["parity512"], name="v1001", V=1001, B=3), 11)


# ----------------------------------------------------------------- head_dim 128
@pytest.mark.parametrize("seed", [0, 1])
def test_parity512_head_dim_128(orc, seed):
    """Matrix-core path (bf16, 64 rows per kv head) at head_dim 128."""
    run_case(orc, wl.scaled(wl.WORKLOADS["parity512"], D=128, name="parity512-d128"), seed)


def test_tiny_head_dim_128(orc):
    """VALU path (fp32) at head_dim 128."""
    run_case(orc, wl.scaled(wl.WORKLOADS["tiny"], D=128, name="tiny-d128"), 0)


def test_batched8k_head_dim_128(orc):
    """Paged, shuffled, variable prefix, 512 rows per kv head (two row groups)."""
    w = wl.scaled(wl.WORKLOADS["batched8k"], D=128, B=6, name="batched8k-d128")
    run_case(orc, w, 5, rows=sample_rows(w, 200, 5))


def test_long32k_head_dim_128_full_size(orc):
    """The 32K shape at head_dim 128, full size, every row against the oracle."""
    run_case(orc, wl.WORKLOADS["long32k_d128"], 0)


# ----------------------------------------------------------------- head_dim 512, matrix cores
def _d512(name, **kw):
    base = dict(name=name, B=5, Hq=16, Hkv=2, T=8, tree="random", max_levels=4,
                max_children=3, block_size=16, shuffled=True, prefix=(0, 2100), V=3000)
    base.update(kw)
    return wl.scaled(wl.WORKLOADS["chain2k"], **base)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_head_dim_512_paged_ragged(orc, splits):
    """The head_dim-512 kernel on a paged cache: shuffled 16-row blocks, ragged prefixes
    (0, 1, mid-tile ends), one out-of-range block-table entry, automatic and explicit
    splits."""
    P = [0, 1, 777, 2100, 1599]

    def drop(inp):
        inp.block_table[3, 5] = -1               # keys 80..95 of sequence 3 left out
        inp.block_table[4, 50] = inp.num_blocks  # keys 800..815 of sequence 4 left out
    run_case(orc, _d512("d512paged"), 31, num_splits=splits, mutate=drop, prefix_override=P)


def test_head_dim_512_chunk_beyond_staged_table(orc):
    """One chunk of 40000 keys in 16-row blocks (2500 table entries, more than the
    kernel stages in LDS): its tiles read the block table directly."""
    w = _d512("d512chunk40k", B=1, Hq=8, Hkv=1, prefix=(40000, 40000), tree="chain")
    run_case(orc, w, 32, num_splits=1)


# ----------------------------------------------------------------- few query rows, fp32
def test_bf16_head_dim_128_single_node(orc):
    """bf16, head_dim 128, 8 query rows per kv head (fewer than one 16-row block): the
    matrix-core kernel with its row block padded."""
    run_case(orc, wl.scaled(wl.WORKLOADS["parity512"], name="t1-d128", D=128, T=1,
                            tree="chain", prefix=(333, 333), capacity=352), 12)


def test_valu_f32_head_dim_512(orc):
    """fp32 at head_dim 512 (the tiny workload's tree): the vector-ALU kernel."""
    run_case(orc, wl.scaled(wl.WORKLOADS["tiny"], name="tiny-d512-paged", D=512, B=3, Hq=4,
                            Hkv=2, block_size=16, shuffled=True, prefix=(0, 700)), 15,
             prefix_override=[0, 333, 700])
    run_case(orc, wl.scaled(wl.WORKLOADS["tiny"], name="tiny-d512", D=512), 13)


def test_bf16_head_dim_512_single_node_paged(orc):
    """bf16, head_dim 512, single-node trees on a paged cache with ragged prefixes (the
    shape of the 2K chain's serial single-node verifies): the head_dim-512 matrix-core
    kernel with its row block padded."""
    w = _d512("d512t1", T=1, tree="chain", Hq=8, Hkv=1, B=4)
    run_case(orc, w, 14, prefix_override=[2040, 0, 1001, 17])


@pytest.mark.parametrize("dtype,splits", [("bf16", 0), ("bf16", 3), ("f32", 0), ("f32", 2)])
def test_wide_batch(orc, dtype, splits):
    """300 sequences with short ragged prefixes (0 to 200 keys) on a shuffled paged cache:
    grids of hundreds of workgroups per kv head mapped across the XCDs, one chunk per
    sequence written directly or (explicit splits) several merged inside the kernel across
    hundreds of units.  Every row against the oracle."""
    w = wl.scaled(wl.WORKLOADS["batched8k"], name=f"wide-{dtype}-{splits}", B=300, Hq=4, Hkv=2,
                  D=128, dtype=dtype, T=4, tree="random", max_levels=3, max_children=2,
                  prefix=(0, 200), V=64)
    run_case(orc, w, 16, num_splits=splits)


def test_more_units_than_arrival_counters(orc):
    """4200 sequences x 16 kv heads: 67200 (sequence, kv head, row group) units, more than
    the 65536 arrival counters the merge region holds, so the call takes the separate merge
    kernel instead of merging inside the attention kernel.  Every row against the oracle."""
    w = wl.scaled(wl.WORKLOADS["batched8k"], name="units67200", B=4200, Hq=16, Hkv=16, D=128,
                  T=1, tree="chain", prefix=(0, 48), V=8)
    run_case(orc, w, 17)


@pytest.mark.parametrize("name,Hq,Hkv,T,D,dtype", [
    ("mqa64", 64, 1, 32, 128, "bf16"),      # 2048 query rows on one kv head: 8 row groups
    ("gqa16", 32, 2, 64, 256, "bf16"),      # 1024 rows per kv head: 4 row groups
    ("gqa16-f32", 16, 1, 16, 128, "f32"),   # 256 rows: 16 vector-ALU row groups
    ("gqa32-d512", 32, 1, 16, 512, "bf16"),  # 512 rows at head_dim 512: 4 row groups
])
def test_large_gqa_groups(orc, name, Hq, Hkv, T, D, dtype):
    """GQA groups beyond the sweep's 8 query heads per kv head: many row groups per kv head
    reading the same K/V, ragged paged prefixes, every row against the oracle."""
    w = wl.scaled(wl.WORKLOADS["batched8k"], name=name, B=3, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, T=T,
                  tree="random", max_levels=5, max_children=3, prefix=(100, 900), V=128)
    run_case(orc, w, 18)
