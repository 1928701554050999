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


def run_case(orc, w, seed, num_splits=0, rows=None, **mk):
    _say(f"[case] {w.name} seed={seed} splits={num_splits} B={w.B} T={w.T} D={w.D}")
    inp = wl.make_inputs(w, seed=seed, device=DEV, **mk)
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
    w = wl.WORKLOADS["batched8k"]
    run_case(orc, w, 0, rows=sample_rows(w, 48, 1))


def test_long32k_full_size(orc):
    w = wl.WORKLOADS["long32k"]
    run_case(orc, w, 0, rows=sample_rows(w, 48, 2))


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


@pytest.mark.parametrize("B,splits", [(32, 0), (32, 2), (70, 0)])
def test_varied_prefix_chunking(orc, B, splits):
    """The batched shape's heads with prefix lengths from 0 to 3000, some on either side of
    the chunk boundary the kernel picks.  Automatic chunking at B = 32 (64 (sequence, chunk)
    pairs) cuts the chunks from the actual lengths and starts the largest first; B = 70 and
    an explicit split count keep the plan's uniform chunks.  Two rows of every sequence."""
    rng = np.random.default_rng(B)
    P = [3000, 0, 2999, 1, 2016, 2015, 2017, 32, 31, 33, 2000, 1500]  # chunk length 2016 at B = 32
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
    """The 32K shape at head_dim 128, full size, sampled rows against the oracle."""
    w = wl.WORKLOADS["long32k_d128"]
    run_case(orc, w, 0, rows=sample_rows(w, 120, 9))
