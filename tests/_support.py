"""Test plumbing: moving generated inputs into the oracle's host format.

Only conversions live here (torch tensor -> numpy array, bf16 -> its uint16 bit
pattern).  No arithmetic of the verify step.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tree_masked_verify_amd import workloads  # noqa: E402


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy; bf16 tensors become their uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray, dtype_code: int) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype_code == oracle.BF16 else a.astype(np.float64)


def dtype_code(w: workloads.Workload) -> int:
    return oracle.BF16 if w.dtype == "bf16" else oracle.F32


def oracle_cache(inp: workloads.Inputs, k_pool=None, v_pool=None, table=None) -> oracle.Cache:
    bstr, hstr, rstr = inp.strides
    k = to_np(inp.k_pool) if k_pool is None else k_pool
    v = to_np(inp.v_pool) if v_pool is None else v_pool
    return oracle.Cache(k=k, v=v, table=to_np(inp.block_table) if table is None else table,
                        block_size=inp.block_size, block_stride=bstr, head_stride=hstr,
                        row_stride=rstr, num_blocks=inp.num_blocks, dtype=dtype_code(inp.w))


def gather_prefix(cache: oracle.Cache, b: int, h: int, P: int, which: str = "k") -> np.ndarray:
    """Rows 0..P-1 of sequence b, kv head h as float64 [P, D], by numpy fancy indexing
    over the block table (an addressing independent of the oracle's)."""
    pool = cache.k if which == "k" else cache.v
    nb = pool.shape[0]
    D = cache.row_stride
    pool4 = pool.reshape(nb, -1, cache.block_size, D)
    pos = np.arange(P)
    blk = cache.table[b, pos // cache.block_size]
    rows = pool4[blk, h, pos % cache.block_size, :]
    return as_f64(rows, cache.dtype)
