"""CPU oracle for the tree-masked speculative verify step (ctypes over sv_oracle.c).

TEST INFRASTRUCTURE ONLY.  The functions here are the slow fp64 reference the
GPU library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; it imports nothing from
the GPU library and the GPU library imports nothing from it.

Every function takes and returns host numpy arrays.  Sources are cited in
sv_oracle.c next to each definition.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_sv.so")

TREE_OK, TREE_BAD_ROOT, TREE_BAD_PARENT = 0, 1, 2
F32, BF16 = 0, 1


def build(src: str = _SRC, out: str = _LIB, defines: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (fp contraction off, OpenMP on)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           *[f"-D{d}" for d in defines], src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_i32p = ctypes.POINTER(ctypes.c_int32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_f32p = ctypes.POINTER(ctypes.c_float)
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _declare(lib):
    lib.oracle_build_tree_mask.argtypes = [_i32p, _int, _int, _u64p, _i32p, _i32p]
    lib.oracle_tree_verify_attention.argtypes = [
        _vp, _vp, _vp, _vp, _vp, _i32p, _int, _int, _i64, _i64, _i64, _i64, _int,
        _i32p, _int, _u64p, _int, _int, _int, _int, _int, ctypes.c_double, _i32p, _i64,
        _f32p, _int]
    lib.oracle_argmax.argtypes = [_f32p, _i64, _i64, _i32p, _int]
    lib.oracle_accept_longest_path.argtypes = [
        _f32p, _i32p, _i32p, _i32p, _int, _int, _i64, _i32p, _i32p, _i32p, _i32p]
    lib.oracle_accept_sampled.argtypes = [
        _f32p, _i32p, _i32p, _i32p, _f32p, _f32p, ctypes.c_double, _int, _int, _i64, _i32p,
        _i32p, _i32p]
    lib.oracle_rope_tree.argtypes = [_vp, _vp, _i32p, _i32p, _int, _int, _int, _int, _int, _int,
                                     ctypes.c_double]
    lib.oracle_kv_commit.argtypes = [
        _vp, _vp, _i32p, _i32p, _i32p, _vp, _vp, _i32p, _int, _int, _i64, _i64, _i64, _i64,
        _int, _i32p, _int, _i32p, _int, _int, _int, _int]
    lib.oracle_kv_append.argtypes = [
        _vp, _vp, _i32p, _vp, _vp, _i32p, _int, _int, _i64, _i64, _i64, _i64, _int, _i32p, _int,
        _int, _int, _int, _int]
    lib.oracle_kv_compact.argtypes = [
        _i32p, _i32p, _i32p, _vp, _vp, _i32p, _int, _int, _i64, _i64, _i64, _i64, _int, _i32p,
        _int, _i32p, _int, _int, _int, _int]
    _f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_topk_logprobs.argtypes = [_f32p, _i64, _i64, _int, _i32p, _f64p, _int]
    lib.oracle_draft_tree.argtypes = [_f32p, _i32p, _int, _int, _i64, _int, _int, _i32p, _i32p,
                                      _f64p]
    for f in ("oracle_build_tree_mask", "oracle_tree_verify_attention", "oracle_argmax",
              "oracle_accept_longest_path", "oracle_accept_sampled", "oracle_rope_tree",
              "oracle_kv_commit", "oracle_topk_logprobs", "oracle_draft_tree",
              "oracle_kv_append", "oracle_kv_compact"):
        getattr(lib, f).restype = _int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    path = path or _LIB
    if not os.path.exists(path):
        build(out=path)
    return _declare(ctypes.CDLL(path))


def _p(a: np.ndarray | None, t):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(t)


@dataclass
class Cache:
    """A KV cache in host memory: K and V pools addressed through a block table.

    Position p of sequence b, kv head h is element
    table[b, p // block_size] * block_stride + h * head_stride + (p % block_size) * row_stride.
    """
    k: np.ndarray
    v: np.ndarray
    table: np.ndarray          # int32 [B, max_blocks]
    block_size: int
    block_stride: int
    head_stride: int
    row_stride: int
    num_blocks: int
    dtype: int                 # F32 or BF16 (bf16 stored as uint16 bit patterns)

    @property
    def max_blocks(self) -> int:
        return int(self.table.shape[1])


class Oracle:
    """numpy-facing wrapper of the C oracle."""

    def __init__(self, path: str | None = None):
        self.lib = load(path)

    def build_tree_mask(self, parents: np.ndarray):
        parents = np.ascontiguousarray(parents, dtype=np.int32)
        B, T = parents.shape
        W = (T + 63) // 64
        mask = np.zeros((B, T, W), np.uint64)
        depth = np.zeros((B, T), np.int32)
        err = np.zeros((B,), np.int32)
        rc = self.lib.oracle_build_tree_mask(_p(parents, _i32p), B, T, _p(mask, _u64p),
                                             _p(depth, _i32p), _p(err, _i32p))
        assert rc == 0
        return mask, depth, err

    def tree_verify_attention(self, q, k_tree, v_tree, cache: Cache, prefix_len, max_prefix_len,
                              mask, scale, rows=None, nthreads=0):
        """q [B,Hq,T,D], k_tree/v_tree [B,Hkv,T,D] (float32, or uint16 bf16 bits); with
        k_tree and v_tree None the tree rows are read from the cache at positions P + j.

        Returns out float32 [B,T,Hq,D], or [len(rows), D] when rows (int32 [n,3] of
        (b, h, i)) is given.
        """
        B, Hq, T, D = q.shape
        Hkv = k_tree.shape[1] if k_tree is not None else cache.block_stride // cache.head_stride
        prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32)
        mask = np.ascontiguousarray(mask, dtype=np.uint64)
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
            out = np.zeros((rows.shape[0], D), np.float32)
            nrows = rows.shape[0]
        else:
            out = np.zeros((B, T, Hq, D), np.float32)
            nrows = 0
        for a in (q, k_tree, v_tree, cache.k, cache.v, cache.table):
            assert a is None or a.flags["C_CONTIGUOUS"]
        assert (k_tree is None) == (v_tree is None)
        rc = self.lib.oracle_tree_verify_attention(
            q.ctypes.data, None if k_tree is None else k_tree.ctypes.data,
            None if v_tree is None else v_tree.ctypes.data, cache.k.ctypes.data,
            cache.v.ctypes.data, _p(cache.table, _i32p), cache.block_size, cache.max_blocks,
            cache.block_stride, cache.head_stride, cache.row_stride, cache.num_blocks,
            cache.dtype, _p(prefix_len, _i32p), int(max_prefix_len), _p(mask, _u64p), B, Hq,
            Hkv, T, D, float(scale), _p(rows, _i32p), nrows, _p(out, _f32p), int(nthreads))
        assert rc == 0, rc
        return out

    def argmax(self, logits: np.ndarray, nthreads: int = 0):
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        V = logits.shape[-1]
        flat = logits.reshape(-1, V)
        out = np.zeros((flat.shape[0],), np.int32)
        rc = self.lib.oracle_argmax(_p(flat, _f32p), flat.shape[0], V, _p(out, _i32p),
                                    int(nthreads))
        assert rc == 0
        return out.reshape(logits.shape[:-1])

    def accept_longest_path(self, logits, draft, parents, tree_err=None):
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        draft = np.ascontiguousarray(draft, dtype=np.int32)
        parents = np.ascontiguousarray(parents, dtype=np.int32)
        B, T = parents.shape
        V = logits.shape[-1]
        if tree_err is not None:
            tree_err = np.ascontiguousarray(tree_err, dtype=np.int32)
        am = np.zeros((B, T), np.int32)
        L = np.zeros((B,), np.int32)
        nodes = np.zeros((B, T), np.int32)
        toks = np.zeros((B, T), np.int32)
        rc = self.lib.oracle_accept_longest_path(
            _p(logits, _f32p), _p(draft, _i32p), _p(parents, _i32p), _p(tree_err, _i32p), B, T,
            V, _p(am, _i32p), _p(L, _i32p), _p(nodes, _i32p), _p(toks, _i32p))
        assert rc == 0
        return am, L, nodes, toks

    def accept_sampled(self, logits, draft, parents, u_accept, u_sample, temperature,
                       tree_err=None):
        """Sampled acceptance; returns (accepted_len, accepted_nodes, out_tokens)."""
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        draft = np.ascontiguousarray(draft, dtype=np.int32)
        parents = np.ascontiguousarray(parents, dtype=np.int32)
        u_accept = np.ascontiguousarray(u_accept, dtype=np.float32)
        u_sample = np.ascontiguousarray(u_sample, dtype=np.float32)
        B, T = parents.shape
        V = logits.shape[-1]
        if tree_err is not None:
            tree_err = np.ascontiguousarray(tree_err, dtype=np.int32)
        L = np.zeros((B,), np.int32)
        nodes = np.zeros((B, T), np.int32)
        toks = np.zeros((B, T), np.int32)
        rc = self.lib.oracle_accept_sampled(
            _p(logits, _f32p), _p(draft, _i32p), _p(parents, _i32p), _p(tree_err, _i32p),
            _p(u_accept, _f32p), _p(u_sample, _f32p), float(temperature), B, T, V, _p(L, _i32p),
            _p(nodes, _i32p), _p(toks, _i32p))
        assert rc == 0
        return L, nodes, toks

    def kv_append(self, k_tree, v_tree, tree_err, cache: Cache, prefix_len, max_prefix_len):
        """Writes the tree rows into cache.k / cache.v at [P, P + T) in place; returns the
        updated tree_err (3 where a sequence could not be written)."""
        B, Hkv, T, D = k_tree.shape
        err = np.zeros((B,), np.int32) if tree_err is None else \
            np.array(tree_err, dtype=np.int32, copy=True)
        prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32)
        rc = self.lib.oracle_kv_append(
            k_tree.ctypes.data, v_tree.ctypes.data, _p(err, _i32p), cache.k.ctypes.data,
            cache.v.ctypes.data, _p(cache.table, _i32p), cache.block_size, cache.max_blocks,
            cache.block_stride, cache.head_stride, cache.row_stride, cache.num_blocks,
            cache.dtype, _p(prefix_len, _i32p), int(max_prefix_len), B, Hkv, T, D)
        assert rc == 0
        return err

    def kv_compact(self, accepted_len, accepted_nodes, tree_err, cache: Cache, prefix_len,
                   max_prefix_len, Hkv, T, D):
        """Moves the accepted rows to [P, P + L) in place; returns new_prefix_len."""
        accepted_len = np.ascontiguousarray(accepted_len, dtype=np.int32)
        accepted_nodes = np.ascontiguousarray(accepted_nodes, dtype=np.int32)
        prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32)
        B = accepted_len.shape[0]
        if tree_err is not None:
            tree_err = np.ascontiguousarray(tree_err, dtype=np.int32)
        npl = np.zeros((B,), np.int32)
        rc = self.lib.oracle_kv_compact(
            _p(accepted_len, _i32p), _p(accepted_nodes, _i32p), _p(tree_err, _i32p),
            cache.k.ctypes.data, cache.v.ctypes.data, _p(cache.table, _i32p), cache.block_size,
            cache.max_blocks, cache.block_stride, cache.head_stride, cache.row_stride,
            cache.num_blocks, cache.dtype, _p(prefix_len, _i32p), int(max_prefix_len),
            _p(npl, _i32p), B, Hkv, T, D)
        assert rc == 0
        return npl

    def topk_logprobs(self, logits, K, nthreads: int = 0):
        """Top-K of each row's log-softmax: (tokens int32 [..., K], logp float64 [..., K]),
        best first, ties to the smaller token."""
        logits = np.ascontiguousarray(logits, dtype=np.float32)
        V = logits.shape[-1]
        flat = logits.reshape(-1, V)
        tok = np.zeros((flat.shape[0], K), np.int32)
        lp = np.zeros((flat.shape[0], K), np.float64)
        rc = self.lib.oracle_topk_logprobs(_p(flat, _f32p), flat.shape[0], V, int(K),
                                           _p(tok, _i32p),
                                           _p(lp, ctypes.POINTER(ctypes.c_double)),
                                           int(nthreads))
        assert rc == 0, rc
        return tok.reshape(*logits.shape[:-1], K), lp.reshape(*logits.shape[:-1], K)

    def draft_tree(self, drafter_logits, root_tokens, K, max_levels):
        """Best-first tree expansion over drafter rows [B, T, V] (row i: the drafter's
        output for the node admitted i-th).  Returns (parents int32 [B, T], tokens int32
        [B, T], cum float64 [B, T]); raises ValueError when the shape is refused."""
        dl = np.ascontiguousarray(drafter_logits, dtype=np.float32)
        root_tokens = np.ascontiguousarray(root_tokens, dtype=np.int32)
        B, T, V = dl.shape
        par = np.zeros((B, T), np.int32)
        tok = np.zeros((B, T), np.int32)
        cum = np.zeros((B, T), np.float64)
        rc = self.lib.oracle_draft_tree(_p(dl, _f32p), _p(root_tokens, _i32p), B, T, V, int(K),
                                        int(max_levels), _p(par, _i32p), _p(tok, _i32p),
                                        _p(cum, ctypes.POINTER(ctypes.c_double)))
        if rc == -1:
            raise ValueError("draft_tree: shape refused")
        assert rc == 0, rc
        return par, tok, cum

    def rope_tree(self, q, k_tree, prefix_len, depth, theta, dtype):
        """Returns rotated copies of q [B, Hq, T, D] and k_tree [B, Hkv, T, D] (float32
        arrays, or uint16 bf16 bit patterns with dtype BF16)."""
        q = np.array(q, copy=True, order="C")
        k = np.array(k_tree, copy=True, order="C")
        prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32)
        depth = np.ascontiguousarray(depth, dtype=np.int32)
        B, Hq, T, D = q.shape
        Hkv = k.shape[1]
        rc = self.lib.oracle_rope_tree(q.ctypes.data, k.ctypes.data, _p(prefix_len, _i32p),
                                       _p(depth, _i32p), B, Hq, Hkv, T, D, int(dtype),
                                       float(theta))
        assert rc == 0
        return q, k

    def kv_commit(self, k_tree, v_tree, accepted_len, accepted_nodes, tree_err, cache: Cache,
                  prefix_len, max_prefix_len, new_prefix_len=True):
        """Commits in place into cache.k / cache.v; returns new_prefix_len (or None)."""
        B, Hkv, T, D = k_tree.shape
        accepted_len = np.ascontiguousarray(accepted_len, dtype=np.int32)
        accepted_nodes = np.ascontiguousarray(accepted_nodes, dtype=np.int32)
        prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32)
        if tree_err is not None:
            tree_err = np.ascontiguousarray(tree_err, dtype=np.int32)
        npl = np.zeros((B,), np.int32) if new_prefix_len else None
        rc = self.lib.oracle_kv_commit(
            k_tree.ctypes.data, v_tree.ctypes.data, _p(accepted_len, _i32p),
            _p(accepted_nodes, _i32p), _p(tree_err, _i32p), cache.k.ctypes.data,
            cache.v.ctypes.data, _p(cache.table, _i32p), cache.block_size, cache.max_blocks,
            cache.block_stride, cache.head_stride, cache.row_stride, cache.num_blocks,
            cache.dtype, _p(prefix_len, _i32p), int(max_prefix_len), _p(npl, _i32p), B, Hkv, T,
            D)
        assert rc == 0
        return npl
