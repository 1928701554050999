"""Tree-masked speculative verify on MI355X (gfx950): Python binding of libsv.so.

The functions below carry the names of the C entry points in include/sv.h and only
marshal arguments: torch tensors become device pointers, a torch stream becomes a
hipStream_t.  Every step of the verify path runs in the library's HIP kernels; there
is no fallback.  If libsv.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SV_LIBRARY_PATH names another build of the library (the sanitizer tests load one)
LIB_PATH = os.environ.get("SV_LIBRARY_PATH", os.path.join(_HERE, "libsv.so"))

SV_F32, SV_BF16 = 0, 1
SV_TREE_OK, SV_TREE_BAD_ROOT, SV_TREE_BAD_PARENT = 0, 1, 2
STATUS = {0: "SV_OK", -1: "SV_ERR_NULL", -2: "SV_ERR_SHAPE", -3: "SV_ERR_DTYPE",
          -4: "SV_ERR_GQA", -5: "SV_ERR_HEAD_DIM", -6: "SV_ERR_TREE_SIZE",
          -7: "SV_ERR_CAPACITY", -8: "SV_ERR_OVERFLOW", -9: "SV_ERR_WORKSPACE",
          -10: "SV_ERR_HIP", -11: "SV_ERR_ALIGN", -12: "SV_ERR_SCRATCH"}
ENTRY_POINTS = ("sv_build_tree_mask", "sv_tree_verify_attention_workspace_size",
                "sv_tree_verify_attention", "sv_tree_verify_attention_noalloc",
                "sv_accept_longest_path_workspace_size",
                "sv_accept_longest_path", "sv_accept_sampled_workspace_size",
                "sv_accept_sampled", "sv_rope_tree", "sv_topk_logprobs",
                "sv_draft_tree_workspace_size", "sv_draft_tree", "sv_kv_append",
                "sv_kv_compact", "sv_kv_commit",
                "sv_status_string")


class SvError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {STATUS.get(code, code)} ({code})")
        self.code = code


class sv_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
                ("block_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("dtype", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsv.so (built by __graft_entry__.build()); raise if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libsv.so not found at {path}: build it first "
                           "(python -c 'import __graft_entry__; __graft_entry__.build()')")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.sv_build_tree_mask.argtypes = [vp, i32, i32, vp, vp, vp, vp]
    lib.sv_tree_verify_attention_workspace_size.argtypes = [i32] * 8
    lib.sv_tree_verify_attention_workspace_size.restype = sz
    lib.sv_tree_verify_attention.argtypes = [
        vp, vp, vp, ctypes.POINTER(sv_kv_cache), vp, i32, vp, i32, i32, i32, i32, i32,
        ctypes.c_float, vp, vp, sz, i32, vp]
    lib.sv_tree_verify_attention_noalloc.argtypes = [
        vp, vp, vp, ctypes.POINTER(sv_kv_cache), vp, i32, vp, i32, i32, i32, i32, i32,
        ctypes.c_float, vp, i32, vp]
    lib.sv_accept_longest_path_workspace_size.argtypes = [i32, i32, i64]
    lib.sv_accept_longest_path_workspace_size.restype = sz
    lib.sv_accept_longest_path.argtypes = [vp, vp, vp, vp, i32, i32, i64, vp, vp, vp, vp, vp,
                                           sz, vp]
    lib.sv_accept_sampled_workspace_size.argtypes = [i32, i32, i64]
    lib.sv_accept_sampled_workspace_size.restype = sz
    lib.sv_accept_sampled.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i64, vp,
                                      vp, vp, vp, sz, vp]
    lib.sv_rope_tree.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_double,
                                 vp]
    lib.sv_kv_append.argtypes = [vp, vp, vp, ctypes.POINTER(sv_kv_cache), vp, i32, i32, i32, i32,
                                 i32, vp]
    lib.sv_kv_compact.argtypes = [vp, vp, vp, ctypes.POINTER(sv_kv_cache), vp, i32, vp, i32, i32,
                                  i32, i32, vp]
    lib.sv_topk_logprobs.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.sv_draft_tree_workspace_size.argtypes = [i32, i32, i32]
    lib.sv_draft_tree_workspace_size.restype = sz
    lib.sv_draft_tree.argtypes = [vp, vp, i32, i32, i64, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.sv_kv_commit.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(sv_kv_cache), vp, i32, vp,
                                 i32, i32, i32, i32, vp]
    lib.sv_status_string.argtypes = [ctypes.c_int]
    lib.sv_status_string.restype = ctypes.c_char_p
    for f in ("sv_build_tree_mask", "sv_tree_verify_attention",
              "sv_tree_verify_attention_noalloc", "sv_accept_longest_path",
              "sv_accept_sampled", "sv_rope_tree", "sv_topk_logprobs", "sv_draft_tree",
              "sv_kv_append", "sv_kv_compact", "sv_kv_commit"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    assert t.is_contiguous(), "tensors passed to libsv must be contiguous"
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise SvError(fn, rc)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SV_BF16
    if t.dtype == torch.float32:
        return SV_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def make_cache(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
               num_blocks: int | None = None) -> sv_kv_cache:
    """Descriptor of a pool laid out [num_blocks][Hkv][block_size][D] (a contiguous
    [B][Hkv][cap][D] cache is the case block_size = cap, block_table[b] = b)."""
    nb, hkv, bs, d = k_pool.shape
    return sv_kv_cache(k=_ptr(k_pool), v=_ptr(v_pool), block_table=_ptr(block_table),
                       block_size=bs, max_blocks_per_seq=block_table.shape[1],
                       num_blocks=nb if num_blocks is None else num_blocks,
                       block_stride=hkv * bs * d, head_stride=bs * d, row_stride=d,
                       dtype=dtype_code(k_pool))


# ----------------------------------------------------------------------------- entry points
def sv_build_tree_mask(parents, mask, depth, tree_err, stream=None) -> None:
    B, T = parents.shape
    rc = load_library().sv_build_tree_mask(_ptr(parents), B, T, _ptr(mask), _ptr(depth),
                                           _ptr(tree_err), _stream(stream))
    _check("sv_build_tree_mask", rc)


def sv_tree_verify_attention_workspace_size(B, Hq, Hkv, T, D, max_prefix_len, dtype,
                                            num_splits=0) -> int:
    return int(load_library().sv_tree_verify_attention_workspace_size(
        B, Hq, Hkv, T, D, max_prefix_len, dtype, num_splits))


def sv_tree_verify_attention(q, k_tree, v_tree, cache: sv_kv_cache, prefix_len, max_prefix_len,
                             mask, scale, out, workspace, num_splits=0, stream=None,
                             Hkv=None) -> None:
    """k_tree = v_tree = None: the tree rows are read from the cache at P + j (then Hkv
    must be given)."""
    B, Hq, T, D = q.shape
    Hkv = k_tree.shape[1] if k_tree is not None else int(Hkv)
    rc = load_library().sv_tree_verify_attention(
        _ptr(q), _ptr(k_tree), _ptr(v_tree), ctypes.byref(cache), _ptr(prefix_len),
        int(max_prefix_len), _ptr(mask), B, Hq, Hkv, T, D, float(scale), _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size() if workspace is not None
        else 0, int(num_splits), _stream(stream))
    _check("sv_tree_verify_attention", rc)


def sv_tree_verify_attention_noalloc(q, k_tree, v_tree, cache: sv_kv_cache, prefix_len,
                                     max_prefix_len, mask, scale, out, num_splits=0,
                                     stream=None, Hkv=None) -> None:
    """sv_tree_verify_attention with the library's own per-device scratch (no workspace)."""
    B, Hq, T, D = q.shape
    Hkv = k_tree.shape[1] if k_tree is not None else int(Hkv)
    rc = load_library().sv_tree_verify_attention_noalloc(
        _ptr(q), _ptr(k_tree), _ptr(v_tree), ctypes.byref(cache), _ptr(prefix_len),
        int(max_prefix_len), _ptr(mask), B, Hq, Hkv, T, D, float(scale), _ptr(out),
        int(num_splits), _stream(stream))
    _check("sv_tree_verify_attention_noalloc", rc)


def sv_accept_longest_path_workspace_size(B, T, V) -> int:
    return int(load_library().sv_accept_longest_path_workspace_size(B, T, V))


def sv_accept_longest_path(logits, draft, parents, tree_err, argmax_out, accepted_len,
                           accepted_nodes, out_tokens, workspace, stream=None) -> None:
    B, T = parents.shape
    V = logits.shape[-1]
    rc = load_library().sv_accept_longest_path(
        _ptr(logits), _ptr(draft), _ptr(parents), _ptr(tree_err), B, T, V, _ptr(argmax_out),
        _ptr(accepted_len), _ptr(accepted_nodes), _ptr(out_tokens), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check("sv_accept_longest_path", rc)


def sv_accept_sampled_workspace_size(B, T, V) -> int:
    return int(load_library().sv_accept_sampled_workspace_size(B, T, V))


def sv_accept_sampled(logits, draft, parents, tree_err, u_accept, u_sample, temperature,
                      accepted_len, accepted_nodes, out_tokens, workspace, stream=None) -> None:
    B, T = parents.shape
    V = logits.shape[-1]
    rc = load_library().sv_accept_sampled(
        _ptr(logits), _ptr(draft), _ptr(parents), _ptr(tree_err), _ptr(u_accept), _ptr(u_sample),
        float(temperature), B, T, V, _ptr(accepted_len), _ptr(accepted_nodes), _ptr(out_tokens),
        _ptr(workspace), workspace.numel() * workspace.element_size() if workspace is not None
        else 0, _stream(stream))
    _check("sv_accept_sampled", rc)


def sv_rope_tree(q, k_tree, prefix_len, depth, theta, stream=None) -> None:
    B, Hq, T, D = q.shape
    Hkv = k_tree.shape[1]
    rc = load_library().sv_rope_tree(_ptr(q), _ptr(k_tree), _ptr(prefix_len), _ptr(depth), B, Hq,
                                     Hkv, T, D, dtype_code(q), float(theta), _stream(stream))
    _check("sv_rope_tree", rc)


def sv_kv_append(k_tree, v_tree, tree_err, cache: sv_kv_cache, prefix_len, max_prefix_len,
                 stream=None) -> None:
    B, Hkv, T, D = k_tree.shape
    rc = load_library().sv_kv_append(_ptr(k_tree), _ptr(v_tree), _ptr(tree_err),
                                     ctypes.byref(cache), _ptr(prefix_len), int(max_prefix_len),
                                     B, Hkv, T, D, _stream(stream))
    _check("sv_kv_append", rc)


def sv_kv_compact(accepted_len, accepted_nodes, tree_err, cache: sv_kv_cache, prefix_len,
                  max_prefix_len, new_prefix_len, Hkv, D, stream=None) -> None:
    B, T = accepted_nodes.shape
    rc = load_library().sv_kv_compact(_ptr(accepted_len), _ptr(accepted_nodes), _ptr(tree_err),
                                      ctypes.byref(cache), _ptr(prefix_len), int(max_prefix_len),
                                      _ptr(new_prefix_len), B, int(Hkv), T, int(D),
                                      _stream(stream))
    _check("sv_kv_compact", rc)


def sv_topk_logprobs(logits, K, top_tokens, top_logp, stream=None) -> None:
    """logits float32 [..., V] -> top_tokens int32 / top_logp float64 [..., K]."""
    V = logits.shape[-1]
    R = logits.numel() // V if V else 0
    rc = load_library().sv_topk_logprobs(_ptr(logits), R, V, int(K), _ptr(top_tokens),
                                         _ptr(top_logp), _stream(stream))
    _check("sv_topk_logprobs", rc)


def sv_draft_tree_workspace_size(B, T, K) -> int:
    return int(load_library().sv_draft_tree_workspace_size(B, T, K))


def sv_draft_tree(drafter_logits, root_token, K, max_levels, parents, tokens, cum_logp,
                  workspace, stream=None) -> None:
    B, T, V = drafter_logits.shape
    rc = load_library().sv_draft_tree(
        _ptr(drafter_logits), _ptr(root_token), B, T, V, int(K), int(max_levels), _ptr(parents),
        _ptr(tokens), _ptr(cum_logp), _ptr(workspace),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check("sv_draft_tree", rc)


def sv_kv_commit(k_tree, v_tree, accepted_len, accepted_nodes, tree_err, cache: sv_kv_cache,
                 prefix_len, max_prefix_len, new_prefix_len, stream=None) -> None:
    B, Hkv, T, D = k_tree.shape
    rc = load_library().sv_kv_commit(
        _ptr(k_tree), _ptr(v_tree), _ptr(accepted_len), _ptr(accepted_nodes), _ptr(tree_err),
        ctypes.byref(cache), _ptr(prefix_len), int(max_prefix_len), _ptr(new_prefix_len), B,
        Hkv, T, D, _stream(stream))
    _check("sv_kv_commit", rc)


def sv_status_string(code: int) -> str:
    return load_library().sv_status_string(code).decode()


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled device byte buffer of at least nbytes (256-byte aligned by the
    allocator); the attention call needs the start of its workspace zero before first use."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)
