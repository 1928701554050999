"""One verify step over resident device tensors: the four library calls in stream order.

Allocation (outputs, workspaces) happens once in the constructor through torch; run()
only enqueues sv_build_tree_mask -> sv_tree_verify_attention ->
sv_accept_longest_path -> sv_kv_commit on one stream.  accept_sampled() enqueues the
sampled acceptance instead of the greedy one (same outputs, which commit() reads).
run_in_cache() is the write-before-accept variant: sv_kv_append puts the tree rows into the
cache first, the attention reads them there, and sv_kv_compact replaces the commit.
"""
from __future__ import annotations

import torch

from . import (dtype_code, make_cache, sv_accept_longest_path,
               sv_accept_longest_path_workspace_size, sv_accept_sampled,
               sv_accept_sampled_workspace_size, sv_build_tree_mask, sv_kv_append,
               sv_kv_commit, sv_kv_compact, sv_tree_verify_attention,
               sv_tree_verify_attention_workspace_size, workspace)


class VerifyStep:
    def __init__(self, q, k_tree, v_tree, k_pool, v_pool, block_table, prefix_len,
                 max_prefix_len, parents, logits, draft, scale, num_splits=0,
                 new_prefix_len=None):
        self.q, self.k_tree, self.v_tree = q, k_tree, v_tree
        self.k_pool, self.v_pool, self.block_table = k_pool, v_pool, block_table
        self.prefix_len, self.max_prefix_len = prefix_len, int(max_prefix_len)
        self.parents, self.logits, self.draft = parents, logits, draft
        self.scale, self.num_splits = float(scale), int(num_splits)
        dev = q.device
        B, Hq, T, D = q.shape
        Hkv = k_tree.shape[1]
        V = logits.shape[-1]
        self.cache = make_cache(k_pool, v_pool, block_table)
        self.mask = torch.zeros((B, T, (T + 63) // 64), dtype=torch.int64, device=dev)
        self.depth = torch.zeros((B, T), dtype=torch.int32, device=dev)
        self.tree_err = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.out = torch.zeros((B, T, Hq, D), dtype=torch.float32, device=dev)
        self.argmax = torch.zeros((B, T), dtype=torch.int32, device=dev)
        self.accepted_len = torch.zeros((B,), dtype=torch.int32, device=dev)
        self.accepted_nodes = torch.zeros((B, T), dtype=torch.int32, device=dev)
        self.out_tokens = torch.zeros((B, T), dtype=torch.int32, device=dev)
        self.new_prefix_len = (torch.zeros((B,), dtype=torch.int32, device=dev)
                               if new_prefix_len is None else new_prefix_len)
        self.attn_ws = workspace(sv_tree_verify_attention_workspace_size(
            B, Hq, Hkv, T, D, self.max_prefix_len, dtype_code(q), self.num_splits), dev)
        self.acc_ws = workspace(sv_accept_longest_path_workspace_size(B, T, V), dev)
        self.smp_ws = workspace(sv_accept_sampled_workspace_size(B, T, V), dev)

    @classmethod
    def from_inputs(cls, inp, num_splits=0, new_prefix_len=None):
        return cls(inp.q, inp.k_tree, inp.v_tree, inp.k_pool, inp.v_pool, inp.block_table,
                   inp.prefix_len, inp.max_prefix_len, inp.parents, inp.logits, inp.draft,
                   inp.scale, num_splits=num_splits, new_prefix_len=new_prefix_len)

    def build_mask(self, stream=None):
        sv_build_tree_mask(self.parents, self.mask, self.depth, self.tree_err, stream)

    def attention(self, stream=None):
        sv_tree_verify_attention(self.q, self.k_tree, self.v_tree, self.cache, self.prefix_len,
                                 self.max_prefix_len, self.mask, self.scale, self.out,
                                 self.attn_ws, self.num_splits, stream)

    def accept(self, stream=None):
        sv_accept_longest_path(self.logits, self.draft, self.parents, self.tree_err,
                               self.argmax, self.accepted_len, self.accepted_nodes,
                               self.out_tokens, self.acc_ws, stream)

    def accept_sampled(self, u_accept, u_sample, temperature, stream=None):
        sv_accept_sampled(self.logits, self.draft, self.parents, self.tree_err, u_accept,
                          u_sample, temperature, self.accepted_len, self.accepted_nodes,
                          self.out_tokens, self.smp_ws, stream)

    def commit(self, stream=None):
        sv_kv_commit(self.k_tree, self.v_tree, self.accepted_len, self.accepted_nodes,
                     self.tree_err, self.cache, self.prefix_len, self.max_prefix_len,
                     self.new_prefix_len, stream)

    def run(self, stream=None):
        self.build_mask(stream)
        self.attention(stream)
        self.accept(stream)
        self.commit(stream)

    # ---- write-before-accept variant
    def append(self, stream=None):
        sv_kv_append(self.k_tree, self.v_tree, self.tree_err, self.cache, self.prefix_len,
                     self.max_prefix_len, stream)

    def attention_in_cache(self, stream=None):
        sv_tree_verify_attention(self.q, None, None, self.cache, self.prefix_len,
                                 self.max_prefix_len, self.mask, self.scale, self.out,
                                 self.attn_ws, self.num_splits, stream,
                                 Hkv=self.k_tree.shape[1])

    def compact(self, stream=None):
        sv_kv_compact(self.accepted_len, self.accepted_nodes, self.tree_err, self.cache,
                      self.prefix_len, self.max_prefix_len, self.new_prefix_len,
                      self.k_tree.shape[1], self.k_tree.shape[3], stream)

    def run_in_cache(self, stream=None):
        self.build_mask(stream)
        self.append(stream)
        self.attention_in_cache(stream)
        self.accept(stream)
        self.compact(stream)
