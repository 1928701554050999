"""One workspace across attention calls of different shapes and plans, through the C ABI.

The chunk merge inside the attention kernel keeps arrival counters in the first 256 KiB of
the workspace: they must be zero before a call and every call must leave them zero, whatever
the shapes of the calls before it.  Here one zero-filled workspace serves, in turn, calls
whose chunks are merged inside the kernel (several chunks per sequence, with partials;
balanced and explicit splits), calls whose one chunk per sequence is written directly,
calls merged by the separate kernel (small splits, head_dim 512), at head_dim 128 and 256,
and fp32 calls on the vector-ALU kernel (merged inside it, or one chunk written directly).
After every call the counters are read back (all zero) and the output is compared with the
oracle's, every row.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import tree_masked_verify_amd as sv
from parity import ATOL, REL_RMS, attention_error, host_copy
from tree_masked_verify_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
COUNTER_BYTES = 256 * 1024


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _cases():
    long = wl.WORKLOADS["long32k"]
    return [
        # several chunks per sequence merged inside the kernel, balanced chunk lengths
        (wl.scaled(long, name="ws-fused", B=8, prefix=(900, 1400), V=11), 60, 0),
        # one chunk per sequence on a full grid: the output is written directly
        (wl.scaled(long, name="ws-direct", B=32, T=8, max_levels=4, prefix=(200, 400), V=11),
         61, 0),
        # the separate merge kernel (a small call split into many chunks)
        (wl.WORKLOADS["parity512"], 62, 0),
        # head_dim 128, explicit splits merged inside the kernel
        (wl.scaled(long, name="ws-fused-d128", B=12, D=128, prefix=(900, 1400), V=11), 63, 3),
        # head_dim 128, written directly
        (wl.scaled(long, name="ws-direct-d128", B=32, T=8, max_levels=4, D=128,
                   prefix=(200, 400), V=11), 64, 0),
        # fp32 on the vector ALUs: chunks merged inside the kernel, and one chunk written
        # directly
        (wl.scaled(wl.WORKLOADS["tiny"], name="ws-f32", B=4, prefix=(100, 300)), 67, 0),
        (wl.WORKLOADS["tiny"], 68, 1),
        # head_dim 512 (separate merge), then the first shape again on the used workspace
        (wl.WORKLOADS["chain2k"], 65, 0),
        (wl.scaled(long, name="ws-fused-again", B=8, prefix=(900, 1400), V=11), 66, 0),
    ]


def test_one_workspace_across_shapes():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    orc = O.Oracle()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)
    for w, seed, splits in _cases():
        inp = wl.make_inputs(w, seed=seed, device=DEV)
        B, Hq, T, D = inp.q.shape
        need = sv.sv_tree_verify_attention_workspace_size(
            B, Hq, w.Hkv, T, D, inp.max_prefix_len, sv.dtype_code(inp.q), splits)
        _say(f"[case] {w.name} B={B} Hq={Hq} Hkv={w.Hkv} T={T} D={D} P<={inp.max_prefix_len} "
             f"splits={splits} workspace={need}")
        assert 0 < need <= ws.numel()
        h = host_copy(inp)
        mask = torch.zeros((B, T, (T + 63) // 64), dtype=torch.int64, device=DEV)
        depth = torch.zeros((B, T), dtype=torch.int32, device=DEV)
        err = torch.zeros((B,), dtype=torch.int32, device=DEV)
        sv.sv_build_tree_mask(inp.parents, mask, depth, err)
        out = torch.full((B, T, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        cache = sv.make_cache(inp.k_pool, inp.v_pool, inp.block_table)
        sv.sv_tree_verify_attention(inp.q, inp.k_tree, inp.v_tree, cache, inp.prefix_len,
                                    inp.max_prefix_len, mask, inp.scale, out, ws, splits)
        torch.cuda.synchronize()
        left = int(torch.count_nonzero(ws[:COUNTER_BYTES]).item())
        assert left == 0, f"{w.name}: {left} counter bytes left non-zero"
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got)), f"{w.name}: non-finite output"
        want = orc.tree_verify_attention(h["q"], h["k_tree"], h["v_tree"], h["cache"],
                                         h["prefix"], inp.max_prefix_len,
                                         orc.build_tree_mask(h["parents"])[0], inp.scale)
        mx, rel = attention_error(got, want)
        _say(f"       max-abs {mx:.2e}, relative RMS {rel:.2e}")
        assert mx <= ATOL and rel <= REL_RMS, (w.name, mx, rel)
