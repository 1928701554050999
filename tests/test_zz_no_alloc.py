"""The allocation-free attention entry point (sv_tree_verify_attention_noalloc) against
the workspace entry point on the same inputs, through the C ABI: two calls in a row, the
second on a smaller input (so the second reuses scratch the first left behind), each
output compared byte for byte with the workspace entry point's, and the smaller one also
against the oracle.  A call larger than the scratch is refused before any launch."""
import sys

import pytest
import torch

import oracle as O
import tree_masked_verify_amd as sv
from parity import ATOL, REL_RMS, attention_error, host_copy
from tree_masked_verify_amd import workloads as wl
from tree_masked_verify_amd.step import VerifyStep

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(inp):
    """(workspace entry output, allocation-free entry output) for the same call."""
    st = VerifyStep.from_inputs(inp)
    st.build_mask()
    st.attention()
    ref = st.out.clone()
    got = torch.full_like(st.out, float("nan"))
    sv.sv_tree_verify_attention_noalloc(st.q, st.k_tree, st.v_tree, st.cache, st.prefix_len,
                                        st.max_prefix_len, st.mask, st.scale, got)
    torch.cuda.synchronize()
    return st, ref, got


def test_noalloc_matches_workspace_entry():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    orc = O.Oracle()
    cases = [
        # chunks merged inside the kernel (several per sequence), partials in the scratch
        (wl.scaled(wl.WORKLOADS["long32k"], name="na-long", B=4, prefix=(2500, 3100), V=997), 50),
        # smaller: one sequence, the 504 + 8 parity shape
        (wl.WORKLOADS["parity512"], 51),
    ]
    for w, seed in cases:
        _say(f"[case] noalloc {w.name} B={w.B} D={w.D}")
        inp = wl.make_inputs(w, seed=seed, device=DEV)
        h = host_copy(inp)
        st, ref, got = _both(inp)
        assert torch.equal(ref, got), f"{w.name}: outputs differ"
    # the smaller call against the oracle as well
    o = orc.tree_verify_attention(h["q"], h["k_tree"], h["v_tree"], h["cache"], h["prefix"],
                                  inp.max_prefix_len, orc.build_tree_mask(h["parents"])[0],
                                  inp.scale)
    mx, rel = attention_error(got.cpu().numpy(), o)
    assert mx <= ATOL and rel <= REL_RMS, (mx, rel)


def test_noalloc_head_dim_512_and_vector_alu():
    """head_dim 512 on the matrix cores (partials in the scratch, merged by the separate
    kernel) and fp32 on the vector ALUs (merged inside its kernel, with the arrival
    counters at the start of the scratch); again two calls, larger first."""
    for w, seed in [(wl.WORKLOADS["chain2k"], 52), (wl.WORKLOADS["tiny"], 53)]:
        _say(f"[case] noalloc {w.name} D={w.D} {w.dtype}")
        inp = wl.make_inputs(w, seed=seed, device=DEV)
        st, ref, got = _both(inp)
        assert torch.equal(ref, got), f"{w.name}: outputs differ"


def test_noalloc_refuses_beyond_scratch():
    """A call whose workspace would exceed the 64 MiB scratch returns SV_ERR_SCRATCH."""
    w = wl.scaled(wl.WORKLOADS["long32k"], name="na-big", B=24, prefix=(40000, 40000), V=11,
                  T=60)
    need = sv.sv_tree_verify_attention_workspace_size(w.B, w.Hq, w.Hkv, w.T, w.D, 40000,
                                                      sv.SV_BF16)
    assert need > (64 << 20)
    lib = sv.load_library()
    c = sv.sv_kv_cache(k=0x10000, v=0x10000, block_table=0x10000, block_size=16,
                       max_blocks_per_seq=2600, num_blocks=100000, block_stride=8 * 16 * 256,
                       head_stride=16 * 256, row_stride=256, dtype=sv.SV_BF16)
    rc = lib.sv_tree_verify_attention_noalloc(0x10000, 0x10000, 0x10000, c, 0x10000, 40000,
                                              0x10000, w.B, w.Hq, w.Hkv, w.T, w.D, 0.0625,
                                              0x10000, 0, None)
    assert rc == -12, rc
