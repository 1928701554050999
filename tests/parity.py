"""Run one verify step through the HIP library and through the oracle on the same
inputs, and compare: masks, depths, tree errors, argmax, accepted lengths, nodes,
tokens, new prefix lengths and the whole cache pools bit for bit; attention outputs
within the floating-point tolerance."""
from __future__ import annotations

import math

import numpy as np
import torch

from _support import oracle_cache, to_np
import oracle as O
from tree_masked_verify_amd import workloads as wl
from tree_masked_verify_amd.step import VerifyStep

# Attention tolerance.  max-abs 1e-2 is the stated gate (bf16 inputs, fp32
# accumulation).  The probabilities enter the matrix cores rounded to bf16 (8
# significant bits, relative error <= 2^-8 each); the resulting relative RMS error of
# an output row stays well below 2^-6, which is checked as well.
ATOL = 1e-2
REL_RMS = 2.0 ** -6


def step_result(st: VerifyStep, inp: wl.Inputs) -> dict:
    """Every output of a step that has run, and both cache pools, on the host."""
    torch.cuda.synchronize()
    return dict(mask=to_np(st.mask).view(np.uint64), depth=to_np(st.depth),
                tree_err=to_np(st.tree_err), out=to_np(st.out), argmax=to_np(st.argmax),
                L=to_np(st.accepted_len), nodes=to_np(st.accepted_nodes),
                toks=to_np(st.out_tokens), npl=to_np(st.new_prefix_len),
                k_pool=to_np(inp.k_pool), v_pool=to_np(inp.v_pool))


def gpu_step(inp: wl.Inputs, num_splits: int = 0, repeats: int = 1):
    st = VerifyStep.from_inputs(inp, num_splits=num_splits)
    for _ in range(repeats):
        st.run()
    return step_result(st, inp)


def host_copy(inp: wl.Inputs):
    """Everything the oracle needs, copied to the host before the GPU step runs."""
    return dict(parents=to_np(inp.parents), q=to_np(inp.q), k_tree=to_np(inp.k_tree),
                v_tree=to_np(inp.v_tree), cache=oracle_cache(inp),
                prefix=to_np(inp.prefix_len), logits=to_np(inp.logits), draft=to_np(inp.draft))


def oracle_step(orc: O.Oracle, inp: wl.Inputs, h: dict, rows=None):
    mask, depth, err = orc.build_tree_mask(h["parents"])
    out = orc.tree_verify_attention(h["q"], h["k_tree"], h["v_tree"], h["cache"], h["prefix"],
                                    inp.max_prefix_len, mask, inp.scale, rows=rows)
    am, L, nodes, toks = orc.accept_longest_path(h["logits"], h["draft"], h["parents"], err)
    npl = orc.kv_commit(h["k_tree"], h["v_tree"], L, nodes, err, h["cache"], h["prefix"],
                        inp.max_prefix_len)
    return dict(mask=mask, depth=depth, tree_err=err, out=out, argmax=am, L=L, nodes=nodes,
                toks=toks, npl=npl, k_pool=h["cache"].k, v_pool=h["cache"].v)


def oracle_in_cache(orc: O.Oracle, inp: wl.Inputs, h: dict, rows=None):
    """The write-before-accept step in the oracle: append every tree row to the cache,
    attend over the cache-resident tree, accept, then compact the accepted rows."""
    w = inp.w
    mask, depth, err = orc.build_tree_mask(h["parents"])
    err = orc.kv_append(h["k_tree"], h["v_tree"], err, h["cache"], h["prefix"],
                        inp.max_prefix_len)
    out = orc.tree_verify_attention(h["q"], None, None, h["cache"], h["prefix"],
                                    inp.max_prefix_len, mask, inp.scale, rows=rows)
    am, L, nodes, toks = orc.accept_longest_path(h["logits"], h["draft"], h["parents"], err)
    npl = orc.kv_compact(L, nodes, err, h["cache"], h["prefix"], inp.max_prefix_len, w.Hkv, w.T,
                         w.D)
    return dict(mask=mask, depth=depth, tree_err=err, out=out, argmax=am, L=L, nodes=nodes,
                toks=toks, npl=npl, k_pool=h["cache"].k, v_pool=h["cache"].v)


def attention_error(got: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    err = np.abs(g - r)
    rms_ref = math.sqrt(float(np.mean(r * r))) + 1e-30
    return float(err.max()), math.sqrt(float(np.mean(err * err))) / rms_ref


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def compare(g: dict, o: dict, rows=None, check_pools: bool = True) -> dict:
    assert np.array_equal(g["tree_err"], o["tree_err"]), (g["tree_err"], o["tree_err"])
    assert np.array_equal(g["mask"], o["mask"])
    assert np.array_equal(g["depth"], o["depth"])
    assert np.array_equal(g["argmax"], o["argmax"])
    assert np.array_equal(g["L"], o["L"]), (g["L"], o["L"])
    assert np.array_equal(g["nodes"], o["nodes"])
    assert np.array_equal(g["toks"], o["toks"])
    assert np.array_equal(g["npl"], o["npl"])
    if check_pools:  # byte for byte (NaN payloads included)
        assert np.array_equal(_bits(g["k_pool"]), _bits(o["k_pool"])), "K pool differs after commit"
        assert np.array_equal(_bits(g["v_pool"]), _bits(o["v_pool"])), "V pool differs after commit"
    got = g["out"]
    assert np.all(np.isfinite(got)), "non-finite attention output"
    if rows is not None:
        got = np.stack([got[b, i, h] for b, h, i in rows])
    mx, rel = attention_error(got, o["out"])
    assert mx <= ATOL, f"attention max-abs error {mx}"
    assert rel <= REL_RMS, f"attention relative RMS error {rel}"
    return dict(max_abs=mx, rel_rms=rel)


def sample_rows(w: wl.Workload, n: int, seed: int) -> np.ndarray:
    """(b, h, i) triples: corners first (first/last sequence, head, node), then random."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = {(0, 0, 0), (w.B - 1, w.Hq - 1, w.T - 1), (0, w.Hq - 1, w.T - 1),
            (w.B - 1, 0, 0), (w.B // 2, w.Hq // 2, w.T // 2)}
    while len(rows) < n:
        rows.add((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.T))))
    return np.array(sorted(rows), dtype=np.int32)
