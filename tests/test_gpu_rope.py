"""GPU parity of the tree-position rotary embedding: sv_rope_tree through the C ABI
against the oracle, on the depths sv_build_tree_mask produces.

Both sides evaluate angles, cosines, sines and the rotation in fp64 and round once to
the tensor's type, so at ordinary positions the results agree bit for bit except where
the two fp64 power, sine and cosine implementations differ in their last bit right at a
rounding boundary: at most 1 ulp of the output type, in at most 1e-4 of the elements.
At positions near 2^31 a last-bit difference of a frequency moves the angle by up to
~pos * 2^-52 rad (~5e-7), so there the check is absolute: 1e-5 (the pages' gate for
this rotation is 1e-4 absolute), plus one ulp of the output type.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import tree_masked_verify_amd as sv
from _support import to_np
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


def ulp_diff(a: np.ndarray, b: np.ndarray, bf16: bool) -> np.ndarray:
    """Distance in units in the last place between same-typed arrays (bit patterns)."""
    if bf16:
        ia, ib = a.view(np.int16).astype(np.int64), b.view(np.int16).astype(np.int64)
        flip = lambda x: np.where(x < 0, -32768 - x, x)
    else:
        ia, ib = a.view(np.int32).astype(np.int64), b.view(np.int32).astype(np.int64)
        flip = lambda x: np.where(x < 0, -(1 << 31) - x, x)
    return np.abs(flip(ia) - flip(ib))


def check(orc, inp, theta, prefix=None, label="", large=False):
    w = inp.w
    B, T = inp.parents.shape
    bf16 = w.dtype == "bf16"
    _say(f"[case] rope {label} B={B} Hq={w.Hq} Hkv={w.Hkv} T={T} D={w.D} {w.dtype} theta={theta}")
    prefix_t = inp.prefix_len if prefix is None else torch.tensor(prefix, dtype=torch.int32, device=DEV)
    q0, k0 = to_np(inp.q), to_np(inp.k_tree)
    mask = torch.zeros((B, T, 1), dtype=torch.int64, device=DEV)
    depth = torch.zeros((B, T), dtype=torch.int32, device=DEV)
    err = torch.zeros((B,), dtype=torch.int32, device=DEV)
    sv.sv_build_tree_mask(inp.parents, mask, depth, err)
    sv.sv_rope_tree(inp.q, inp.k_tree, prefix_t, depth, theta)
    torch.cuda.synchronize()
    _, odepth, _ = orc.build_tree_mask(to_np(inp.parents))
    assert np.array_equal(to_np(depth), odepth)
    qo, ko = orc.rope_tree(q0, k0, to_np(prefix_t), odepth, theta, O.BF16 if bf16 else O.F32)
    n_off = 0
    worst = 0.0
    for got, want in ((to_np(inp.q), qo), (to_np(inp.k_tree), ko)):
        d = ulp_diff(got, want, bf16)
        n_off += int((d > 0).sum())
        if large:
            g = (got.astype(np.uint32) << 16).view(np.float32) if bf16 else got
            t = (want.astype(np.uint32) << 16).view(np.float32) if bf16 else want
            g, t = g.astype(np.float64), t.astype(np.float64)
            ulp = np.abs(t) * (2.0 ** -7 if bf16 else 2.0 ** -23)   # >= one ulp of t
            err = np.abs(g - t) - ulp
            worst = max(worst, float(err.max()))
            assert err.max() <= 1e-5, f"{label}: absolute error {err.max()}"
        else:
            assert d.max() <= 1, f"{label}: {int(d.max())} ulp"
    n = q0.size + k0.size
    if large:
        _say(f"       {n_off} of {n} elements differ; worst absolute error beyond 1 ulp {worst:.2e}")
    else:
        assert n_off <= max(1, n * 1e-4), f"{label}: {n_off} of {n} elements off by 1 ulp"
        _say(f"       {n_off} of {n} elements 1 ulp apart, the rest identical")


@pytest.mark.parametrize("name", ["tiny", "parity512", "chain2k"])
def test_workload_shapes(orc, name):
    inp = wl.make_inputs(wl.WORKLOADS[name], seed=1, device=DEV)
    check(orc, inp, 1e4, label=name)


def test_long32k_full_size(orc):
    inp = wl.make_inputs(wl.WORKLOADS["long32k"], seed=2, device=DEV, with_logits=False)
    check(orc, inp, 1e6, label="long32k")


@pytest.mark.parametrize("D", [128, 2, 64])
def test_head_dims(orc, D):
    w = wl.scaled(wl.WORKLOADS["parity512"], D=D, B=3, name=f"parity512-d{D}")
    check(orc, wl.make_inputs(w, seed=D, device=DEV, with_logits=False), 1e4, label=w.name)


def test_large_positions_and_thetas(orc):
    """Positions near 2^31 (an fp32 angle would be off by ~1e-3 rad there) and several
    bases, on fp32 and bf16 tensors."""
    for dtype in ("f32", "bf16"):
        w = wl.scaled(wl.WORKLOADS["parity512"], B=3, dtype=dtype, name=f"parity512-{dtype}")
        inp = wl.make_inputs(w, seed=7, device=DEV, with_logits=False)
        check(orc, inp, 5e5, prefix=[0, 2_000_000_000, 123_456_789], label=w.name + " large",
              large=True)
        inp = wl.make_inputs(w, seed=8, device=DEV, with_logits=False)
        check(orc, inp, 10.0, label=w.name + " theta 10")


def test_unaligned_tensors(orc):
    """Q and tree keys that start one element past a 16-byte boundary take the
    element-wise form; the same data at aligned addresses the 16-byte one."""
    for dtype in ("bf16", "f32"):
        w = wl.scaled(wl.WORKLOADS["parity512"], B=2, dtype=dtype, name=f"unaligned-{dtype}")
        inp = wl.make_inputs(w, seed=11, device=DEV, with_logits=False)
        for name in ("q", "k_tree"):
            t = getattr(inp, name)
            buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=DEV)
            view = buf[1:1 + t.numel()].view(t.shape)
            view.copy_(t)
            assert view.data_ptr() % 16 != 0
            setattr(inp, name, view)
        check(orc, inp, 1e4, label=w.name)
