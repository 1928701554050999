"""The C ABI on the CPU: the library loads, exports every entry point include/sv.h
declares, and rejects bad arguments on the host before anything reaches a GPU.
(No call here gets past validation, so none launches a kernel.)"""
import ctypes
import os
import re

import pytest

import tree_masked_verify_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")

FAKE = 0x10000  # a 16-byte aligned non-NULL address; never dereferenced by these calls


@pytest.fixture(scope="module")
def lib():
    return sv.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(sv.ENTRY_POINTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in sv.STATUS.items():
        s = sv.sv_status_string(code)
        assert s and s != "unknown status", (code, s)
    assert sv.sv_status_string(12345) == "unknown status"


def test_mask_validation(lib):
    f = lib.sv_build_tree_mask
    assert f(FAKE, 2, 0, FAKE, None, FAKE, None) == -6
    assert f(FAKE, 2, 65, FAKE, None, FAKE, None) == -6
    assert f(FAKE, -1, 8, FAKE, None, FAKE, None) == -2
    assert f(None, 0, 8, None, None, None, None) == 0       # nothing to do
    assert f(None, 2, 8, FAKE, None, FAKE, None) == -1
    assert f(FAKE, 2, 8, FAKE, None, None, None) == -1


def cache(**kw):
    c = dict(k=FAKE, v=FAKE, block_table=FAKE, block_size=16, max_blocks_per_seq=10,
             num_blocks=100, block_stride=2 * 16 * 256, head_stride=16 * 256, row_stride=256,
             dtype=sv.SV_BF16)
    c.update(kw)
    return sv.sv_kv_cache(**c)


def attn(lib, c=None, q=FAKE, B=2, Hq=8, Hkv=2, T=8, D=256, maxp=100, ws=FAKE, wsb=1 << 30,
         splits=0, out=FAKE, null_cache=False, scale=0.0625, kt=FAKE, vt=FAKE):
    c = c or cache()
    return lib.sv_tree_verify_attention(q, kt, vt, None if null_cache else ctypes.byref(c),
                                        FAKE, maxp, FAKE, B, Hq, Hkv, T, D, scale, out, ws, wsb,
                                        splits, None)


def test_noalloc_attention_validation(lib):
    """The allocation-free attention entry point shares the workspace entry point's host
    checks, and refuses a call whose workspace would exceed its 64 MiB scratch, all before
    touching the device."""
    def call(c=None, B=2, Hq=8, Hkv=2, T=8, D=256, maxp=100, splits=0, scale=0.0625):
        c = c or cache()
        return lib.sv_tree_verify_attention_noalloc(FAKE, FAKE, FAKE, ctypes.byref(c), FAKE,
                                                    maxp, FAKE, B, Hq, Hkv, T, D, scale, FAKE,
                                                    splits, None)
    assert lib.sv_tree_verify_attention_noalloc(FAKE, FAKE, FAKE, None, FAKE, 10, FAKE, 2, 8, 2,
                                                8, 256, 0.0625, FAKE, 0, None) == -1
    assert call(Hkv=0) == -4 and call(D=64) == -5 and call(T=65) == -6
    assert call(maxp=153) == -7 and call(scale=0.0) == -2
    assert call(B=0) == 0
    big = cache(max_blocks_per_seq=2600, num_blocks=100000, block_stride=8 * 16 * 256)
    assert sv.sv_tree_verify_attention_workspace_size(24, 32, 8, 60, 256, 40000, sv.SV_BF16) > (64 << 20)
    assert call(c=big, B=24, Hq=32, Hkv=8, T=60, maxp=40000) == -12
    assert "64 MiB" in sv.sv_status_string(-12)


def test_attention_validation(lib):
    assert attn(lib, null_cache=True) == -1
    assert attn(lib, Hkv=0) == -4
    assert attn(lib, Hq=0) == -4
    assert attn(lib, Hq=6, Hkv=4) == -4
    assert attn(lib, D=64) == -5 and attn(lib, D=100) == -5 and attn(lib, D=1024) == -5
    assert attn(lib, T=0) == -6 and attn(lib, T=65) == -6
    assert attn(lib, B=-1) == -2 and attn(lib, maxp=-1) == -2 and attn(lib, splits=-2) == -2
    assert attn(lib, c=cache(dtype=9)) == -3
    assert attn(lib, c=cache(block_size=8)) == -2
    assert attn(lib, c=cache(num_blocks=0)) == -2
    assert attn(lib, maxp=153) == -7                  # 153 + 8 > 10 * 16
    assert attn(lib, maxp=152, ws=None) == -9         # exactly at capacity, but no workspace
    assert attn(lib, wsb=16) == -9
    assert attn(lib, q=FAKE + 2) == -11
    assert attn(lib, out=FAKE + 4) == -11
    assert attn(lib, c=cache(row_stride=260)) == -11
    assert attn(lib, c=cache(k=FAKE + 8)) == -11
    assert attn(lib, ws=FAKE + 16) == -11             # workspace must be 256-byte aligned
    assert attn(lib, B=0, null_cache=False) == 0
    assert attn(lib, c=cache(block_table=None)) == -1
    assert attn(lib, c=cache(num_blocks=1 << 62, block_stride=1 << 20)) == -8
    assert attn(lib, scale=0.0) == -2 and attn(lib, scale=-1.0) == -2
    assert attn(lib, scale=float("inf")) == -2 and attn(lib, scale=float("nan")) == -2
    # tree rows in the cache: both tree buffers NULL, never just one
    assert attn(lib, kt=None) == -1 and attn(lib, vt=None) == -1
    assert attn(lib, kt=None, vt=None, ws=None) == -9      # both NULL passes the NULL check
    assert attn(lib, kt=FAKE + 8) == -11


def test_attention_workspace_size(lib):
    f = sv.sv_tree_verify_attention_workspace_size
    a = f(16, 32, 8, 60, 256, 32768, sv.SV_BF16)
    b = f(16, 32, 8, 60, 256, 32768, sv.SV_BF16, 4)
    assert a > 0 and b > 0
    assert b >= 16 * 8 * 4 * 240 * 256 * 4            # 4 chunks of fp32 partials per row
    assert f(16, 32, 0, 60, 256, 32768, sv.SV_BF16) == 0
    assert f(16, 32, 8, 60, 64, 32768, sv.SV_BF16) == 0
    assert f(16, 32, 8, 60, 128, 32768, sv.SV_BF16) > 0   # head_dim 128 is supported
    assert f(1, 1, 1, 1, 256, 0, sv.SV_F32) > 0
    # a full grid of one chunk per sequence writes its output directly: only the merge's
    # arrival counters and the header remain; head_dim 512 still stores its partials
    assert f(32, 32, 4, 64, 256, 8192, sv.SV_BF16) == 256 * 1024 + 256
    assert f(32, 32, 4, 64, 512, 8192, sv.SV_BF16) >= 32 * 4 * 512 * 512 * 4


def test_accept_validation(lib):
    f = lib.sv_accept_longest_path
    args = lambda B=2, T=8, V=1000, lg=FAKE, ws=FAKE, wsb=1 << 30: (
        lg, FAKE, FAKE, None, B, T, V, None, FAKE, FAKE, FAKE, ws, wsb, None)
    assert f(*args(V=0)) == -2
    assert f(*args(B=-3)) == -2
    assert f(*args(T=0)) == -6 and f(*args(T=65)) == -6
    assert f(*args(V=1 << 31)) == -8
    assert f(*args(lg=None)) == -1
    assert f(*args(lg=FAKE + 2)) == -11
    assert f(*args(wsb=8)) == -9
    assert f(*args(ws=None)) == -9
    assert f(*args(B=0)) == 0
    assert sv.sv_accept_longest_path_workspace_size(2, 8, 1000) > 0
    assert sv.sv_accept_longest_path_workspace_size(2, 0, 1000) == 0
    # rows cut into chunks of at most 16384 logits: one (value, index) pair per row and chunk
    assert sv.sv_accept_longest_path_workspace_size(1, 1, 151936) >= 10 * 8
    # one workgroup per row and chunk: 2^26 rows of 31 chunks fit in 2^31 - 1 workgroups,
    # 33 chunks do not (size 0: the plan is refused)
    assert sv.sv_accept_longest_path_workspace_size(1 << 20, 64, 16384 * 31) > 0
    assert sv.sv_accept_longest_path_workspace_size(1 << 20, 64, 16384 * 33) == 0


def test_accept_sampled_validation(lib):
    f = lib.sv_accept_sampled
    args = lambda B=2, T=8, V=1000, lg=FAKE, ua=FAKE, tau=0.5, ws=FAKE, wsb=1 << 30: (
        lg, FAKE, FAKE, None, ua, FAKE, tau, B, T, V, FAKE, FAKE, FAKE, ws, wsb, None)
    assert f(*args(V=0)) == -2
    assert f(*args(B=-3)) == -2
    assert f(*args(tau=0.0)) == -2 and f(*args(tau=-1.0)) == -2
    assert f(*args(tau=float("inf"))) == -2 and f(*args(tau=float("nan"))) == -2
    assert f(*args(T=0)) == -6 and f(*args(T=65)) == -6
    assert f(*args(V=1 << 31)) == -8
    assert f(*args(lg=None)) == -1 and f(*args(ua=None)) == -1
    assert f(*args(lg=FAKE + 2)) == -11
    assert f(*args(wsb=8)) == -9
    assert f(*args(ws=None)) == -9
    assert f(*args(B=0)) == 0
    assert sv.sv_accept_sampled_workspace_size(2, 8, 1000) > 0
    assert sv.sv_accept_sampled_workspace_size(2, 0, 1000) == 0
    # chunks of at most 16384 elements: (max, sum) per row and chunk
    assert sv.sv_accept_sampled_workspace_size(1, 1, 151936) >= 10 * 8
    assert sv.sv_accept_sampled_workspace_size(1 << 20, 64, 16384 * 31) > 0
    assert sv.sv_accept_sampled_workspace_size(1 << 20, 64, 16384 * 33) == 0


def test_rope_validation(lib):
    f = lib.sv_rope_tree
    args = lambda B=2, Hq=4, Hkv=2, T=8, D=128, dt=sv.SV_BF16, th=1e4, q=FAKE: (
        q, FAKE, FAKE, FAKE, B, Hq, Hkv, T, D, dt, th, None)
    assert f(*args(D=127)) == -2 and f(*args(D=0)) == -2 and f(*args(D=2048)) == -2
    assert f(*args(th=0.0)) == -2 and f(*args(th=-1.0)) == -2
    assert f(*args(th=float("inf"))) == -2 and f(*args(th=float("nan"))) == -2
    assert f(*args(Hq=0)) == -2 and f(*args(Hkv=0)) == -2 and f(*args(B=-1)) == -2
    assert f(*args(T=0)) == -6 and f(*args(T=65)) == -6
    assert f(*args(dt=3)) == -3
    assert f(*args(q=None)) == -1
    assert f(*args(q=FAKE + 1)) == -11 and f(*args(q=FAKE + 2, dt=sv.SV_F32)) == -11
    assert f(*args(B=0)) == 0


def test_commit_validation(lib):
    f = lib.sv_kv_commit
    def call(c=None, Hkv=2, T=8, D=256, maxp=100, kt=FAKE, B=2):
        c = c or cache()
        return f(kt, FAKE, FAKE, FAKE, None, ctypes.byref(c), FAKE, maxp, None, B, Hkv, T, D,
                 None)
    assert f(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1, None, 2, 2, 8, 256, None) == -1
    assert call(Hkv=0) == -4
    assert call(T=70) == -6
    assert call(D=100) == -5
    assert call(c=cache(dtype=3)) == -3
    assert call(maxp=153) == -7
    assert call(maxp=-1) == -2
    assert call(kt=FAKE + 2) == -11
    assert call(kt=None) == -1
    assert call(B=0) == 0


def test_topk_validation(lib):
    f = lib.sv_topk_logprobs
    args = lambda R=4, V=1000, K=8, lg=FAKE, tk=FAKE, lp=FAKE: (lg, R, V, K, tk, lp, None)
    assert f(*args(K=0)) == -2 and f(*args(K=65)) == -2 and f(*args(V=5, K=6)) == -2
    assert f(*args(R=-1)) == -2 and f(*args(V=0)) == -2
    assert f(*args(V=1 << 31)) == -8 and f(*args(R=1 << 31)) == -8
    assert f(*args(R=0, lg=None, tk=None, lp=None)) == 0          # nothing to do
    assert f(*args(lg=None)) == -1 and f(*args(lp=None)) == -1
    assert f(*args(lg=FAKE + 2)) == -11 and f(*args(lp=FAKE + 4)) == -11
    assert f(*args(tk=FAKE + 2)) == -11


def test_draft_tree_validation(lib):
    f = lib.sv_draft_tree
    args = lambda B=2, T=8, V=1000, K=4, lv=4, dl=FAKE, cum=FAKE, ws=FAKE, wsb=1 << 20: (
        dl, FAKE, B, T, V, K, lv, FAKE, FAKE, cum, ws, wsb, None)
    assert f(*args(T=0)) == -6 and f(*args(T=65)) == -6
    assert f(*args(K=0)) == -2 and f(*args(K=65)) == -2 and f(*args(V=3)) == -2
    assert f(*args(lv=0)) == -2 and f(*args(B=-1)) == -2
    # a full binary tree of 3 levels has 7 nodes; a chain of K = 1 has max_levels nodes
    assert f(*args(K=2, lv=3)) == -2 and f(*args(K=1, lv=7)) == -2
    assert f(*args(V=1 << 31)) == -8
    assert f(*args(B=0)) == 0
    assert f(*args(dl=None)) == -1
    assert f(*args(cum=FAKE + 4)) == -11 and f(*args(dl=FAKE + 2)) == -11
    assert f(*args(wsb=16)) == -9 and f(*args(ws=None)) == -9
    assert f(*args(ws=FAKE + 8)) == -11
    ws = sv.sv_draft_tree_workspace_size
    assert ws(2, 8, 4) == 512 + 256     # [2][7][4] fp64 log-probs, then int32 tokens
    assert ws(2, 1, 4) == 0 and ws(-1, 8, 4) == 0 and ws(2, 65, 4) == 0 and ws(2, 8, 65) == 0


def test_append_compact_validation(lib):
    fa, fc = lib.sv_kv_append, lib.sv_kv_compact
    def app(c=None, Hkv=2, T=8, D=256, maxp=100, kt=FAKE, err=FAKE, B=2):
        c = c or cache()
        return fa(kt, FAKE, err, ctypes.byref(c), FAKE, maxp, B, Hkv, T, D, None)
    def cmp(c=None, Hkv=2, T=8, D=256, maxp=100, L=FAKE, B=2):
        c = c or cache()
        return fc(L, FAKE, None, ctypes.byref(c), FAKE, maxp, None, B, Hkv, T, D, None)
    assert fa(FAKE, FAKE, FAKE, None, FAKE, 1, 2, 2, 8, 256, None) == -1
    assert fc(FAKE, FAKE, None, None, FAKE, 1, None, 2, 2, 8, 256, None) == -1
    for f in (app, cmp):
        assert f(Hkv=0) == -4 and f(T=0) == -6 and f(T=65) == -6 and f(D=100) == -5
        assert f(c=cache(dtype=3)) == -3 and f(maxp=153) == -7 and f(maxp=-1) == -2
        assert f(B=-1) == -2 and f(B=0) == 0
        assert f(c=cache(k=FAKE + 8)) == -11
    assert app(kt=FAKE + 2) == -11 and app(kt=None) == -1 and app(err=None) == -1
    assert cmp(L=None) == -1


# ----------------------------------------------------------------------------- fuzzing
# Random (often extreme) sizes through every size query and every entry point.  Each
# entry-point call leaves one required pointer NULL, so no call may get past the host
# checks: it returns a negative status, or 0 for an empty batch (nothing enqueued).  Under
# the sanitizer build (test_sanitizers.py) this also checks the host code's size
# arithmetic for overflow and out-of-bounds reads.
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

I32 = st.one_of(st.integers(-3, 70), st.sampled_from([128, 256, 512, 1000, 1024, 4096, 65536,
                                                      1 << 20, (1 << 31) - 1, -(1 << 31)]),
                st.integers(-(1 << 31), (1 << 31) - 1))
I64 = st.one_of(I32, st.sampled_from([1 << 32, 1 << 40, (1 << 62), (1 << 63) - 1, -(1 << 63)]))
FUZZ = settings(max_examples=150, deadline=None,
                suppress_health_check=[HealthCheck.function_scoped_fixture])


def _ok_or_empty(rc, *sizes):
    assert rc < 0 or (rc == 0 and min(sizes) <= 0), (rc, sizes)


@FUZZ
@given(B=I32, Hq=I32, Hkv=I32, T=I32, D=I32, P=I32, dt=st.integers(-2, 4), splits=I32,
       V=I64, K=I32)
def test_fuzz_workspace_sizes(lib, B, Hq, Hkv, T, D, P, dt, splits, V, K):
    n = lib.sv_tree_verify_attention_workspace_size(B, Hq, Hkv, T, D, P, dt, splits)
    assert n == 0 or (n >= 256 * 1024 + 256 and n % 256 == 0), n
    for f in (lib.sv_accept_longest_path_workspace_size, lib.sv_accept_sampled_workspace_size):
        assert f(B, T, V) >= 0
    assert lib.sv_draft_tree_workspace_size(B, T, K) >= 0


@FUZZ
@given(B=I32, Hq=I32, Hkv=I32, T=I32, D=I32, P=I32, splits=I32, bs=I32, mbs=I32, nb=I64,
       bstr=I64, hstr=I64, rstr=I64, dt=st.integers(-2, 4), which=st.integers(0, 2))
def test_fuzz_attention_rejects(lib, B, Hq, Hkv, T, D, P, splits, bs, mbs, nb, bstr, hstr, rstr,
                                dt, which):
    c = sv.sv_kv_cache(k=FAKE, v=FAKE, block_table=FAKE, block_size=bs, max_blocks_per_seq=mbs,
                       num_blocks=nb, block_stride=bstr, head_stride=hstr, row_stride=rstr,
                       dtype=dt)
    q, out, mask = (None if which == 0 else FAKE, None if which == 1 else FAKE,
                    None if which == 2 else FAKE)
    rc = lib.sv_tree_verify_attention(q, FAKE, FAKE, ctypes.byref(c), FAKE, P, mask, B, Hq, Hkv,
                                      T, D, 0.0625, out, FAKE, 1 << 40, splits, None)
    _ok_or_empty(rc, B)
    rc = lib.sv_tree_verify_attention_noalloc(q, FAKE, FAKE, ctypes.byref(c), FAKE, P, mask, B,
                                              Hq, Hkv, T, D, 0.0625, out, splits, None)
    _ok_or_empty(rc, B)


@FUZZ
@given(B=I32, Hq=I32, Hkv=I32, T=I32, D=I32, P=I32, V=I64, K=I32, lv=I32, bs=I32, mbs=I32,
       nb=I64, dt=st.integers(-2, 4), temp=st.floats(allow_nan=True, allow_infinity=True))
def test_fuzz_entry_points_reject(lib, B, Hq, Hkv, T, D, P, V, K, lv, bs, mbs, nb, dt, temp):
    c = sv.sv_kv_cache(k=FAKE, v=FAKE, block_table=FAKE, block_size=bs, max_blocks_per_seq=mbs,
                       num_blocks=nb, block_stride=(1 << 20), head_stride=(1 << 12),
                       row_stride=256, dtype=dt)
    cr = ctypes.byref(c)
    _ok_or_empty(lib.sv_build_tree_mask(None, B, T, FAKE, FAKE, FAKE, None), B)
    _ok_or_empty(lib.sv_accept_longest_path(None, FAKE, FAKE, None, B, T, V, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, 1 << 40, None), B)
    _ok_or_empty(lib.sv_accept_sampled(None, FAKE, FAKE, None, FAKE, FAKE, temp, B, T, V, FAKE,
                                       FAKE, FAKE, FAKE, 1 << 40, None), B)
    _ok_or_empty(lib.sv_rope_tree(None, FAKE, FAKE, FAKE, B, Hq, Hkv, T, D, dt, 10000.0, None),
                 B)
    _ok_or_empty(lib.sv_kv_append(None, FAKE, FAKE, cr, FAKE, P, B, Hkv, T, D, None), B)
    _ok_or_empty(lib.sv_kv_compact(None, FAKE, FAKE, cr, FAKE, P, FAKE, B, Hkv, T, D, None), B)
    _ok_or_empty(lib.sv_kv_commit(None, FAKE, FAKE, FAKE, FAKE, cr, FAKE, P, FAKE, B, Hkv, T, D,
                                  None), B)
    _ok_or_empty(lib.sv_topk_logprobs(None, B, V, K, FAKE, FAKE, None), B)
    _ok_or_empty(lib.sv_draft_tree(None, FAKE, B, T, V, K, lv, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                   None), B)


def test_entry_point_imports_resolve():
    """Every `from M import a, b` inside the functions of __graft_entry__.py (the build
    and smoke entry points) names something M defines, so that the smoke run does not
    fail on a helper that moved.  Checked on the CPU by importing M, without running
    anything on a GPU."""
    import ast
    import importlib

    with open(os.path.join(ROOT, "__graft_entry__.py")) as f:
        src = f.read()
    missing = []
    for fn in ast.parse(src).body:
        if not isinstance(fn, ast.FunctionDef):
            continue
        for node in ast.walk(fn):
            if isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                mod = importlib.import_module(node.module)
                for a in node.names:
                    if hasattr(mod, a.name):
                        continue
                    try:  # a submodule
                        importlib.import_module(f"{node.module}.{a.name}")
                    except ImportError:
                        missing.append(f"{node.module}.{a.name}")
    assert not missing, missing
