"""AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.

The oracle (gcc) runs all its pins, every planted mistake of test_oracle_mutants is run
against the pins again, and the host side of libsv (hipcc, host pass only; the device
code is built as usual) runs the C-ABI boundary checks, each in a subprocess with the
sanitizer runtime preloaded; any report from the real oracle or libsv fails the test, and
a mutant counts as caught by a failing pin or by a sanitizer report.  A canary -- a small
CPU library with a planted heap overflow and an oversized shift, built the same way --
shows that each harness does report.  Nothing here touches a GPU.
"""
import concurrent.futures as cf
import ctypes.util  # noqa: F401  (the subprocesses use ctypes)
import glob
import os
import subprocess
import sys
import textwrap

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

ORACLE_SRC = os.path.join(ROOT, "oracle", "sv_oracle.c")
CLANG = "/opt/rocm/llvm/bin/clang"
# host-pass sanitizers for hipcc (each flag directly after -Xarch_host)
HOST_SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
            "-Xarch_host -fno-sanitize-recover=undefined "
            "-Xarch_host -fno-omit-frame-pointer").split()
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "OMP_NUM_THREADS": "4"}

CANARY_C = textwrap.dedent("""
    #include <stdlib.h>
    int canary_overflow(int n) { int *p = malloc(sizeof(int) * n); p[0] = 1;
                                 int s = p[n]; free(p); return s; }
    int canary_shift(int x) { return 1 << x; }
""")


def _gcc_asan_runtime():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()


def _clang_asan_runtime():
    libs = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return libs[-1] if libs else None


def _run(code, preload, extra_env=None, timeout=600):
    env = {**os.environ, "LD_PRELOAD": preload, **ENV_SAN, **(extra_env or {})}
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          env=env, timeout=timeout, cwd=ROOT)


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitizers"))


def _canary(build_dir, compiler, preload):
    src = os.path.join(build_dir, "canary.c")
    with open(src, "w") as f:
        f.write(CANARY_C)
    lib = os.path.join(build_dir, f"canary_{os.path.basename(compiler)}.so")
    subprocess.run([compiler, "-O0", "-shared", "-fPIC", *GCC_SAN, src, "-o", lib], check=True)
    for fn, arg, what in (("canary_overflow", 4, "heap-buffer-overflow"),
                          ("canary_shift", 40, "shift exponent")):
        r = _run(f"import ctypes; ctypes.CDLL({lib!r}).{fn}({arg})", preload)
        assert r.returncode != 0 and what in r.stderr, (fn, r.returncode, r.stderr[-2000:])


def test_gcc_harness_reports(build_dir):
    _canary(build_dir, "gcc", _gcc_asan_runtime())


def test_oracle_pins_under_asan_ubsan(build_dir):
    lib = os.path.join(build_dir, "liboracle_asan.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                    *GCC_SAN, ORACLE_SRC, "-o", lib, "-lm"], check=True)
    code = textwrap.dedent(f"""
        import sys
        sys.path[:0] = [{HERE!r}, {ROOT!r}]
        import oracle, oracle_pins
        orc = oracle.Oracle({lib!r})
        for pin in oracle_pins.ALL_PINS:
            pin(orc)
        print("pins", len(oracle_pins.ALL_PINS))
    """)
    r = _run(code, _gcc_asan_runtime())
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert "pins" in r.stdout


def test_mutants_caught_under_asan_ubsan(build_dir):
    sys.path.insert(0, HERE)
    import test_oracle_mutants as tm
    src = open(ORACLE_SRC).read()
    runtime = _gcc_asan_runtime()

    def one(m):
        name, old, new, occ = m
        path = os.path.join(build_dir, f"mutant_{name}.c")
        with open(path, "w") as f:
            f.write(tm._mutate(src, old, new, occ))
        lib = os.path.join(build_dir, f"libmutant_{name}.so")
        subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fopenmp", "-shared",
                        "-fPIC", *GCC_SAN, path, "-o", lib, "-lm"], check=True)
        r = _run(tm._RUNNER.format(tests=HERE, root=ROOT, lib=lib), runtime,
                 {"OMP_NUM_THREADS": "1"}, timeout=300)
        by_pin = r.returncode == 3
        by_sanitizer = r.returncode != 0 and ("AddressSanitizer" in r.stderr or
                                              "runtime error" in r.stderr)
        return name, by_pin or by_sanitizer, r.returncode, r.stderr[-1500:]

    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(one, tm.MUTANTS))
    missed = [(n, rc, err) for n, ok, rc, err in results if not ok]
    assert not missed, missed


@pytest.mark.skipif(_clang_asan_runtime() is None, reason="clang ASan runtime not installed")
def test_clang_harness_reports(build_dir):
    _canary(build_dir, CLANG, _clang_asan_runtime())


@pytest.mark.skipif(_clang_asan_runtime() is None, reason="clang ASan runtime not installed")
def test_boundary_checks_under_asan_ubsan(build_dir):
    from tree_masked_verify_amd import build as b
    lib = b.build_library(extra=HOST_SAN, out=os.path.join(build_dir, "libsv_asan.so"),
                          obj_dir=os.path.join(build_dir, "obj"))
    code = textwrap.dedent(f"""
        import sys
        import pytest
        rc = pytest.main(["-q", "-p", "no:cacheprovider", {os.path.join(HERE, "test_boundary.py")!r}])
        maps = open("/proc/self/maps").read()
        assert {lib!r} in maps, "the sanitizer build was not the library loaded"
        sys.exit(int(rc))
    """)
    r = _run(code, _clang_asan_runtime(), {"SV_LIBRARY_PATH": lib})
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert " passed" in r.stdout
