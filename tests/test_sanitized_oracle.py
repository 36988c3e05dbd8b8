"""The oracle (oracle/moe_oracle.c) and the host input generator
(gen/gen_host.c) built with gcc's AddressSanitizer and
UndefinedBehaviorSanitizer, then the oracle's pin tests run against those
builds in a child process (the sanitizer runtime preloaded into it).  An
out-of-bounds access, a use after free, a signed overflow or an invalid shift
in either library ends the child with a report and fails this test.

The first test plants an out-of-bounds read in a throwaway C function built
the same way and checks that the child dies with the report, so that a green
run below means the instrumentation was live, not absent."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SAN_CFLAGS = ["-O1", "-g", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-shared", "-fPIC",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"]


def _gcc(src, out):
    r = subprocess.run(["gcc", *SAN_CFLAGS, src, "-o", out, "-lm"], cwd=ROOT,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _san_env(extra):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4", **extra)
    return env


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    lo, lg = str(d / "liboracle_san.so"), str(d / "libgen_san.so")
    _gcc("oracle/moe_oracle.c", lo)
    _gcc("gen/gen_host.c", lg)
    return lo, lg


def test_planted_overflow_is_reported(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(textwrap.dedent("""
        #include <stdlib.h>
        int probe(int n) {
          int* a = (int*)malloc(sizeof(int) * n);
          for (int i = 0; i < n; ++i) a[i] = i;
          volatile int v = a[n];   /* one past the end */
          free(a);
          return v;
        }
    """))
    lib = str(tmp_path / "libprobe.so")
    _gcc(str(src), lib)
    code = f"import ctypes; ctypes.CDLL({lib!r}).probe(8)"
    r = subprocess.run([sys.executable, "-c", code], env=_san_env({}), capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_sanitizers(san_libs):
    lo, lg = san_libs
    env = _san_env({"MOE_ORACLE_LIB": lo, "MOE_GEN_LIB": lg})
    # the child loads the instrumented builds, not the in-tree ones
    check = ("import oracle, gen; "
             f"assert oracle.lib()._name == {lo!r}, oracle.lib()._name; "
             f"assert gen.host_lib()._name == {lg!r}, gen.host_lib()._name")
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    tests = sorted(f"tests/{f}" for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    tests.append("tests/test_page_identities.py")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *tests], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-6000:]
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, out
