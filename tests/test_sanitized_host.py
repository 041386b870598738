"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (argument checks, split planning, launch set-up) is
built with both sanitizers into libdiffattn_san.so, and the fp64 oracle into
liboracle_san.so (build.py --sanitize, oracle.build(sanitize=True)).  A child
process with the sanitizer runtime preloaded runs the ABI tests and the
oracle's pins against those builds; any report fails it.  A planted
out-of-bounds write in a copy of the oracle shows that the runtime is live.
No GPU is touched: every ABI call here is rejected before a launch.
"""
import os
import subprocess
import sys

import pytest

import oracle
from transformer_attention_diffattn_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD_TESTS = ["tests/test_abi.py", "tests/test_oracle_pins.py",
               "tests/test_oracle_backward_pins.py", "tests/test_oracle_fp8_pins.py",
               "tests/test_oracle_proj_pins.py"]


def _stale(lib, sources):
    return not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib)
                                          for s in sources)


@pytest.fixture(scope="module")
def san_env():
    try:
        rt = libbuild.sanitizer_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    csrc = [os.path.join(libbuild.CSRC, f) for f in os.listdir(libbuild.CSRC)]
    csrc.append(os.path.join(ROOT, "include", "diffattn.h"))
    if _stale(libbuild.SAN_LIB, csrc):
        libbuild.build(jobs=8, sanitize=True)
    olib = oracle.build(force=False, sanitize=True)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               DIFFATTN_LIBRARY=libbuild.SAN_LIB, DIFFATTN_ORACLE_LIB=olib)
    return env


def test_abi_and_oracle_pins_clean_under_asan_and_ubsan(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", *CHILD_TESTS, "-m", "not gpu", "-q",
                        "-x", "-p", "no:cacheprovider"], cwd=ROOT, env=san_env,
                       capture_output=True, text=True, timeout=900)
    tail = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout


def test_child_loaded_the_sanitized_builds(san_env):
    code = ("import transformer_attention_diffattn_amd as da, oracle, numpy as np;"
            "da.lib(); oracle.num_threads();"
            "maps=open('/proc/self/maps').read();"
            "print('san' if 'libdiffattn_san.so' in maps and 'liboracle_san.so' in maps else 'no')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san_env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().endswith("san")


def test_planted_overflow_is_reported(san_env, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "diffattn_oracle.c")).read()
    planted = src.replace("for (int c = 0; c < dv; ++c) D[c] = 0.0;",
                          "for (int c = 0; c <= dv; ++c) D[c] = 0.0;")
    assert planted != src
    csrc = tmp_path / "planted.c"
    csrc.write_text(planted)
    lib = oracle.build(force=True, src=str(csrc), lib=str(tmp_path / "libplanted_san.so"),
                       sanitize=True)
    env = dict(san_env, DIFFATTN_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    code = ("import numpy as np, oracle;"
            "r=np.random.default_rng(0); q=r.standard_normal((4,8)); v=r.standard_normal((4,16));"
            "oracle.head_rows(q,q,q,q,v,None,causal=True,lam=0.5)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
