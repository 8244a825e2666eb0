"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

- The oracle (oracle/jbo.c) driven through every entry point on small shapes
  (tests/sanitize/oracle_driver.c).
- The host side of libjetblock (sanitizers on the host code only) driven through the
  argument validation of every C-ABI entry point and the workspace-size queries up to
  the documented shape limits (tests/sanitize/abi_driver.c).

Any out-of-bounds access, use after free, leak or undefined operation fails the test."""
import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_jetblock_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_SOURCES = ["jb_api", "jb_gen", "jb_prefill", "jb_fwd", "jb_decode", "jb_proj", "jb_backward"]
SAN = ["-fsanitize=address", "-fsanitize=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-2000:], r.stderr[-4000:])
    return r


def _env():
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    return env


def _clean(r):
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", *SAN, "-fno-sanitize-recover=all",
              "-o", exe, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
              os.path.join(ROOT, "oracle", "jbo.c"), "-lm", "-lpthread"])
        r = _run([exe], env=_env(), timeout=300)
        _clean(r)
        assert "all calls clean" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_validation_under_asan_ubsan():
    host_san = [f for s in SAN for f in ("-Xarch_host", s)]
    # device code is compiled too (the objects carry it) but never run
    common = [HIPCC, "--offload-arch=gfx950", "-O1", "-Xarch_host", "-g", "-fno-omit-frame-pointer",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-sanitize-recover=all", *host_san]
    with tempfile.TemporaryDirectory() as d:
        def obj(name):
            o = os.path.join(d, name + ".o")
            _run([*common, "-std=c++17", "-fPIC", "-c", os.path.join(CSRC, name + ".hip"), "-o", o])
            return o
        with ThreadPoolExecutor(min(len(LIB_SOURCES), os.cpu_count() or 1)) as ex:
            objs = list(ex.map(obj, LIB_SOURCES))
        drv = os.path.join(d, "abi_driver.o")
        _run(["/opt/rocm/llvm/bin/clang", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", *SAN,
              "-fno-sanitize-recover=all", "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "-o", drv])
        exe = os.path.join(d, "abi_driver")
        _run([*common, "-o", exe, drv, *objs, "-Wl,-rpath,/opt/rocm/lib"])
        r = _run([exe], env=_env(), timeout=300)
        _clean(r)
        if r.stdout.startswith("skipped"):
            pytest.skip(r.stdout.strip())
        assert "checks passed" in r.stdout, r.stdout
