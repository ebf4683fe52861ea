"""Host code under sanitizers (CPU only).

- The C ABI's host code (mfa_api.hip compiled host-only) linked with a
  host-memory stand-in for the HIP runtime and the kernel launchers
  (tests/sanitize/hip_stub.cpp) and driven through every entry point by
  tests/sanitize/api_driver.cpp, under AddressSanitizer + UndefinedBehavior-
  Sanitizer (every shape sweep, stale handles, allocation failures) and
  under ThreadSanitizer (handles created, used and destroyed on 8 threads).
  The stand-in's launchers check that each kernel's workspace regions lie in
  the handle's allocations.
- The oracle (oracle/mfa_oracle.c) built with gcc's AddressSanitizer +
  UndefinedBehaviorSanitizer and driven over every exported function on
  small ragged, paged and split cases by tests/sanitize/oracle_driver.c.

Each build goes to a temporary directory; nothing here touches a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "decode_attention_mfa_amd", "csrc")
INC = os.path.join(ROOT, "include")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _env(**extra):
    """A small environment for the sanitized programs (only what they need)."""
    env = {k: os.environ[k] for k in ("PATH", "HOME", "TMPDIR", "LANG") if k in os.environ}
    env.update(extra)
    return env


def _run(cmd, **kw):  # noqa: D103
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    if r.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\nexit {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-8000:]}")
    return r


def _build_api_driver(tmp, sanitizers):
    """Link the host-only ABI, the stand-in and the driver under `sanitizers`
    (host pass only: -Xarch_host before each -fsanitize)."""
    host_san = []
    for s in sanitizers:
        host_san += ["-Xarch_host", f"-fsanitize={s}"]
    hip = [CLANG, "-x", "hip", "--offload-host-only", "--offload-arch=gfx950", "-O1", "-g",
           "-fno-omit-frame-pointer", *host_san, "-I", INC, "-I", CSRC, "-I", SAN]
    objs = []
    for name, src in (("api", os.path.join(CSRC, "mfa_api.hip")), ("stub", os.path.join(SAN, "hip_stub.cpp"))):
        o = os.path.join(tmp, name + ".o")
        _run(hip + ["-c", src, "-o", o])
        objs.append(o)
    cxx_san = [f"-fsanitize={s}" for s in sanitizers]
    drv = os.path.join(tmp, "driver.o")
    _run([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", *cxx_san, "-I", INC, "-I", SAN, "-c",
          os.path.join(SAN, "api_driver.cpp"), "-o", drv])
    objs.append(drv)
    # the host-only object names the device image it would register; the
    # stand-in's registration ignores its contents
    sym = [ln.split()[-1] for ln in _run(["nm", "-u", objs[0]]).stdout.splitlines() if "__hip_fatbin_" in ln]
    if sym:
        fb = os.path.join(tmp, "fatbin.cpp")
        with open(fb, "w") as f:
            f.write("".join(f'extern "C" {{ char {s}[64]; }}\n' for s in sym))
        _run([CLANG, "-c", fb, "-o", fb + ".o"])
        objs.append(fb + ".o")
    exe = os.path.join(tmp, "api_driver")
    _run([CLANG, *cxx_san, *objs, "-o", exe, "-lpthread"])
    return exe


needs_clang = pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")


@needs_clang
@pytest.mark.timeout(600)
def test_api_host_asan_ubsan(tmp_path):
    exe = _build_api_driver(str(tmp_path), ["address", "undefined"])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"),
             timeout=540)
    assert "api_driver: ok" in r.stdout


@needs_clang
@pytest.mark.timeout(600)
def test_api_host_tsan(tmp_path):
    exe = _build_api_driver(str(tmp_path), ["thread"])
    r = _run([exe, "threads"], env=_env(TSAN_OPTIONS="halt_on_error=1"), timeout=540)
    assert "api_driver: ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.timeout(600)
def test_oracle_asan_ubsan(tmp_path):
    exe = os.path.join(str(tmp_path), "oracle_driver")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "mfa_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"),
             timeout=540)
    assert "oracle_driver: ok" in r.stdout
