"""AddressSanitizer and UBSan runs of the host code, on the CPU.

* The float64 oracle (oracle/mta_oracle.c) is built with gcc under
  ``-fsanitize=address,undefined`` together with
  tests/sanitize/oracle_driver.c, which calls every entry point over all
  placements, mixing-group sizes and the general layer.
* The library's host code (validation, kernel selection and LDS fit, workspace
  sizing, argument checks) is built from the same sources as libmta.so, with
  the sanitizers on the host pass only, and linked with
  tests/sanitize/abi_driver.c.  That driver never reaches a kernel launch or any
  other GPU call, so it runs here without a GPU.

Any sanitizer report aborts the driver (``halt_on_error``) and fails the test.
"""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "transformer_attention_variant_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "transformer_attention_variant_amd", "_build", "sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"

ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "mta_oracle.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=600)
    assert "oracle driver: ok" in r.stdout


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# The sanitizers go on the host pass only (each -fsanitize= directly after
# -Xarch_host); the device code is compiled as usual, at -O1 to keep the build
# short, and is never run.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _build_host_objects():
    srcs = _sources()
    hdrs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if not f.endswith(".hip"))
    tag = _digest(srcs + hdrs + [os.path.join(INCLUDE, "mta.h")])
    out = os.path.join(OUT, tag)
    stamp = os.path.join(out, "done")
    objs = [os.path.join(out, os.path.basename(s) + ".o") for s in srcs]
    if os.path.exists(stamp):
        return objs
    os.makedirs(out, exist_ok=True)

    def one(src_obj):
        src, obj = src_obj
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", f"-I{INCLUDE}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-w"] + HOST_SAN +
             ["-c", src, "-o", obj])

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(one, zip(srcs, objs)))
    open(stamp, "w").close()
    return objs


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="hipcc not found")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    objs = _build_host_objects()
    drv = str(tmp_path / "abi_driver.o")
    _run([CLANG, "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", f"-I{INCLUDE}", "-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-fPIC"] + HOST_SAN + ["-o", exe, drv] + objs)
    r = _run([exe], env=ENV, timeout=300)
    assert "abi driver: ok" in r.stdout, r.stdout
