"""Host-only native checks, built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code (tests/native/host_checks.cpp):

* the stream-K split of the MFMA gradient kernel and the slot arithmetic of
  its update kernel, exhaustively over many shapes (bit-exact cover of every
  (pair, tile), slots below G*J written once and read back by the right pair),
  and the update kernel's map from the partials' register order to row-wise
  matrix blocks (every element once, distinct LDS slots, exact read-back);
* the C ABI's host-side validation and workspace planning.

The checker links the sanitized ttt_api.cpp with the library's own device
objects; it makes no GPU call that could succeed, so it runs on any machine
with the ROCm toolchain.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_complexity_attention_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "host_checks")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# sanitizers on the host pass only (the device code is unchanged)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
INC = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


@pytest.fixture(scope="module")
def checker():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from linear_complexity_attention_amd import build_lib

    os.makedirs(OUT, exist_ok=True)
    dev_objs = [build_lib._compile(os.path.join(CSRC, f)) for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
    objs = []
    for src in (os.path.join(ROOT, "tests", "native", "host_checks.cpp"), os.path.join(CSRC, "ttt_api.cpp")):
        obj = os.path.join(OUT, os.path.basename(src) + ".san.o")
        _run([HIPCC, "-O1", "-g", "-std=c++17", *INC, *SAN, "-c", src, "-o", obj])
        objs.append(obj)
    exe = os.path.join(OUT, "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, *objs, *dev_objs])
    return exe


def test_streamk_cover_and_abi_under_sanitizers(checker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([checker], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "stream-K update blocks checked" in r.stdout
    assert "ABI host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
