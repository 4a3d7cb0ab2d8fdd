"""The library's host-only code (config validation, parameter layout,
workspace plan and regions, argument checks, the launch sequencing of every
entry point) under AddressSanitizer and UndefinedBehaviorSanitizer.

host.hip is compiled with the sanitizers on its host side only (device code
is unaffected) and linked with the library's other objects into
tests/sanitize/host_driver.cpp, which runs every host entry point over valid
and invalid configurations, including dry runs of the launch sequence
(gpt_debug_launches), so no GPU is involved. The build is cached under the
package's _build directory, keyed by a hash of the sources it uses."""
import hashlib
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decoder_only_pretraining_amd")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
OUT = os.path.join(BUILD, "sanitize")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _objects():
    from decoder_only_pretraining_amd import build as B
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "host.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    return objs


def _build_driver():
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [
        DRIVER, os.path.join(ROOT, "include", "gpt_step.h")]
    objs = _objects()
    key = _digest(srcs + objs)
    exe = os.path.join(OUT, f"host_driver_{key}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    host_o = os.path.join(OUT, f"host_{key}.o")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, *inc,
           "-c", os.path.join(CSRC, "host.hip"), "-o", host_o]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    drv_o = os.path.join(OUT, f"driver_{key}.o")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    subprocess.run([CLANG, "-O1", "-g", "-std=c++17", *san, *inc, "-c", DRIVER, "-o", drv_o],
                   check=True, capture_output=True, text=True)
    subprocess.run([CLANG, *san, drv_o, host_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True, capture_output=True,
                   text=True)
    return exe


@pytest.mark.timeout(600)
def test_host_code_is_clean_under_asan_and_ubsan():
    try:
        exe = _build_driver()
    except subprocess.CalledProcessError as e:
        raise AssertionError(f"sanitizer build failed: {e.cmd}\n{e.stderr[-3000:]}")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in r.stdout
