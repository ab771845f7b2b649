"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/sanitize/ are built with both sanitizers on and
recovery off, then run; any report (an out-of-bounds access, a use after free,
a leak, signed overflow, an out-of-range index or shift) fails the test:

- the C oracle (oracle/moe_oracle.c) with oracle_driver.c, built by gcc, on
  small seeded inputs and the degenerate cases (no tokens, a token subset,
  top_k == E, experts with no token, equal logits, empty and clamped
  sequences);
- the host side of the C ABI (bit_expert_grouped_amd/csrc/moe_api.cpp, its
  host code instrumented, its device code built as usual) with abi_driver.c,
  linked with the library's other objects: workspace sizes, stage names,
  status strings and every argument check that refuses a call before a device
  call.  No GPU is used.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm/bin"

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
}
REPORTS = ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:")

pytestmark = pytest.mark.slow


def _run_checked(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr)


def _run_driver(exe, banner):
    env = dict(os.environ, **SAN_ENV)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text
    assert banner in r.stdout, text
    for marker in REPORTS:
        assert marker not in text, text


def test_oracle_under_sanitizers():
    if not shutil.which("gcc"):
        pytest.skip("gcc is not installed")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run_checked(["gcc", "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
                  "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                  "-I" + os.path.join(ROOT, "oracle"),
                  os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
                  "-lm", "-o", exe])
    _run_driver(exe, "all cases ran clean")


def _library_objects():
    """Objects of every library source but the C-ABI one, rebuilt when missing or older than a source."""
    from bit_expert_grouped_amd import build

    srcs = [s for s in build.sources() if os.path.basename(s) != "moe_api.cpp"]
    objs = [os.path.join(build.BUILD, os.path.basename(s) + ".o") for s in srcs]
    headers = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC) if f.endswith(".h")]
    newest = max(os.path.getmtime(p) for p in srcs + headers)
    if not all(os.path.exists(o) and os.path.getmtime(o) >= newest for o in objs):
        build.build()
    return build, objs


def test_c_abi_host_under_sanitizers():
    if not (os.path.exists(os.path.join(LLVM, "clang++")) and shutil.which("hipcc")):
        pytest.skip("the ROCm compilers are not installed")
    build, objs = _library_objects()
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "moe_api_san.o")
    # the sanitizers instrument the host code only; the device code is built as for the library
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run_checked([build.HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall",
                  "-I" + os.path.join(ROOT, "include"), "-I" + build.CSRC, "-x", "hip"]
                 + build.DEVICE + host_san + ["-c", os.path.join(build.CSRC, "moe_api.cpp"), "-o", api])
    drv = os.path.join(OUT, "abi_driver.o")
    _run_checked([os.path.join(LLVM, "clang"), "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
                  "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
                  "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                  "-c", os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = os.path.join(OUT, "abi_driver")
    _run_checked([os.path.join(LLVM, "clang++"), "-fsanitize=address,undefined", drv, api] + objs
                 + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    _run_driver(exe, "all checks passed")
