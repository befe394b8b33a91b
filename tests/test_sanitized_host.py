"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (plain C) runs whole small layers; the library's host side
(argument checks, workspace sizing, error strings: `moe_api.cpp`, built
with the host compiler against the HIP headers) runs its validation paths,
linked with the library's device objects from the in-tree build.  Neither
needs a GPU.  Each driver prints "ok"; a sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_main.c"),
           "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)
    _run(exe)


def test_api_host_side_under_sanitizers(tmp_path):
    objdir = os.path.join(ROOT, "_build", "libmoe")
    dev = [os.path.join(objdir, s + ".o") for s in ("moe_kernels.hip", "moe_probe.hip", "moe_pack.hip", "moe_noalloc.hip")]
    if not all(os.path.exists(o) for o in dev) or not os.path.exists("/opt/rocm/lib/libamdhip64.so"):
        pytest.skip("needs the in-tree build's device objects and the HIP runtime")
    csrc = os.path.join(ROOT, "mixture_experts_decode_sigmoid_amd", "csrc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    api = str(tmp_path / "moe_api_san.o")
    subprocess.run(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(csrc, "moe_api.cpp"), "-o", api],
                   check=True, capture_output=True)
    exe = str(tmp_path / "api_san")
    subprocess.run(["g++", "-std=c++17", *SAN, *inc, os.path.join(ROOT, "tests", "sanitize", "api_main.cpp"),
                    api, *dev, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe],
                   check=True, capture_output=True)
    _run(exe)
