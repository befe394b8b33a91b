"""Builds libmoe.so (the C-ABI library of include/moe.h) for gfx950 with hipcc.

    python -m mixture_experts_decode_sigmoid_amd.build

Each source is compiled to an object of its own, in parallel, then linked.
`defines` adds preprocessor definitions (e.g. MOE_TIMELINE for the phase
stamps build, written to another path).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["moe_kernels.hip", "moe_probe.hip", "moe_pack.hip", "moe_noalloc.hip", "moe_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_*_f32 in the device code
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _clean(stderr: str) -> str:
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    objdir = os.path.join(ROOT, "_build", os.path.basename(out).replace(".so", ""))
    os.makedirs(objdir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *FLAGS, *dflags, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        return obj, r.returncode, _clean(r.stderr)

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    errs = [f"{os.path.basename(o)}: {e}" for o, rc, e in results if rc != 0]
    if errs:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose:
        for o, _, e in results:
            if e:
                print(e)
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for o, _, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{_clean(r.stderr)}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
