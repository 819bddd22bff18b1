"""Build libirm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libirm.so")

SOURCES = ["irm_table.cpp", "irm_abi.cpp", "irm_producer.cpp", "irm_gather.hip", "irm_decode.hip", "irm_prefill.hip",
           "irm_gqa.hip", "irm_nonabsorbed.hip"]
DEPS = SOURCES + ["irm_internal.h", "irm_device.h", "irm_attn.h", "irm_launch.h"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libirm.so)")


# Sources whose MFMA accumulators stay in arch VGPRs, where the online-softmax
# rescale works on them directly (Q operands are kept in AGPRs instead).
VGPR_FORM = {"irm_decode.hip", "irm_gather.hip", "irm_prefill.hip"}


def flags() -> list:
    return [
        "--offload-arch=gfx950",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # packed-FP32 instructions are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def source_flags(name: str) -> list:
    extra = ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"] if name in VGPR_FORM else []
    return flags() + extra


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB) -> str:
    """Compile every source (each with its own flags) and link libirm.so."""
    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s + ".o")
        inc = [] if csrc == CSRC else [f"-I{csrc}"]
        _run([hipcc()] + inc + source_flags(s) + ["-c", os.path.join(csrc, s), "-o", obj], verbose)
        objs.append(obj)
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
