"""Build libirm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc."""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libirm.so")

SOURCES = ["irm_table.cpp", "irm_abi.cpp", "irm_producer.cpp", "irm_gather.hip", "irm_decode.hip", "irm_prefill.hip",
           "irm_gqa.hip", "irm_nonabsorbed.hip", "irm_upproj.hip"]
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


# Sources scheduled with another of the compiler's machine-scheduler
# strategies: the non-absorbed attention kernel needs 230-250 registers, and
# the default strategy spills it; iterative-ilp fits it in 250 with no spill.
SCHED_STRATEGY = {"irm_nonabsorbed.hip": "iterative-ilp"}


def source_flags(name: str) -> list:
    extra = ["-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form"] if name in VGPR_FORM else []
    if name in SCHED_STRATEGY:
        extra += ["-Xarch_device", f"-mllvm=-amdgpu-sched-strategy={SCHED_STRATEGY[name]}"]
    return flags() + extra


RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"LDS Size \[bytes/block\]):\s*(\S+)")
_KEYS = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch_bytes_per_lane",
         "Occupancy [waves/SIMD]": "waves_per_simd", "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_usage(text: str) -> dict:
    """Per-kernel register, scratch, occupancy and LDS figures from the
    compiler's kernel-resource-usage remarks."""
    usage, cur = {}, None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = usage.setdefault(val, {})
        elif cur is not None:
            cur[_KEYS[key]] = int(val)
    return usage


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    msgs = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return "\n".join(lines)


def check_build_output(text: str, usage: dict) -> None:
    """Refuse a build whose kernels spill to scratch memory (the attention
    kernels count their copies with explicit s_waitcnt vmcnt, which a
    compiler-made scratch access would silently break) or whose inline
    assembly clobbers a reserved register."""
    if "Reserved registers on the clobber list" in text:
        raise RuntimeError("inline assembly clobbers a reserved register:\n" + text)
    spills = {k: v["scratch_bytes_per_lane"] for k, v in usage.items() if v.get("scratch_bytes_per_lane", 0)}
    if spills:
        raise RuntimeError(f"kernels use scratch memory (bytes per lane): {spills}")


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB) -> str:
    """Compile every source (each with its own flags), check every kernel's
    resource usage and link libirm.so.  The compiler's per-kernel figures are
    written to _build/resource_usage.json beside the library."""
    objdir = os.path.join(os.path.dirname(out), "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, usage = [], {}
    for s in SOURCES:
        obj = os.path.join(objdir, s + ".o")
        inc = [] if csrc == CSRC else [f"-I{csrc}"]
        remark = [RESOURCE_REMARK] if s.endswith(".hip") else []
        text = _run([hipcc()] + inc + source_flags(s) + remark + ["-c", os.path.join(csrc, s), "-o", obj], verbose)
        found = parse_resource_usage(text)
        check_build_output(text, found)
        usage.update(found)
        objs.append(obj)
    with open(os.path.join(objdir, "resource_usage.json"), "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    tmp = out + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
