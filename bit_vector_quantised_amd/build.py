"""Build the HIP library libmoe_vq.so for gfx950 in the package directory.

    python bit_vector_quantised_amd/build.py

Every kernel is compiled with hipcc for gfx950 only.  Packed-fp32 VALU forms are
disabled (-packed-fp32-ops): scalar and float2 code stays on plain fp32 ops.
Only the moe_vq_* C entry points are exported (hidden visibility elsewhere, and
-Bsymbolic), so another copy of the library loaded into the same process cannot
take over its internal functions.

The build fails when a kernel uses scratch (private) memory: on this stack every
launch of such a kernel pays a set-up cost of about 17 us, more than the decode-batch
kernels themselves take.  The compiler's per-kernel resource report is written to
_build/kernel_resources.txt.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmoe_vq.so")
SOURCES = ["api.hip", "route.hip", "fc.hip", "fc_mfma.hip", "fc2_single.hip", "decode.hip", "prefill.hip",
           "probe.hip"]
CPP_SOURCES = ["cpu_experts.cpp"]  # host code (the expert path on the host cores), built with g++
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wno-unused-result", "-Rpass-analysis=kernel-resource-usage"]


def kernel_resources(text: str):
    """(kernel, {field: value}) from hipcc's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                      r"LDS Size \[bytes/block\]|Dynamic Stack): (\S+)", line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = (val, {})
            out.append(cur)
        elif cur is not None:
            cur[1][key.split()[0] if key != "Dynamic Stack" else "DynamicStack"] = (
                val == "True" if key == "Dynamic Stack" else int(val))
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        text = r.stdout + r.stderr
        out = "\n".join(l for l in text.splitlines()
                        if "is not a recognized feature for this target" not in l and "remark:" not in l
                        and "-Rpass-analysis" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out)
        return obj, kernel_resources(text)

    def compile_cpp(src):
        obj = os.path.join(objdir, src + ".o")
        cmd = ["g++", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-fvisibility-inlines-hidden", "-pthread", "-Wall", "-I", INCLUDE,
               "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"g++ failed on {src}:\n{r.stdout}{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
        cpp_objs = list(ex.map(compile_cpp, CPP_SOURCES))
    objs = [o for o, _ in results] + cpp_objs
    res = [k for _, ks in results for k in ks]
    with open(os.path.join(objdir, "kernel_resources.txt"), "w") as f:
        for name, v in res:
            f.write(f"{name} " + " ".join(f"{k}={x}" for k, x in v.items()) + "\n")
    spilling = [name for name, v in res if v.get("ScratchSize", 0) > 0 or v.get("DynamicStack")]
    if spilling:
        raise RuntimeError("kernels use scratch memory: " + ", ".join(spilling))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-Wl,-Bsymbolic", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
