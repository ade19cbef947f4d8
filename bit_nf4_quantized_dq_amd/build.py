"""Build the HIP library libqlora_nf4.so in-tree for gfx950 with hipcc.

Every call compiles every source (objects in _build/, then one shared library next to
this file).  Usage: python -m bit_nf4_quantized_dq_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libqlora_nf4.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["api.cpp", "codebook.cpp", "quantize.hip", "dequant.hip", "lora.hip", "gemv.hip",
    "gemv_stream.hip", "gemm.hip", "gemm_nt.hip", "merge.hip", "adamw.hip", "mlp.hip", "noalloc.hip", "gemv_rows.hip"]

COMMON = [
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-ffp-contract=off",  # the decode steps are defined as separate FP32 roundings
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]
DEVICE = [
    "--offload-arch=gfx950",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Private (scratch) memory per lane that a kernel may use; every other kernel must use none.
# A kernel that starts spilling registers runs many times slower (a fused reduction split once
# went from 6.9 to 11 ms per 8B-shaped layer step that way), so the build refuses it.
SCRATCH_ALLOWANCE = {
    "k_gemm_dx": 8,  # one spilled register in the fused mid-size dX kernel
}


def _kernel_resources(stderr: str) -> list[tuple[str, int, int]]:
    """(kernel name, VGPRs, scratch bytes per lane) from the compiler's resource remarks."""
    out, name, vgpr = [], None, 0
    for line in stderr.splitlines():
        if "remark:" not in line:
            continue
        text = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if text.startswith("Function Name:"):
            name = text.split(":", 1)[1].strip()
        elif text.startswith("VGPRs:") and name:
            vgpr = int(text.split(":", 1)[1])
        elif text.startswith("ScratchSize") and name:
            out.append((name, vgpr, int(text.split(":", 1)[1])))
            name = None
    return out


def _short(mangled: str) -> str:
    """The kernel's own name inside an Itanium-mangled symbol: a decimal length, then the name
    (the digits before it may also end the anonymous namespace's tag, so each split of them
    is tried; the name is the one that ends where the nested name or its template arguments
    begin)."""
    import re

    for m in re.finditer(r"(\d+)k_", mangled):
        digits, start = m.group(1), m.end(1)
        for i in range(len(digits) - 1, -1, -1):
            n = int(digits[i:])
            name = mangled[start:start + n]
            after = mangled[start + n:start + n + 1]
            if len(name) == n and re.fullmatch(r"k_[a-z0-9_]+", name) and after in ("E", "I"):
                return name
    return mangled


# Extra device flags per source: the whole-row stream takes its first 16 argument dwords
# preloaded into SGPRs (its first loads then need no argument fetch).
EXTRA_DEVICE = {
    "gemv_rows.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=16"],
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [_hipcc(), *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE, *EXTRA_DEVICE.get(src, []), "-Rpass-analysis=kernel-resource-usage"]
    else:
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]  # host-only units
    cmd += ["-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    if src.endswith(".hip"):
        res = _kernel_resources(r.stderr)
        with open(os.path.splitext(obj)[0] + ".resources.txt", "w") as f:
            for name, vgpr, scratch in res:
                f.write(f"{name} vgpr={vgpr} scratch={scratch}\n")
        bad = [(n, sc) for n, _, sc in res if sc > SCRATCH_ALLOWANCE.get(_short(n), 0)]
        if bad:
            raise RuntimeError(f"{src}: kernels use scratch memory (spilled registers): {bad}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
