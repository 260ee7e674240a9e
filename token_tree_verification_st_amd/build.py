"""Build libst.so (HIP, gfx950) in-tree with hipcc.

    python -m token_tree_verification_st_amd.build

Every .hip file under csrc/ is compiled separately (in parallel) into _build/
and linked into token_tree_verification_st_amd/libst.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libst.so")
ARCH = os.environ.get("ST_OFFLOAD_ARCH", "gfx950")

# Packed fp32 arithmetic is switched off for all device code.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Per-file device flags.  The streaming attention kernel keeps 128 fp32
# accumulators per lane; letting the register allocator place MFMA results in
# ordinary VGPRs (spilling the remainder to AGPRs) avoids copying the
# accumulators between the two files on every loop iteration.
PER_FILE = {
    # accumulators stay in VGPRs; device code assumes no NaN operands, so a
    # max of MFMA results needs no canonicalising move before it (the kernel
    # tests logits for inf/NaN with bit tests)
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true", "-Xarch_device", "-fno-honor-nans"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *PER_FILE.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        # the host pass does not know the packed-fp32 feature; anything else is shown
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln
                 and "not a recognized feature" not in ln and ln.strip()]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources for {ARCH}")
    return LIB


if __name__ == "__main__":
    build()
