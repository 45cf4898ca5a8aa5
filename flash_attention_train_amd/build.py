"""Build ``libfa_train.so`` (the HIP kernels and the C ABI) for gfx950, in-tree.

Every ``csrc/*.hip`` file is compiled to an object in parallel with hipcc, then
linked into ``flash_attention_train_amd/libfa_train.so``. Packed fp32 VALU
instructions are disabled for the device code (``-packed-fp32-ops``); the host
pass warns that it does not know that feature, which is harmless.

Run as ``python -m flash_attention_train_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfa_train.so")
# the checked build (-DFA_CHECK): every launch's index space verified on the host first, and
# fa_train_check_launch exported (include/fa_train_check.h)
CHECK_LIB = os.path.join(HERE, "libfa_train_check.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Wno-unused-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # no NaN quieting around min/max: the kernels never form NaNs (-inf is
            # handled explicitly), so IEEE-mode canonicalization would be pure overhead
            "-fno-honor-nans",
            # MFMA accumulators in arch VGPRs: the softmax reads them, and the AGPR form
            # cost a v_accvgpr_read per element in the hot loops
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, check: bool = False) -> str:
    obj = os.path.join(OBJDIR, ("check_" if check else "") + os.path.basename(src) + ".o")
    cmd = [hipcc(), *_flags(), *(["-DFA_CHECK"] if check else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = True, check: bool = False) -> str:
    """Compile and link the library; always rebuilds. Returns the library path. With
    check=True, the checked build (-DFA_CHECK) goes to libfa_train_check.so instead."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(lambda f: _compile(f, check), srcs))
    lib_path = CHECK_LIB if check else LIB
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


if __name__ == "__main__":
    build(check="--check" in sys.argv[1:])
    sys.exit(0)
