"""Build ``libvplmhead.so`` (HIP C++ for gfx950) in-tree with hipcc.

    python vocab_lm_head_amd/build.py             # compile every source, link the library
                                                  # (and the C-ABI test program)
    python vocab_lm_head_amd/build.py --sanitize  # host side under ASan + UBSan, in _build/

(Run it by path: importing the package loads the library this script builds.)

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that the Python binding finds it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvplmhead.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "embed.hip", "embed_bwd.hip", "ce_fwd.hip", "ce_combine.hip", "ce_bwd.hip",
           "logits.hip"]

# packed-fp32 VALU forms are disabled on purpose: the compiler would otherwise
# emit them from plain float code in the epilogues.
# The "iterative-minreg" machine scheduler keeps each of the GEMM's 256 fp32
# accumulators in one AGPR across the K loop; the default strategy splits their
# live ranges and adds ~140 v_accvgpr copies per 128 MFMAs.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def _compile(src: str, extra: list[str], out_dir: str = BUILD) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
           "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


# host-side AddressSanitizer + UndefinedBehaviorSanitizer (the device code is unchanged)
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(BUILD, "sanitize", "libvplmhead.so")


def build(verbose: bool = True, extra: list[str] | None = None, sanitize: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link ``libvplmhead.so``. Returns its path.

    ``sanitize``: build the host side under ASan + UBSan into ``_build/sanitize/`` instead
    (load it with VP_LMHEAD_LIB and the ASan runtime preloaded)."""
    out_dir = os.path.dirname(SANITIZED_LIB) if sanitize else BUILD
    lib_path = SANITIZED_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    extra = list(extra or []) + (SANITIZE_HOST if sanitize else [])
    with concurrent.futures.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, out_dir), SOURCES))
    tmp = lib_path + ".tmp"
    link_san = ["-fsanitize=address,undefined", "-shared-libsan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", *link_san, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


C_DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "vp_step.cpp")
C_DRIVER = os.path.join(ROOT, "tests", "c_abi", "vp_step")


def build_c_driver(verbose: bool = True) -> str:
    """Compile the C-ABI test program (host code linked against libvplmhead.so, found next
    to this file at run time)."""
    cmd = [hipcc(), "-O2", "-std=c++17", "-Wall", "-I", INCLUDE, C_DRIVER_SRC, "-L", PKG,
           "-lvplmhead", "-Wl,-rpath,$ORIGIN/../../vocab_lm_head_amd", "-o", C_DRIVER]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the C-ABI test program:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {C_DRIVER}")
    return C_DRIVER


if __name__ == "__main__":
    sanitize = "--sanitize" in sys.argv[1:]
    build(sanitize=sanitize)
    if not sanitize:
        build_c_driver()
