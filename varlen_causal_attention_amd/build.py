"""Build ``libvlca.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m varlen_causal_attention_amd.build`` (or
``__graft_entry__.build()``).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import sysconfig

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvlca.so")
SOURCES = [os.path.join(CSRC, "vlca_kernels.hip"), os.path.join(CSRC, "vlca_backward.hip"),
           os.path.join(CSRC, "vlca_masked.hip"), os.path.join(CSRC, "vlca_proj.hip"),
           os.path.join(CSRC, "vlca_noalloc.hip"),
           os.path.join(CSRC, "vlca_api.cpp"), os.path.join(CSRC, "vlca_graph.cpp")]
# The CPython call trampoline (argument marshalling for the two launch entry points).
CALL_SOURCE = os.path.join(CSRC, "vlca_pyext.c")
CALL_MODULE = os.path.join(PKG, "_vlca_call" + (sysconfig.get_config_var("EXT_SUFFIX") or ".so"))

# Packed fp32 VALU forms are disabled for all device code.  MFMA results are kept
# in VGPRs (not AGPRs): the softmax reads every score and rescales the
# accumulators, and AGPR results would need a v_accvgpr copy each way.  The
# atomic optimizer is off: it rewrites the attention kernel's one-lane work
# claim into a wave-aggregated atomic whose result is waited for at once, which
# would put the claim's round trip at the start of every item.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libvlca.so)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *DEVICE_FLAGS, "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln]  # host pass does not know the device feature
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    build_call_module(verbose)
    return LIB


def build_call_module(verbose: bool = False) -> str:
    """Compile the CPython trampoline (host C only, no HIP)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the call module")
    tmp = CALL_MODULE + ".tmp"
    cmd = [cc, "-O2", "-shared", "-fPIC", "-Wall", "-I", sysconfig.get_paths()["include"], "-I", INCLUDE,
           CALL_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building the call module failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, CALL_MODULE)
    return CALL_MODULE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
