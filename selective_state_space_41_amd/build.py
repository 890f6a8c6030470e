"""Compile the HIP library in-tree for gfx950.

``python -m selective_state_space_41_amd.build`` (or ``build()``) runs hipcc on
``csrc/vmscan.hip`` and writes ``libvmscan.so`` next to this file; it always recompiles.
``python -m selective_state_space_41_amd.build --probe`` builds only the issue-rate
microbenchmark (``csrc/probe.hip`` -> ``vmscan_probe``), which is not part of the library.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libvmscan.so")
PROBE = os.path.join(PKG, "vmscan_probe")

# Packed fp32 VALU forms are kept out of every gfx950 code object.
HIP_FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build vmscan")
    return h


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name; that warning is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    """Compile libvmscan.so."""
    hipcc = _hipcc()
    tmp = LIB + ".tmp"
    out = _run([hipcc, *HIP_FLAGS, "-shared", "-I", os.path.join(ROOT, "include"),
                "-o", tmp, os.path.join(PKG, "csrc", "vmscan.hip")])
    os.replace(tmp, LIB)
    if verbose and out.strip():
        print(out)
    return LIB


def build_probe(verbose=False):
    """Compile the issue-rate microbenchmark executable (measures the gfx950 VALU, exp2 and
    scan-token rates the kernel design relies on)."""
    out = _run([_hipcc(), *HIP_FLAGS, "-o", PROBE + ".tmp", os.path.join(PKG, "csrc", "probe.hip")])
    os.replace(PROBE + ".tmp", PROBE)
    if verbose and out.strip():
        print(out)
    return PROBE


if __name__ == "__main__":
    print(build_probe(verbose="-v" in sys.argv) if "--probe" in sys.argv else build(verbose="-v" in sys.argv))
