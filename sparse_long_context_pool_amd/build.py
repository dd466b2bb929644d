"""Build libcsa.so (the gfx950 HIP kernels + the C ABI of include/csa.h).

Each csrc/*.hip file is compiled on its own with hipcc for gfx950 only, then
the objects are linked into sparse_long_context_pool_amd/libcsa.so in-tree.
The same objects, with the C ABI compiled with CSA_DEBUG, also make
libcsa_debug.so: it checks device-side inputs (attention index rows) before
each launch, synchronizing the caller's stream.  The achievable-peak probes
(probes/peaks.hip, include/csa_probe.h) go into libcsa_probe.so.
Usage: python -m sparse_long_context_pool_amd.build [--resource-usage]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions: plain fp32 VALU only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


DEBUG_LIB = os.path.join(PKG, "libcsa_debug.so")
API_SRC = os.path.join(CSRC, "csa_api.hip")
# the achievable-peak probes (include/csa_probe.h): a library of their own
PROBE_SRC = os.path.join(PKG, "probes", "peaks.hip")
PROBE_LIB = os.path.join(PKG, "libcsa_probe.so")


def _compile(src: str, extra: list[str], suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", suffix + ".o"))
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr)
    # hipcc's host pass does not know the gfx950 feature flag; that note is noise
    lines = [l for l in out.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in l]
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    jobs = [(s, extra, "") for s in srcs] + [(API_SRC, extra + ["-DCSA_DEBUG"], "_debug"),
                                             (PROBE_SRC, extra, "")]
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    probe_obj = objs.pop()
    api_debug = objs.pop()
    for lib, members in ((LIB, objs),
                         (DEBUG_LIB, [api_debug if os.path.basename(o) == "csa_api.o" else o
                                      for o in objs])):
        tmp = lib + ".tmp"
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
                        *members], check=True)
        _check_stubs(tmp)
        os.replace(tmp, lib)
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, probe_obj],
                   check=True)
    _check_stubs(tmp)
    os.replace(tmp, PROBE_LIB)
    return LIB


def _check_stubs(lib: str) -> None:
    """Fail the build when a kernel's host launch stub is referenced but not
    defined: hipcc's host pass can drop the stub of a kernel template without
    a diagnostic, and the library would then fail to load."""
    r = subprocess.run(["nm", "-u", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return  # no nm: nothing to check with
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]
    if missing:
        os.remove(lib)
        raise RuntimeError("kernel launch stubs missing from the host objects: "
                           + ", ".join(missing))


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
