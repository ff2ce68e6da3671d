"""Build the HIP library liblowbit.so (and the benchmark's probe library
liblowbit_probe.so) for gfx950, in-tree.

Every source is compiled with hipcc for --offload-arch=gfx950 with packed-fp32
instruction selection disabled.  The quantizer is compiled with
-ffp-contract=off so that its fp32 steps stay single operations.  The
decode and MFMA kernels are compiled once per bit width (-DLOWBIT_BITS=b).
The build fails if any kernel spills registers to scratch memory (read from
the compiler's kernel resource remarks).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "liblowbit.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def _units():
    units = [("lowbit_api.cpp", "lowbit_api.o", []),
             ("quant_pack.hip", "quant_pack.o", ["-ffp-contract=off"]),
             ("device_scratch.hip", "device_scratch.o", []),
             ("act_quant.hip", "act_quant.o", ["-ffp-contract=off"])]
    for b in range(1, 8):
        units.append(("qmm_a8.hip", f"qmm_a8_b{b}.o",
                      [f"-DLOWBIT_BITS={b}", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]))
        units.append(("qmv.hip", f"qmv_b{b}.o", [f"-DLOWBIT_BITS={b}"]))
        units.append(("qmm.hip", f"qmm_b{b}.o", [f"-DLOWBIT_BITS={b}"]))
        units.append(("qmm_bf16.hip", f"qmm_bf16_b{b}.o",
                      [f"-DLOWBIT_BITS={b}", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]))
    return units


# the benchmark's measurement probes: their own library, not part of the layer
PROBE_UNITS = [("probe.hip", "probe.o", [])]
PROBE_LIB_NAME = "liblowbit_probe.so"
PROBE_LIB_PATH = os.path.join(PKG, PROBE_LIB_NAME)


RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
_NAME_RE = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH_RE = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def _compile(unit):
    """Compile one unit; returns (diagnostics, {kernel: scratch bytes per lane})."""
    src, obj, extra = unit
    cmd = [hipcc()] + COMMON_FLAGS + extra + RESOURCE_REMARKS + [
        "-c", os.path.join(CSRC, src), "-o", os.path.join(BUILD_DIR, obj)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    scratch, name = {}, None
    for line in r.stderr.splitlines():
        m = _NAME_RE.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH_RE.search(line)
        if m and name:
            scratch[name] = int(m.group(1))
    # hipcc's host pass does not know the packed-fp32 feature, and the
    # resource remarks are collected above; neither is a diagnostic.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} ({obj}):\n{' '.join(cmd)}\n{err}")
    return err.strip(), scratch


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link liblowbit.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    units = _units() + PROBE_UNITS
    jobs = jobs or min(len(units), max(1, min(16, os.cpu_count() or 4)))
    spills = {}
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for unit, (msg, scratch) in zip(units, ex.map(_compile, units)):
            if msg and verbose:
                print(f"[{unit[1]}] {msg}", file=sys.stderr)
            spills.update({k: v for k, v in scratch.items() if v > 0})
    # A kernel that spills registers to scratch memory runs several times
    # slower; none of the decode or MFMA kernels may.
    if spills:
        listing = "\n".join(f"  {k}: {v} bytes/lane" for k, v in sorted(spills.items()))
        raise RuntimeError(f"kernels spill registers to scratch memory:\n{listing}")
    for lib, lib_units in ((LIB_PATH, _units()), (PROBE_LIB_PATH, PROBE_UNITS)):
        objs = [os.path.join(BUILD_DIR, u[1]) for u in lib_units]
        tmp = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
        os.replace(tmp, lib)
    build_fastcall()
    return LIB_PATH


FASTCALL_SRC = os.path.join(PKG, "_fastcall.c")


def fastcall_path() -> str:
    import sysconfig
    return os.path.join(PKG, "_lowbit_fastcall" + (sysconfig.get_config_var("EXT_SUFFIX") or ".so"))


def build_fastcall() -> str | None:
    """The binding's argument-marshalling module for eager calls (plain C
    against the Python headers; the binding uses ctypes without it)."""
    import sysconfig
    cc = shutil.which("gcc") or shutil.which("cc")
    inc = sysconfig.get_paths().get("include")
    if cc is None or inc is None or not os.path.exists(os.path.join(inc, "Python.h")):
        return None
    out = fastcall_path()
    tmp = out + ".tmp"
    cmd = [cc, "-O2", "-Wall", "-Wextra", "-shared", "-fPIC", "-I", inc, "-I", INCLUDE,
           FASTCALL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"fastcall module build failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
