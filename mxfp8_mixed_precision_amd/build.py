"""Build libtemx.so (the C-ABI library of HIP kernels for gfx950) in-tree.

Usage: python mxfp8_mixed_precision_amd/build.py   (or call build()).  Run it as a script, not
as a package module: importing the package loads the library being rebuilt.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtemx.so")
SOURCES = ["quantize.hip", "amax_cast.hip", "gemm.hip", "block_gemm.hip", "block_gemm_e8m0.hip", "block_gemm_fp32.hip", "block_scale.hip",
           "block_quantize.hip", "status.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libtemx.so")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        # packed-fp32 instructions stay off (the compiler would otherwise form
        # v_pk_{add,mul,fma}_f32 from scalar float code)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


_FUNC = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def spilled_kernels(remarks: str) -> list[tuple[str, int]]:
    """(kernel, scratch bytes per lane) for every kernel of the compiler's resource report that uses
    scratch memory (register spills)."""
    out, name = [], None
    for line in remarks.splitlines():
        m = _FUNC.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and name is not None and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libtemx.so; returns its path.  Fails if any kernel spills
    registers to scratch memory: every kernel of the library is meant to run from registers, and a
    spill (from a change elsewhere in a kernel's template) costs far more than it shows in the source."""
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    objs, procs = [], []
    for src in SOURCES:  # compiled in parallel (the GEMM sources take the longest)
        obj = os.path.join(obj_dir, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(), "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed, spills = [], []
    for src, proc in procs:
        _, err = proc.communicate()
        if proc.returncode != 0:
            sys.stderr.write(err)
            failed.append(src)
        else:
            spills += [(src, k, b) for k, b in spilled_kernels(err)]
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    if spills:
        listing = "; ".join(f"{src}: {k} ({b} B/lane)" for src, k, b in spills[:10])
        raise RuntimeError(f"{len(spills)} kernel(s) spill registers to scratch: {listing}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
