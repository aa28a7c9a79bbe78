"""Ahead-of-time build of libdg.so for gfx950 with hipcc.

``python -m moe_grouped_gemm_tiles_amd.build`` compiles the HIP sources into
``moe_grouped_gemm_tiles_amd/libdg.so`` (in-tree).  The build asks the
compiler for each kernel's resource usage and fails if any kernel spills to
scratch memory (the counterpart of DeepGEMM's DG_JIT_PTXAS_CHECK switch,
README section "Utilities", which asserts no local memory use); the usage
table is written next to the library as ``libdg.resources.txt``.

It also builds ``libdg_debug.so``: the same sources with
``-DDG_DEBUG_LDS_BARRIERS=1``, which puts a full wait and a workgroup barrier
after every phase of LDS traffic in the GEMM kernels.  Tests compare its
outputs bit for bit with the normal library's (an LDS race shows up as a
difference); it is never loaded by the package.
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
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdg.so")
DEBUG_LIB = os.path.join(PKG, "libdg_debug.so")
RES = os.path.join(PKG, "libdg.resources.txt")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, f) for f in ("dg_api.hip", "dg_quant.hip", "dg_mqa.hip", "dg_layout.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("dg_kernels.hpp", "dg_common.hpp")] + [os.path.join(INCLUDE, "dg.h")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_cmd(out: str, debug_barriers: bool = False) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        *(["-DDG_DEBUG_LDS_BARRIERS=1"] if debug_barriers else []),
        # packed FP32 instructions stay off for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA results feed VALU promotion: keep them in VGPRs (no AGPR round trip)
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-Rpass-analysis=kernel-resource-usage",
        "-I", INCLUDE, "-I", CSRC,
        *SOURCES, "-o", out,
    ]


def _parse_resources(stderr: str):
    kernels = []
    cur = None
    for line in stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        if cur is None:
            continue
        for key, pat in (("sgpr", r"SGPRs: (\d+)"), ("vgpr", r"VGPRs: (\d+)"), ("agpr", r"AGPRs: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)"),
                         ("lds", r"LDS Size \[bytes/block\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                cur[key] = int(m.group(1))
    return kernels


def build(verbose: bool = False, debug: bool = True) -> str:
    """Builds libdg.so (and, unless debug=False, libdg_debug.so, compiled at the
    same time); returns the library path."""
    jobs = [(LIB, RES, False)] + ([(DEBUG_LIB, None, True)] if debug else [])
    running = []
    for lib, res, dbg in jobs:
        cmd = compile_cmd(lib + ".tmp", dbg)
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((lib, res, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    for lib, res, proc in running:
        out, err = proc.communicate()
        _finish(lib, res, proc.returncode, out, err, verbose)
    return LIB


def _finish(lib: str, res, returncode: int, out: str, err: str, verbose: bool):
    tmp = lib + ".tmp"
    if returncode != 0:
        sys.stderr.write(out + err)
        raise RuntimeError(f"hipcc failed with exit code {returncode} building {os.path.basename(lib)}")
    kernels = _parse_resources(err)
    lines = [f"{'kernel':<90} {'vgpr':>5} {'agpr':>5} {'sgpr':>5} {'scratch':>8} {'lds':>7} {'occ':>4}"]
    spills = []
    for kr in kernels:
        lines.append(f"{kr['name'][:90]:<90} {kr.get('vgpr', -1):>5} {kr.get('agpr', -1):>5} "
                     f"{kr.get('sgpr', -1):>5} {kr.get('scratch', -1):>8} {kr.get('lds', -1):>7} "
                     f"{kr.get('occupancy', -1):>4}")
        if kr.get("scratch", 0) != 0:
            spills.append(kr["name"])
    if res is not None:
        with open(res, "w") as f:
            f.write("\n".join(lines) + "\n")
    if spills:
        print("\n".join(lines), file=sys.stderr)
        os.unlink(tmp)
        raise RuntimeError(f"{os.path.basename(lib)}: kernels use scratch memory (register spills): "
                           + ", ".join(spills))
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
        if res is not None:
            print("\n".join(lines))


if __name__ == "__main__":
    build(verbose=True)
