"""Build libsfm.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m selective_scan_segmented_amd.build      # or build() from Python

Every call compiles every source; SFM_BUILD_INCREMENTAL=1 reuses objects that
are newer than their source and all headers (development only).

Objects go to selective_scan_segmented_amd/_build/ (not committed); the shared
library lands next to this file as libsfm.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsfm.so")
SOURCES = ["scan.hip", "scan_cl.hip", "conv.hip", "aux.hip", "bwd.hip", "layout.hip", "sfm_api.cpp"] + [
    f"scan_{io}_n{n}.hip" for io in ("f32", "bf16") for n in (4, 8, 16)] + [
    f"split_{io}_n{n}.hip" for io in ("f32", "bf16") for n in (4, 8, 16)]
ARCH = os.environ.get("SFM_OFFLOAD_ARCH", "gfx950")
# Sources whose kernels may use scratch (register spills), with the pattern of
# the kernels in them that still must not: in bwd.hip the backward's wide
# variants spill by design, while its split-row forward instances (16-position
# chunks, modes 2 and 3, behind sfm_selective_scan_fwd_ws) are held to the rule.
SPILL_OK = {"bwd.hip": re.compile(r"bwd_kernel.*Li16ELi[23]EE")}


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # packed FP32 (v_pk_*_f32) stays off: the kernels are written for scalar fp32 VALU
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|Dynamic Stack):\s+(\S+)")


def scratch_users(remarks: str):
    """Kernels whose resource-usage remarks report scratch (private) memory or a dynamic stack."""
    bad, name = [], None
    for key, val in _REMARK.findall(remarks):
        if key == "Function Name":
            name = val
        elif key.startswith("ScratchSize") and val != "0":
            bad.append(f"{name} ({val} bytes/lane)")
        elif key == "Dynamic Stack" and val != "False":
            bad.append(f"{name} (dynamic stack)")
    return bad


def _local_includes(path: str, seen: set) -> None:
    """Files reached from path through #include "..." (csrc/ and include/), transitively."""
    if path in seen or not os.path.exists(path):
        return
    seen.add(path)
    with open(path) as f:
        for m in re.finditer(r'^\s*#\s*include\s+"([^"]+)"', f.read(), re.M):
            for d in (os.path.dirname(path), CSRC, os.path.join(ROOT, "include")):
                cand = os.path.join(d, m.group(1))
                if os.path.exists(cand):
                    _local_includes(cand, seen)
                    break


def _up_to_date(src: str, obj: str) -> bool:
    """Object newer than its source and every local header it includes
    (SFM_BUILD_INCREMENTAL=1 only)."""
    if os.environ.get("SFM_BUILD_INCREMENTAL") != "1" or not os.path.exists(obj):
        return False
    deps: set = set()
    _local_includes(os.path.join(CSRC, src), deps)
    t = os.path.getmtime(obj)
    return all(os.path.getmtime(d) < t for d in deps)


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    if _up_to_date(src, obj):
        return obj
    cmd = [_hipcc(), *_flags(), "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # No forward kernel may keep state in scratch: a per-wave object that lands
    # there (e.g. through an array indexed at run time) also turns its LDS
    # accesses into flat accesses through pointers reloaded from scratch.  The
    # backward kernels' wide variants (f32, 8-tap conv, 16 states) spill
    # registers there by design (SPILL_OK).
    bad = scratch_users(r.stderr)
    if src in SPILL_OK:
        bad = [b for b in bad if SPILL_OK[src].search(b)]
    if bad:
        os.remove(obj)
        raise RuntimeError(f"{src}: kernels use scratch memory: " + "; ".join(bad))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
