"""Builds libkda.so (HIP, gfx950) in-tree.

    python -m gated_delta_rule_46_amd.build

Every .hip file under csrc/ is compiled with hipcc for gfx950 and linked into
gated_delta_rule_46_amd/libkda.so.  Packed fp32 VALU instructions are turned
off (-packed-fp32-ops): the kernels rely on plain fp32 arithmetic only.

The device assembly of every source is emitted alongside (_build/*.s) and
checked by isa_check: the build fails if any MFMA accumulates onto the fresh
result of an MFMA of another shape (see isa_check for why).
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _assemble_listing(src: str) -> str:
    out = os.path.join(BUILD, os.path.basename(src) + ".s")
    cmd = [HIPCC, *COMMON, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def check_listings(paths) -> None:
    from .isa_check import check_file
    bad = []
    for p in paths:
        bad += [(os.path.basename(p),) + h for h in check_file(p)]
    if bad:
        lines = "\n".join(f"  {f}:{ln} ({fn[:60]}): {a}  ->  {b}  [{d} wait states]"
                           for (f, fn, ln, a, b, d) in bad[:20])
        raise RuntimeError(f"{len(bad)} MFMA accumulator chain(s) switch MFMA shape:\n{lines}")


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max(1, min(8, 2 * len(srcs)))) as ex:
        objs_f = [ex.submit(_compile, s_) for s_ in srcs]
        lst_f = [ex.submit(_assemble_listing, s_) for s_ in srcs]
        objs = [f.result() for f in objs_f]
        listings = [f.result() for f in lst_f]
    check_listings(listings)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library(verbose=True)
