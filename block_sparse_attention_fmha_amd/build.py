"""Build libfmha.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m block_sparse_attention_fmha_amd.build [--jobs N] [--verbose]

Every source under csrc/ is compiled by hipcc for gfx950 only, objects go to
csrc/_build/, and the shared library lands next to this file. Packed-fp32 VALU
instructions are disabled for device code (-packed-fp32-ops), matching the rule that
this library never relies on them. -fno-honor-nans: no kernel relies on NaN semantics
(infinities are still honoured: masked scores are -inf).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(CSRC, "_build")
LIB = os.path.join(HERE, "libfmha.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",   # no kernel relies on NaN semantics; lets fmaxf map to v_max3 directly
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def kernels_using_scratch(remarks: str):
    """(kernel, what, amount) for every kernel whose resource-usage remarks show scratch
    memory or spilled VGPRs (SGPR spills go to VGPR lanes and are not counted)."""
    import re
    bad, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill): (\d+)", line)
        if m and cur and int(m.group(2)) > 0:
            bad.append((cur, m.group(1), int(m.group(2))))
    return bad


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    else:
        # every kernel must keep its state in registers: a kernel that spills to scratch
        # runs many times slower, so the build stops on one (see kernels_using_scratch)
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{r.stdout}\n{r.stderr}")
    bad = kernels_using_scratch(r.stderr)
    if bad:
        lines = "\n".join(f"  {k}: {what} = {n}" for k, what, n in bad)
        raise RuntimeError(f"{os.path.basename(src)}: kernels use scratch memory:\n{lines}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libfmha.so; returns the library path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4) // 2), 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libfmha.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    main()
