"""Build the HIP library libgqafa.so for gfx950 in-tree.

Every HIP source is compiled by hipcc for gfx950 only, with packed fp32
arithmetic disabled, then linked into one shared library next to this file.
The kernel resource report (VGPR/AGPR/SGPR/LDS/scratch per kernel) is
written to _build/resource_usage.txt; the build fails if any kernel uses
scratch (register spills).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgqafa.so")
SOURCES = ["fa_split_d128.hip", "fa_split_d64.hip", "fa_split_d256.hip", "fa_split_d512.hip",
           "fa_prefill.hip", "fa_decode.hip", "fa_cache.hip", "fa_api.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in ordinary VGPRs: the softmax rescales them with
    # VALU ops, which cannot address AGPRs (AGPR accumulators cost a copy in
    # and out for every rescale)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr[-8000:]}")
    return obj, p.stderr


def _scratch_kernels(report: str) -> list[str]:
    bad = []
    fn = None
    for line in report.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            fn = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{fn}: {m.group(1)} bytes/lane")
    return bad


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    report = "\n".join(r[1] for r in results)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(report)
    spills = _scratch_kernels(report)
    if spills:
        raise RuntimeError("kernels spill to scratch:\n  " + "\n  ".join(spills))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[r[0] for r in results]]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
