"""Builds libnc.so (the HIP library) in-tree for gfx950 with hipcc.

Usage: python -m dense_pretraining_amd.build [-j N]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libnc.so")
SOURCES = ["api.hip", "gemm.hip", "rows.hip", "attn.hip", "embed_bwd.hip", "infer.hip", "skinny.hip", "opt.hip", "fp8.hip", "prof.hip", "products.hip", "noalloc.hip"]
HEADERS = ["common.h", "frag.h", "gemm.h", "kernels.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Wno-unused-variable",
    # packed fp32 ops stay off (only ordinary scalar float code is emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file code generation options. The attention kernels keep their MFMA
# accumulators in VGPRs (the default heuristic moves them through AGPRs every
# iteration there).
FILE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src, extra):
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is harmless
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    return src, p.returncode, err, obj


def build(jobs=None, extra=None, verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    extra = list(extra or [])
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    objs = []
    failed = False
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, rc, err, obj in ex.map(lambda s: _compile(s, extra), SOURCES):
            if err.strip() and (rc != 0 or verbose):
                print(f"--- {src}\n{err}", file=sys.stderr)
            if rc != 0:
                failed = True
            objs.append(obj)
    if failed:
        raise RuntimeError("hipcc compilation failed")
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (say, a kernel stub never instantiated) fails here, not at load time
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        print(p.stderr, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=None)
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel register/LDS usage from the compiler")
    a = ap.parse_args()
    extra = ["-Rpass-analysis=kernel-resource-usage"] if a.resource_usage else []
    print(build(a.j, extra, verbose=a.v or a.resource_usage))


if __name__ == "__main__":
    main()
