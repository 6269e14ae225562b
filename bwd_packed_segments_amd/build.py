"""Build libbps_attn.so (HIP for gfx950) in the package directory.

Usage: python -m bwd_packed_segments_amd.build  [--jobs N] [--verbose]

Compiles every translation unit with hipcc in parallel (one unit per
head-dim pair of the attention kernels) and links the shared library next
to this file.  Objects go to _build/ (not committed).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbps_attn.so")

ARCH = "gfx950"

# (element type, Dqk, Dv) instantiations of the attention kernels.
INSTANCES = [
    ("bf16", 64, 64), ("bf16", 64, 128), ("bf16", 128, 64), ("bf16", 128, 128),
    ("bf16", 192, 64), ("bf16", 192, 128),
    ("float", 64, 64), ("float", 64, 128), ("float", 128, 64), ("float", 128, 128),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")
    return path


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wno-unused-command-line-argument",
    ]


def units():
    out = []
    out.append(("seg_meta", [os.path.join(CSRC, "seg_meta.hip")], []))
    out.append(("ring", [os.path.join(CSRC, "ring.hip")], []))
    out.append(("attn_api", ["-x", "hip", os.path.join(CSRC, "attn_api.cpp")], []))
    out.append(("variant", [os.path.join(CSRC, "variant.hip")], []))
    for t, dqk, dv in INSTANCES:
        for part, tag in ((0, "fwd"), (1, "dq"), (2, "dkdv")):
            for var in ((0, 1, 2) if part == 0 else (0, 1)):
                name = f"attn_{tag}_{t}_{dqk}_{dv}" + ("" if var == 0 else f"_var{var}")
                out.append((name, [os.path.join(CSRC, "attn_inst.hip")],
                            [f"-DINST_T={t}", f"-DINST_DQK={dqk}", f"-DINST_DV={dv}", f"-DINST_PART={part}",
                             f"-DINST_VAR={var}"]))
    return out


def _compile(cc, name, srcs, defs, verbose):
    obj = os.path.join(BUILD, name + ".o")
    cmd = [cc] + common_flags() + defs + ["-c"] + srcs + ["-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so;
    # that line is expected and dropped.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {name} failed:\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return name, obj, time.time() - t0


def build(jobs: int | None = None, verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, cc, name, srcs, defs, verbose) for name, srcs, defs in units()]
        for f in futs:
            name, obj, dt = f.result()
            objs.append(obj)
            if verbose:
                print(f"  {name}: {dt:.1f}s")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    t0 = time.time()
    path = build(args.jobs, args.verbose)
    print(f"built {path} in {time.time() - t0:.1f}s")


if __name__ == "__main__":
    main()
