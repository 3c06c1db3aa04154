"""Build libpkv.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_kv_cache_slots_amd.build [--jobs N]

Every source is compiled on each call (the build is the "does it compile"
check); objects go to ``paged_kv_cache_slots_amd/_build`` and the library to
``paged_kv_cache_slots_amd/libpkv.so``.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["pkv_api.hip", "scatter.hip", "merge.hip", "decode.hip", "prefill.hip", "prefill_fp8.hip", "commit.hip",
           "layout.hip", "check.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source flags.  The prefill kernel runs two waves per SIMD with the whole
# softmax state in registers; MFMA results feed vector ALU work every step, so
# its MFMAs use the VGPR form (accumulators in VGPRs, never copied from AGPRs).
SOURCE_FLAGS = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                # the fp8 kernel also schedules with the AMDGPU register-pressure
                # trackers (measured 1.5 % faster for it, 0.8 % slower for bf16)
                "prefill_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-use-amdgpu-trackers"]}


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False, out: str = LIB, build_dir: str = BUILD,
          defines=()) -> str:
    """Compile every source and link ``out``; ``defines`` are extra -D macros
    (tuning constants such as PKV_MIN_SPLIT_TOKENS)."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
