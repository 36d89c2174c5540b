"""Build libmoefp8.so (the HIP kernels and their C ABI) for gfx950 in-tree.

    python -m moe_fp8_grouped_amd.build [--jobs N] [--save-temps DIR]

Compiles every ``csrc/*.hip`` to an object with hipcc and links the shared
library next to this file.  Always rebuilds (the caller asked for a build).
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoefp8.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no fast math: the quantizer's float32 divide must stay correctly rounded
    "-fno-fast-math",
    # never emit packed float32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, save_temps=None):
    out_dir = os.path.abspath(save_temps) if save_temps else BUILD
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    if save_temps:
        cmd.append("-save-temps")      # intermediate files land in the working directory
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=out_dir)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and "ignoring feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    return obj, msgs


def build(jobs=None, save_temps=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, msgs in ex.map(lambda s: _compile(s, save_temps), srcs):
            objs.append(obj)
            if verbose and msgs.strip():
                print(msgs)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--save-temps", default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        sys.exit(f"hipcc not found at {HIPCC}")
    print(build(a.jobs, a.save_temps, a.verbose))


if __name__ == "__main__":
    main()
