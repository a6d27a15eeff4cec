"""Build libsimar.so for gfx950 with hipcc (all HIP sources and the host
C++ around them), in-tree: the library lands next to this file."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "simar")
LIB = os.path.join(HERE, "libsimar.so")
# extra compiler flags (space separated), e.g. "-DSIMAR_STORE_NT=0" for a variant build
EXTRA = os.environ.get("SIMAR_EXTRA_FLAGS", "").split()

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                      # every fp32 op rounds on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx950 feature name; that note is harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(jobs: int = 0, out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every source and link libsimar.so (or `out`); always rebuilds."""
    global BUILD
    BUILD = build_dir
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


def build_pycall(out_dir: str = HERE) -> str:
    """Compile the prepared-call extension (_pycall) with the host C compiler
    against this interpreter's headers; always rebuilds."""
    import sysconfig
    cc = os.environ.get("CC", "gcc")
    out = os.path.join(out_dir, "_pycall" + sysconfig.get_config_var("EXT_SUFFIX"))
    tmp = out + ".tmp"
    cmd = [cc, "-O2", "-shared", "-fPIC", "-std=c11", "-Wall", "-Werror",
           "-I", sysconfig.get_paths()["include"], "-I", INCLUDE,
           os.path.join(CSRC, "pycall.c"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("pycall build failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--build-dir", default=BUILD)
    a = ap.parse_args()
    print(build(out=a.out, build_dir=a.build_dir))
    print(build_pycall())
