"""Build libhy3moe.so (gfx950) in-tree with hipcc.

    python -m sparse_moe_layer_wave_amd.build      # or __graft_entry__.build()

Every .hip file under csrc/ is compiled to an object in csrc/_build/ and the
objects are linked into sparse_moe_layer_wave_amd/libhy3moe.so.  Always
recompiles (a build is a few seconds per file)."""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libhy3moe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 VALU ops (v_pk_{add,mul,fma}_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(os.path.dirname(PKG), 'include')}",
]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=True):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, warn in results:
        if warn and verbose:
            print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def clean():
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build()
