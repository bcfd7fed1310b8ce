"""Build libhy3moe.so (gfx950) in-tree with hipcc.

    python -m sparse_moe_layer_wave_amd.build [--sanitize]   # or __graft_entry__.build()

Every .hip file under csrc/ is compiled to an object in csrc/_build/ and the
objects are linked into sparse_moe_layer_wave_amd/libhy3moe.so.  Always
recompiles (a build is a few seconds per file).  --sanitize builds a separate
copy with host-side AddressSanitizer and UndefinedBehaviorSanitizer into
csrc/_build/san/ for the CPU tests of the C ABI."""

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


# Host-only AddressSanitizer + UndefinedBehaviorSanitizer (argument checks,
# workspace carving, launch set-up).  Each -fsanitize= sits right after
# -Xarch_host, so device code is built exactly as in the product library.
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_DIR = os.path.join(OBJDIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libhy3moe_san.so")


# Flags of single files.  gemm_grouped.hip: block-scale accumulators are rescaled
# by VALU multiplies between MFMAs, so its MFMAs read and write them in VGPRs
# rather than AGPRs (which would take a copy out and back per multiply).
FILE_FLAGS = {
    "gemm_grouped.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src, objdir=OBJDIR, extra=()):
    obj = os.path.join(objdir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=True, sanitize=False):
    """Build the library; with sanitize=True, a copy whose host code carries
    the sanitizers (SAN_LIB, outside the package; load it with the
    sanitizer runtime preloaded, see sanitizer_runtime())."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objdir = SAN_DIR if sanitize else OBJDIR
    lib = SAN_LIB if sanitize else LIB
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(objdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda src: _compile(src, objdir, extra), srcs))
    for _, warn in results:
        if warn and verbose:
            print(warn, file=sys.stderr)
    tmp = lib + ".tmp"
    link_extra = [*SAN_FLAGS, "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], *link_extra,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def sanitizer_runtime():
    """Path of the clang AddressSanitizer runtime (it carries the
    UndefinedBehaviorSanitizer handlers too) that a process loading SAN_LIB
    must preload."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True, check=True)
    return r.stdout.strip()


def clean():
    shutil.rmtree(OBJDIR, ignore_errors=True)


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv)
