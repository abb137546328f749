"""Build libhierasparse.so (the attention library) and libhspeaks.so (the measurement kernels of
include/hs_peaks.h) for gfx950 in-tree: hipcc compiles each csrc/*.hip to an object under _build/
(in parallel) and links the shared libraries next to this file."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhierasparse.so")
SOURCES = ["hs_api.hip", "hs_compress.hip", "hs_decode.hip", "hs_prefill.hip",
           "hs_recompress.hip", "hs_masked.hip"]
PEAKS_LIB = os.path.join(PKG, "libhspeaks.so")
PEAKS_SOURCES = ["hs_peaks.hip"]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Wall", "-Wno-unused-result",
         # packed fp32 VALU ops stay off (compiler-generated v_pk_*_f32 forms are avoided)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source extra flags. The attention kernels mix dense MFMA and SMFMAC on the same
# accumulators; SMFMAC's accumulator is always a VGPR tuple, so dense MFMAs there use the VGPR form
# as well (no copies between accumulation and arch registers).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
EXTRA = {"hs_prefill.hip": _VGPR_FORM, "hs_decode.hip": _VGPR_FORM, "hs_peaks.hip": _VGPR_FORM}


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def _link(objs, lib, verbose):
    tmp = f"{lib}.tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
