"""Build libmsda.so (HIP, gfx950 only) in-tree with hipcc.

    python -m scale_deformable_attention_forward_amd.build [-v] [--checked]

Each csrc/*.hip file is compiled to an object under _build/, then linked
into scale_deformable_attention_forward_amd/libmsda.so next to this file.
With checked=True (--checked) the same sources are built with MSDA_CHECKED
(device-side bounds checks that count violations, read back with
msda_check_counts) into _build/checked/ and libmsda_checked.so.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsda.so")
CHECKED_LIB = os.path.join(PKG, "libmsda_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in any of the code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src, verbose, out_dir, defines):
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *HIP_FLAGS, *defines, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, checked: bool = False) -> str:
    out_dir = os.path.join(BUILD, "checked") if checked else BUILD
    lib = CHECKED_LIB if checked else LIB
    defines = ["-DMSDA_CHECKED"] if checked else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, out_dir, defines), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, checked="--checked" in sys.argv))
