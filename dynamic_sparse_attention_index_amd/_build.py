"""Build the gfx950 HIP library ``libvsattn.so`` in-tree with hipcc."""
import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvsattn.so")
# bounds-checked variant (VS_DEBUG_BOUNDS): same sources, own objects
DEBUG_OBJ = os.path.join(PKG, "_build_debug")
DEBUG_LIB = os.path.join(PKG, "libvsattn_debug.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    # scores are never NaN: plain v_max without the NaN-quieting duplicate
    "-fno-honor-nans",
]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(DEBUG_OBJ if debug else OBJ, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *(["-DVS_DEBUG_BOUNDS=1"] if debug else []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every kernel source and link the shared library (with
    `debug`: the bounds-checked variant); returns its path."""
    out = DEBUG_LIB if debug else LIB
    os.makedirs(DEBUG_OBJ if debug else OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, debug=True)
