"""Build liblsf.so (the gfx950 HIP library) in-tree with hipcc.

    python -m layer_streamed_frozen_amd.build        # or build() from Python
    python -m layer_streamed_frozen_amd.build --asan # host AddressSanitizer build

Every source is compiled for gfx950 only, without fast-math (the NF4 codes
depend on IEEE fp32 division and comparisons), with packed-fp32 instructions
disabled, and linked into layer_streamed_frozen_amd/liblsf.so.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblsf.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

SOURCES = ["nf4.hip", "gemm.hip", "gemm_wide.hip", "lora.hip", "elementwise.hip", "attention.hip", "optim.hip", "layer.cpp", "api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Host-side AddressSanitizer: instruments the host code of every source (the
# C ABI, validation, layer composition, the streamer, the launchers) and
# leaves the gfx950 device code as it is.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
ASAN_DIR = os.path.join(ROOT, "_build", "asan")
ASAN_OUT = os.path.join(ASAN_DIR, "liblsf.so")


def asan_runtime():
    """Path of the clang AddressSanitizer runtime that the host build links."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


def _compile(src, verbose, objdir=OBJDIR, extra=()):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + list(extra) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose=False, asan=False):
    """Compile every HIP source and link liblsf.so (always rebuilds).  With
    asan=True the host code is built with AddressSanitizer into
    _build/asan/liblsf.so instead (load it through LSF_LIB with the runtime
    preloaded; device code is unchanged)."""
    objdir = os.path.join(ASAN_DIR, "obj") if asan else OBJDIR
    out = ASAN_OUT if asan else OUT
    extra = ASAN_FLAGS if asan else []
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, objdir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + \
        (["-Xarch_host", "-fsanitize=address", "-shared-libasan"] if asan else []) + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv))
