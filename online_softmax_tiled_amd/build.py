"""Build libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m online_softmax_tiled_amd.build``; ``__graft_entry__.build()``
calls :func:`build`. The library lands next to this file so it travels with
the source tree. Sources are compiled in parallel to objects under
``_build/`` and linked with the HIP runtime (resolved at load time; when
torch is imported first, its already-loaded libamdhip64.so.7 serves it).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libattn.so")

SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "merge.hip", "merge_lse.hip", "gather.hip", "stream.hip", "noalloc.hip"]
# Per-source extra flags. The prefill kernel never compares against NaN and
# treats no NaN operand specially, so NaN-quieting of fmax inputs is not
# needed (it costs a v_max per score); infinities keep their IEEE meaning.
EXTRA_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    f"--offload-arch={ARCH}",
    "-mcode-object-version=5",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is needed to build libattn.so")


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + lang + COMMON_FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(
        line for line in (res.stdout + res.stderr).splitlines()
        if "is not a recognized feature for this target" not in line
    )
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose=False):
    """Compile every source and link libattn.so. Returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
