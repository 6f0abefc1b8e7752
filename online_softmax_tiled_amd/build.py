"""Build libattn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m online_softmax_tiled_amd.build``; ``__graft_entry__.build()``
calls :func:`build`. The library lands next to this file so it travels with
the source tree. Sources are compiled in parallel to objects under
``_build/`` and linked with the HIP runtime (resolved at load time; when
torch is imported first, its already-loaded libamdhip64.so.7 serves it).

The same sources built with ATTN_DEVICE_CHECKS give libattn_checked.so, the
debug library whose kernels test every raw global access against the extent
of its tensor (include/attn.h, attn_check_report); the tests load it beside
the product library.
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
CHECKED_LIB_PATH = os.path.join(HERE, "libattn_checked.so")

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


def _compile(src, verbose, checked=False):
    obj = os.path.join(BUILD_DIR, ("checked_" if checked else "") + os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    defs = ["-DATTN_DEVICE_CHECKS"] if checked else []
    cmd = [hipcc()] + lang + COMMON_FLAGS + defs + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
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


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, path)


def build(verbose=False, checked=True):
    """Compile every source and link libattn.so, and (checked=True) the
    bounds-checking debug library libattn_checked.so. Returns the product
    library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + ([(s, True) for s in SOURCES] if checked else [])
    workers = min(len(jobs), os.cpu_count() or 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    if checked:
        _link(objs[len(SOURCES):], CHECKED_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
