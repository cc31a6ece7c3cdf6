"""Build libsla.so (gfx950) in-tree with hipcc.

Each source compiles to an object under _build/ (in parallel), then one link
step writes block_sparse_attention_meanpool_amd/libsla.so.  Packed fp32 ops
are disabled for all device code.

Two more variants of the same library, each under its own _build/ folder:
  debug  (-DSLA_DEBUG_CHECKS): every call that reads tile lists validates them
         first into the library's debug flag (sla_debug_flag);
  san    the host-side C ABI (api.cpp) built with AddressSanitizer and
         UndefinedBehaviorSanitizer (host code only; the kernels are the
         release objects); load it with the clang ASan runtime preloaded.

Run:  python -m block_sparse_attention_meanpool_amd.build [-v] [--debug] [--san]
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "pool_classify.hip", "block_mask.hip", "sparse_attn.hip", "linear_branch.hip",
           "attn_bwd.hip", "attn_bwd_generic.hip", "linear_bwd.hip",
           "linear_bwd_generic.hip", "recall.hip",
           "tile_permute.hip", "noalloc.hip", "check_lists.hip", "clock_probe.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag: drop that warning
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


# host-only sanitizer flags (each -fsanitize= applies to the host pass only)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
SAN_RUNTIME = "libclang_rt.asan-x86_64.so"


def variant_lib(variant):
    """Path of the library a variant builds."""
    if variant == "release":
        return LIB
    return os.path.join(BUILD, variant, "libsla.so")


def san_runtime():
    """The clang ASan runtime the sanitized library needs preloaded."""
    r = subprocess.run([HIPCC, "-print-file-name=" + SAN_RUNTIME], capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if not os.path.isabs(path) or not os.path.exists(path):
        r = subprocess.run([HIPCC, "-print-resource-dir"], capture_output=True, text=True)
        path = os.path.join(r.stdout.strip(), "lib", "linux", SAN_RUNTIME)
    return path


def build(verbose=False, jobs=None, variant="release"):
    """Compile every source and link one library; variant is "release",
    "debug" or "san" (see the module docstring).  Returns the library path."""
    if variant not in ("release", "debug", "san"):
        raise ValueError(f"unknown variant {variant}")
    os.makedirs(BUILD, exist_ok=True)
    vdir = BUILD if variant == "release" else os.path.join(BUILD, variant)
    os.makedirs(vdir, exist_ok=True)
    extra = {"release": [], "debug": ["-DSLA_DEBUG_CHECKS=1"], "san": []}[variant]
    objs = []
    cmds = []
    for src in SOURCES:
        # the sanitized variant instruments only the host C ABI; its kernels
        # are the release objects
        own = variant == "debug" or (variant == "san" and src == "api.cpp") or variant == "release"
        odir = vdir if own else BUILD
        obj = os.path.join(odir, src.rsplit(".", 1)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        flags = FLAGS + extra + (SAN_FLAGS if variant == "san" and src == "api.cpp" else [])
        if own or not os.path.exists(obj):
            cmds.append([HIPCC, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs or max(1, min(8, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    lib = variant_lib(variant)
    tmp = lib + ".tmp"
    link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if variant == "san":
        link += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-shared-libsan"]
    _run(link, verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    v = "debug" if "--debug" in sys.argv else "san" if "--san" in sys.argv else "release"
    print(build(verbose="-v" in sys.argv, variant=v))
