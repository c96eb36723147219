"""Builds libpakv.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

Two diagnostic builds of the same sources sit beside it:
  libpakv_bounds.so   every source with PAKV_DEBUG_BOUNDS: the kernels count the
                      page-table entries outside the pool that they meet
                      (pakv_debug_bounds_counts);
  libpakv_hostsan.so  the host-only sources under AddressSanitizer and
                      UndefinedBehaviorSanitizer (the kernels' sources as in
                      libpakv.so), for the CPU tests of the host logic; a
                      process loads it with the ASan runtime preloaded
                      (asan_runtime()).
The binding loads PAKV_LIBRARY when that is set, else libpakv.so.
"""

import argparse
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpakv.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
          "-Wall", "-Wno-unused-function"]
# Device code: gfx950 only; packed-FP32 instructions stay off.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Host-only sources under the sanitizers (each -fsanitize= after -Xarch_host:
# nothing here instruments device code)
HOSTSAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-fno-sanitize-recover=undefined"]

SOURCES = ["pakv_api.cpp", "pakv_pool.cpp", "pakv_step.cpp", "kernels_store.hip", "kernels_decode.hip", "kernels_extend.hip",
           "kernels_extend_general.hip", "kernels_extend_stage.hip"]

VARIANTS = {
    None: "libpakv.so",
    "bounds": "libpakv_bounds.so",
    "hostsan": "libpakv_hostsan.so",
}


def library_path(variant=None):
    return os.path.join(HERE, VARIANTS[variant])


def asan_runtime():
    """The clang ASan runtime that libpakv_hostsan.so links (None if absent)."""
    pat = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "lib", "clang", "*", "lib",
                       "linux", "libclang_rt.asan-x86_64.so")
    found = sorted(glob.glob(pat))
    return os.path.realpath(found[-1]) if found else None


def _compile(src, out_dir, extra):
    path = os.path.join(CSRC, src)
    obj = os.path.join(out_dir, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC] + COMMON + extra + DEVICE + ["-x", "hip"]
    else:
        cmd = [HIPCC] + COMMON + extra
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, extra):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC"] + extra + ["-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_library(verbose=False, variant=None):
    """Compiles every source and links the library of `variant` (None: the
    product, libpakv.so); always rebuilds.  The hostsan build reuses the
    product's kernel objects (building them first if they are missing)."""
    out = library_path(variant)
    if variant is None:
        os.makedirs(BUILD_DIR, exist_ok=True)
        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            objs = list(ex.map(lambda s: _compile(s, BUILD_DIR, []), SOURCES))
        _link(objs, out, ["--offload-arch=" + ARCH])
    elif variant == "bounds":
        d = os.path.join(BUILD_DIR, "bounds")
        os.makedirs(d, exist_ok=True)
        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            objs = list(ex.map(lambda s: _compile(s, d, ["-DPAKV_DEBUG_BOUNDS"]), SOURCES))
        _link(objs, out, ["--offload-arch=" + ARCH])
    elif variant == "hostsan":
        rt = asan_runtime()
        if rt is None:
            raise RuntimeError("the clang ASan runtime (libclang_rt.asan-x86_64.so) was not found")
        d = os.path.join(BUILD_DIR, "hostsan")
        os.makedirs(d, exist_ok=True)
        os.makedirs(BUILD_DIR, exist_ok=True)
        host = [s for s in SOURCES if s.endswith(".cpp")]
        dev = [s for s in SOURCES if s.endswith(".hip")]
        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            objs = list(ex.map(lambda s: _compile(s, d, HOSTSAN), host))
            dobjs = [os.path.join(BUILD_DIR, s + ".o") for s in dev]
            missing = [s for s, o in zip(dev, dobjs) if not os.path.exists(o)]
            list(ex.map(lambda s: _compile(s, BUILD_DIR, []), missing))
        _link(objs + dobjs, out, ["-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                  "-fsanitize=undefined", "-Wl,-rpath," + os.path.dirname(rt)])
    else:
        raise ValueError(f"unknown variant {variant!r}")
    if verbose:
        print(f"built {out}", file=sys.stderr)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--variant", choices=["bounds", "hostsan"], default=None)
    build_library(verbose=True, variant=ap.parse_args().variant)
