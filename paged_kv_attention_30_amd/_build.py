"""Build the HIP library (libmsgl.so) for gfx950 with hipcc, in-tree.

Compiles every ``csrc/*.hip`` translation unit (hipcc) and every host-only
``csrc/*.cpp`` one (g++) in parallel into ``_build/`` and links them into
``paged_kv_attention_30_amd/libmsgl.so``; the same sources with
MSGL_DEBUG_CHECKS defined (device-side index checks before each call) into
``_build/debug/`` and ``libmsgl_debug.so``.
Always recompiles (the caller asked for a build).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libmsgl.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
DEBUG_LIB_PATH = os.path.join(PKG_DIR, "libmsgl_debug.so")
ARCH = os.environ.get("MSGL_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libmsgl")
    return path


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def host_cxx() -> str:
    path = shutil.which("g++")
    if not path:
        raise RuntimeError("g++ not found: the host compiler is required to build libmsgl")
    return path


def _run(cmd: list[str]) -> None:
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; that warning is expected
    lines = [ln for ln in res.stdout.splitlines()
             if "packed-fp32-ops" not in ln and "--hip-link" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


def build_variant(debug: bool, verbose: bool = False) -> str:
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    lib_path = DEBUG_LIB_PATH if debug else LIB_PATH
    defines = ["-DMSGL_DEBUG_CHECKS"] if debug else []
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in sources():
        stem, ext = os.path.splitext(os.path.basename(src))
        obj = os.path.join(out_dir, stem + ".o")
        objs.append(obj)
        if ext == ".cpp":
            cmds.append([host_cxx(), *HOST_FLAGS, *defines, "-c", src, "-o", obj])
        else:
            cmds.append([cc, *COMMON_FLAGS, *defines, "-c", src, "-o", obj])
    with ThreadPoolExecutor(min(8, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    tmp = lib_path + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path}")
    return lib_path


def build(verbose: bool = False) -> str:
    """Both libraries; returns the release one's path."""
    path = build_variant(False, verbose)
    build_variant(True, verbose)
    return path


if __name__ == "__main__":
    build(verbose=True)
