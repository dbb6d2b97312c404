"""Builds libmoesq.so in-tree with hipcc for gfx950.

    python -m sparse_fp4_expert_amd.build

Every HIP source is compiled to an object under _build/ (in parallel), then
linked into sparse_fp4_expert_amd/libmoesq.so.  Packed-FP32 VALU forms are
switched off for device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoesq.so")
ARCH = os.environ.get("MOESQ_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compiles every source and links libmoesq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def build_host_checker(out_dir: str, verbose: bool = False) -> str:
    """Builds the library with AddressSanitizer and UndefinedBehaviorSanitizer
    on its host code (the device code is built as usual: the sanitizers
    apply to the host pass only), linked with tests/abi_checks.c, into
    out_dir/abi_checks; returns its path.  The program calls every entry
    point with arguments that the host checks reject before any HIP call,
    so it runs without a GPU."""
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".san.o")
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", *san,
               "-c", src, "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = DEVICE
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"host build failed for {src}:\n{r.stderr}")
        return obj

    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    clang = os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang")
    driver = os.path.join(ROOT, "tests", "abi_checks.c")
    dobj = os.path.join(out_dir, "abi_checks.o")
    r = subprocess.run([clang, "-x", "c", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
                        "-I/opt/rocm/include", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-c", driver, "-o", dobj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed:\n{r.stderr}")
    exe = os.path.join(out_dir, "abi_checks")
    rocm_lib = os.path.join(os.path.dirname(HIPCC), "..", "lib")
    r = subprocess.run([clang + "++", "-fsanitize=address,undefined", "-o", exe, dobj, *objs,
                        f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {exe}")
    return exe


if __name__ == "__main__":
    build()
