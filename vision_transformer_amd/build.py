"""Build libjepa_mi355x.so for gfx950 with hipcc, in-tree.

usage: python -m vision_transformer_amd.build [-j N] [--debug] [--sanitize]

--sanitize builds a second copy, _build/sanitize/libjepa_mi355x.so, whose
host code (argument checks, the quantizer, block packing, the rotary table,
the GGUF reader) carries AddressSanitizer and UndefinedBehaviorSanitizer
checks; device code is built as usual.  It runs on the CPU only, loaded into
a Python whose first preloaded library is the sanitizer runtime
(SANITIZER_RUNTIME), with JEPA_LIB_PATH pointing at it.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libjepa_mi355x.so")
SAN_DIR = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libjepa_mi355x.so")
# host-only sanitizer flags (-Xarch_host keeps them off the device code)
SAN_FLAGS = "-Xarch_host -fsanitize=address,undefined -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer -g".split()
SOURCES = ["gemm.hip", "attention.hip", "misc.hip", "api.hip", "gguf.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags(debug: bool) -> list[str]:
    f = [f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-O1" if debug else "-O3",
         "-I", os.path.join(ROOT, "include"),
         # no packed fp32 ops anywhere in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]
    return f


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    return r.returncode, out


def sanitizer_runtime() -> str:
    """The clang ASan runtime hipcc's host compiler links against."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


def build(jobs: int = 4, debug: bool = False, verbose: bool = False, sanitize: bool = False) -> str:
    out_dir = SAN_DIR if sanitize else BUILD
    out_lib = SAN_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    fl = flags(debug or sanitize) + (SAN_FLAGS if sanitize else [])

    def compile_one(src):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc()] + fl + ["-c", os.path.join(CSRC, src), "-o", obj]
        rc, out = _run(cmd)
        if verbose or rc:
            print(" ".join(cmd), file=sys.stderr)
            if out.strip():
                print(out, file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed on {src}")
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out_lib + ".tmp"
    # (the sanitized copy leaves the runtime's symbols to the preloaded runtime)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    rc, out = _run(cmd)
    if rc:
        print(" ".join(cmd) + "\n" + out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, out_lib)
    return out_lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=4)
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--sanitize", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.debug, a.v, a.sanitize))
