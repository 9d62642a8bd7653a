"""Build librfattn.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m attention_pass_cascaded_amd.build [-v]

Each translation unit is compiled to an object in parallel, then linked into
``attention_pass_cascaded_amd/librfattn.so``.  Packed-FP32 instructions are
disabled for the device code.

``--sanitize`` builds a second copy, ``_build/sanitized/librfattn.so``, whose
HOST code (argument validation, workspace arithmetic, the C ABI) carries
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is the same
as in the normal build.  It is for CPU runs of the ABI tests only: load it by
naming it in RF_ATTN_LIB with clang's ASan runtime preloaded
(tests/test_sanitized_abi.py does exactly that).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librfattn.so")
SOURCES = ["api.hip", "inst_f16.hip", "inst_bf16.hip", "inst_f32.hip"]
SANITIZED_LIB = os.path.join(OBJ, "sanitized", "librfattn.so")
# host-only sanitizers: each -fsanitize= is scoped to the host pass
SANITIZE_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g")
ARCH = os.environ.get("RF_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags(extra=()):
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-result", *extra]


def _compile(src: str, verbose: bool, obj_dir: str, extra=()) -> str:
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags(extra), "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)
    return out


def build(verbose: bool = False, jobs: int | None = None, extra_flags=(), out: str | None = None,
          link_flags=()) -> str:
    """Compile every source and link the library.

    ``extra_flags`` (e.g. -D tuning macros) and ``out`` (another library path)
    let a tile or schedule setting be built beside the default one.
    """
    lib = out or LIB
    if out is None:
        obj_dir = OBJ
    elif os.path.basename(out) == "librfattn.so":
        obj_dir = os.path.join(os.path.dirname(out), "obj")
    else:
        obj_dir = os.path.join(OBJ, os.path.basename(out).replace(".so", ""))
    os.makedirs(obj_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, obj_dir, tuple(extra_flags)), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *link_flags, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build_sanitized(verbose: bool = False) -> str:
    """The ASan + UBSan host build (see the module docstring)."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    return build(verbose, extra_flags=SANITIZE_FLAGS, out=SANITIZED_LIB,
                 link_flags=("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"))


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
