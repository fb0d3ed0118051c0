"""Build the HIP libraries in-tree for gfx950 with hipcc.

``python -m online_softmax_exact_amd.build`` compiles every ``csrc/*.hip``
into ``_build/*.o`` (in parallel) and links ``libattn_mi355x.so`` (the
attention ABI of ``include/attn_mi355x.h``) and ``libattn_probes.so`` (the
unit microbenchmarks of ``include/attn_probes.h``) next to this file.
``build_sanitized()`` links a copy of the attention library whose host code
in ``attn_api.hip`` (argument validation, kernel choice) carries AddressSanitizer
and UndefinedBehaviorSanitizer checks, for the CPU tests of the ABI.
``build()`` also links ``libattn_mi355x_poison.so``, every kernel
compiled with ``-DATTN_DEBUG_POISON=1`` (LDS filled with NaN bytes at kernel
entry and ahead of every HBM -> LDS copy), which the GPU tests run beside
the normal build.  Always rebuilds when called.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn_mi355x.so")
PROBES_LIB = os.path.join(PKG, "libattn_probes.so")
SANITIZED_LIB = os.path.join(OUT_DIR, "sanitized", "libattn_mi355x.so")
POISON_LIB = os.path.join(PKG, "libattn_mi355x_poison.so")
POISON = ["-DATTN_DEBUG_POISON=1"]
PROBES_SRC = "probes.hip"
# Sanitizers on the host pass only (device code is built as usual).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-g"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.
COMMON = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    """Sources of the attention library (every csrc/*.hip but the probes)."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") and f != PROBES_SRC)


def _compile(src: str, verbose: bool, extra=(), out_dir: str = OUT_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool, extra=()) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, jobs: int = 8) -> str:
    poison_dir = os.path.join(OUT_DIR, "poison")
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(poison_dir, exist_ok=True)
    srcs = sources() + [os.path.join(CSRC, PROBES_SRC)]
    jobs_list = [(s, (), OUT_DIR) for s in srcs] + [(s, POISON, poison_dir) for s in sources()]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(jobs_list)))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1], j[2]), jobs_list))
    n = len(srcs)
    _link(objs[:n - 1], LIB, verbose)
    _link(objs[n - 1:n], PROBES_LIB, verbose)
    _link(objs[n:], POISON_LIB, verbose)
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """The attention library with attn_api.hip's host code under ASan and
    UBSan (the other objects as built by ``build``, which must have run)."""
    out = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out, exist_ok=True)
    api = _compile(os.path.join(CSRC, "attn_api.hip"), verbose, HOST_SANITIZE, out)
    others = [os.path.join(OUT_DIR, os.path.basename(src)[:-4] + ".o") for src in sources()
              if os.path.basename(src) != "attn_api.hip"]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing}")
    return _link([api, *others], SANITIZED_LIB, verbose,
                 ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"])


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
