"""Build libfa.so from csrc/*.hip with hipcc for gfx950 (in-tree, no JIT cache).

Each source is compiled to an object in parallel, then linked into
``flashattention_online_softmax_fa_amd/libfa.so``; the same sources compiled
with FA_STATS=1 give the debug build ``libfa_stats.so``, whose kernels also
count events (include/fa_stats.h).  Run it as a script
(``python flashattention_online_softmax_fa_amd/build.py``) or through
``__graft_entry__.build()``; importing the package itself needs the built
library.

``--variant NAME -DMACRO=VALUE ...`` builds ``variants/libfa_NAME.so`` from
the same sources with other compile-time tile constants (the FA_FWD_*,
FA_BWD_* and FA_TILE_GROUP macros of the kernels); setting FA_LIBRARY to its
path makes the package load it in place of libfa.so, so that the tile-size
choices can be timed and profiled against each other with the same scripts.
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
OBJDIR = os.path.join(ROOT, "_build")
SO = os.path.join(PKG, "libfa.so")
STATS_SO = os.path.join(PKG, "libfa_stats.so")
VARIANT_DIR = os.path.join(PKG, "variants")

SOURCES = ["fa_api.hip", "fwd_f32.hip", "fwd_bf16.hip", "bwd.hip", "bwd_f32.hip", "decode.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    # no kernel produces or tests NaN on purpose; lets max/min skip canonicalisation
    "-fno-honor-nans",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libfa.so")


def _compile(job) -> str:
    src, objdir, extra = job
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(x for x in (r.stderr or "").splitlines()
                     if "not a recognized feature" not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return obj


def _link(objs, so: str) -> None:
    tmp = so + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, so)


def build(verbose: bool = False, stats: bool = True) -> str:
    """Compile every source and link libfa.so (and, with ``stats``, the debug
    build libfa_stats.so); returns the path of libfa.so."""
    variants = [(SO, OBJDIR, [])]
    if stats:
        variants.append((STATS_SO, os.path.join(OBJDIR, "stats"), ["-DFA_STATS=1"]))
    jobs = []
    for _, objdir, extra in variants:
        os.makedirs(objdir, exist_ok=True)
        jobs += [(src, objdir, extra) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, jobs))
    for k, (so, _, _) in enumerate(variants):
        _link(objs[k * len(SOURCES):(k + 1) * len(SOURCES)], so)
        if verbose:
            print(f"built {so}")
    return SO


def build_variant(name: str, defines, verbose: bool = False) -> str:
    """libfa.so built with extra -D definitions, as variants/libfa_<name>.so."""
    if not name.replace("_", "").isalnum():
        raise ValueError(f"variant name {name!r}: letters, digits and '_' only")
    for d in defines:
        if not d.startswith("-DFA_"):
            raise ValueError(f"{d!r}: variants take -DFA_... definitions only")
    objdir = os.path.join(OBJDIR, "variants", name)
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(VARIANT_DIR, exist_ok=True)
    jobs = [(src, objdir, list(defines)) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, jobs))
    so = os.path.join(VARIANT_DIR, f"libfa_{name}.so")
    _link(objs, so)
    if verbose:
        print(f"built {so} ({' '.join(defines)})")
    return so


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--variant":
        build_variant(sys.argv[2], sys.argv[3:], verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
