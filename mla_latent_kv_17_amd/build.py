"""Build libmla.so (the C-ABI HIP library) in-tree for gfx950.

    python mla_latent_kv_17_amd/build.py [--verbose]

(run as a script: importing the package would load the library being rebuilt)

Each kernel source is compiled to an object with hipcc, then linked into
``mla_latent_kv_17_amd/libmla.so``.  Always rebuilds (the sources are small).
The hash of the sources (``source_hash()``) is compiled into the library,
which reports it through ``mla_source_hash()``: the binding refuses a library
built from other sources than the ones beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
PEAKS_LIB = os.path.join(PKG, "libmla_peaks.so")
SOURCES = ["api.hip", "decode.hip", "absorb.hip", "combine.hip", "out_uv.hip", "append.hip", "gate.hip", "explicit.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # never form packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over every kernel and header source
    the library is built from (csrc/*.hip, csrc/*.h, include/*.h), by name
    and content."""
    h = hashlib.sha256()
    files = []
    for d, exts in ((CSRC, (".hip", ".h")), (os.path.join(ROOT, "include"), (".h",))):
        files += sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(exts))
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def built_hash(lib: str = LIB) -> str | None:
    """The source hash compiled into a built library (read from the file, so
    the library need not be loaded), or None."""
    if not os.path.exists(lib):
        return None
    with open(lib, "rb") as fh:
        data = fh.read()
    i = data.find(b"mla-source-hash:")
    return data[i + 16:i + 32].decode("ascii", "replace") if i >= 0 else None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    stamp = f'-DMLA_SOURCE_HASH="{source_hash()}"'
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append(([HIPCC, *FLAGS, stamp, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]], verbose)
    os.replace(tmp, LIB)
    # the benchmark's measurement probes, a library of their own
    tmp = PEAKS_LIB + ".tmp"
    _run([HIPCC, *FLAGS, *extra_flags, "-shared", "-o", tmp, os.path.join(CSRC, "peaks.hip")], verbose)
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv)
    print(LIB)
