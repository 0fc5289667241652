"""Build libhsa.so in-tree with hipcc for gfx950.

    python -m token_sparse_attention_compact_amd.build [-v]

Compiles every csrc/*.hip to an object (in parallel) and links
token_sparse_attention_compact_amd/lib/libhsa.so; probe/*.hip (measurement
helpers used by the benchmark only) become lib/libhsa_probe.so.  Always
rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libhsa.so")
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(LIBDIR, "libhsa_probe.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libhsa)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(cc, src, obj, verbose):
    cmd = [cc, *FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _link(cc, objs, lib, verbose):
    tmp_lib = lib + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp_lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp_lib, lib)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(LIBDIR, exist_ok=True)
    probes = sorted(os.path.join(PROBE_DIR, f) for f in os.listdir(PROBE_DIR) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory(prefix="hsa_build_") as tmp:
        objs, probe_objs, jobs = [], [], []
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
            for src, dst in [(p, objs) for p in sources()] + [(p, probe_objs) for p in probes]:
                obj = os.path.join(tmp, os.path.basename(src) + ".o")
                dst.append(obj)
                jobs.append(ex.submit(_compile, cc, src, obj, verbose))
            for j in jobs:
                j.result()
        _link(cc, objs, LIB, verbose)
        _link(cc, probe_objs, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
