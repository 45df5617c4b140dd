"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_171_amd.build          # or: python paged_kv_cache_171_amd/build.py

Kernels (.hip) are compiled for gfx950 only; host sources (.cpp) as C++17.
The bench's read probes (probes/pkv_probes.hip) go into libpkv_probes.so, a
library of their own that the product never loads.
Every HIP compile disables packed-fp32 instruction selection.  The shared
library gets an rpath to torch's bundled HIP runtime first (the process that
imports torch already has it loaded under the same soname) and to /opt/rocm.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpkv.so")
PROBE_SRC = os.path.join(PKG, "probes", "pkv_probes.hip")
PROBE_OUT = os.path.join(PKG, "libpkv_probes.so")
ARCH = "gfx950"
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _torch_lib() -> str | None:
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            d = os.path.join(os.path.dirname(spec.origin), "lib")
            return d if os.path.isdir(d) else None
    except Exception:
        return None
    return None


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    objs = []
    with tempfile.TemporaryDirectory(prefix="pkv_build_") as tmp:
        for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            out = _run([hipcc, "-x", "hip", "-c", src, "-o", obj] + HIP_FLAGS + inc)
            if verbose and out.strip():
                print(out)
            objs.append(obj)
        for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            out = _run([hipcc, "-c", src, "-o", obj] + CXX_FLAGS + inc)
            if verbose and out.strip():
                print(out)
            objs.append(obj)
        rpaths = [p for p in (_torch_lib(), "/opt/rocm/lib") if p]
        link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", OUT + ".tmp"] + objs
        link += [f"-Wl,-rpath,{p}" for p in rpaths] + ["-Wl,--no-undefined", "-lamdhip64"]
        _run(link)
        os.replace(OUT + ".tmp", OUT)
        # the bench's read probes: a library of their own, outside the ABI
        pobj = os.path.join(tmp, "pkv_probes.o")
        _run([hipcc, "-x", "hip", "-c", PROBE_SRC, "-o", pobj] + HIP_FLAGS)
        _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", PROBE_OUT + ".tmp", pobj]
             + [f"-Wl,-rpath,{p}" for p in rpaths] + ["-Wl,--no-undefined", "-lamdhip64"])
        os.replace(PROBE_OUT + ".tmp", PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
