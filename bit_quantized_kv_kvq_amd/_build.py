"""Build libkvq.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvq.so")
SOURCES = ["kvq_api.cpp", "kvq_quant.hip", "kvq_decode.hip", "kvq_probe.hip", "kvq_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # a fetch-add whose result is read much later must not be rewritten into a wave-wide
    # add whose result is broadcast (and so waited for) right away
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def torch_lib_dir() -> str | None:
    """Directory of the HIP runtime bundled with PyTorch.  libkvq must use the same runtime
    instance as torch (one process cannot drive the GPU through two HIP/HSA runtimes)."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or spec.origin is None:
        return None
    d = os.path.join(os.path.dirname(spec.origin), "lib")
    return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-8000:])


def build(verbose: bool = False) -> str:
    """Compile each source to an object with hipcc, then link against the HIP runtime that
    PyTorch loads (falling back to the system one when torch is absent)."""
    objdir = os.path.join(PKG, "_objs")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        flags = [f for f in HIPCC_FLAGS if f != "-shared"]
        _run([hipcc(), *flags, "-x", "hip", "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    tl = torch_lib_dir()
    rt = [f"-L{tl}", "-l:libamdhip64.so", f"-Wl,-rpath,{tl}"] if tl else \
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    tmp = LIB + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, *rt], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
