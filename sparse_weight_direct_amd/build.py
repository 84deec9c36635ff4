"""Build the gfx950 shared library (libsparseconv.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsparseconv.so")
PROBE_LIB = os.path.join(HERE, "libscprobe.so")  # roof probes timed by the benchmark
PROBE_SOURCE = os.path.join(HERE, "csrc", "probes.hip")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "escoin.hip", "dense.hip", "pack.cpp", "bake.cpp", "api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 instructions are disabled for all device code: hipcc would otherwise form
# v_pk_fma_f32 from scalar float code by itself.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-inline-asm",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source (one hipcc per source, in parallel) and link
    libsparseconv.so (always recompiles)."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-c", src, "-o", obj] for src, obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    msgs = []
    for (rc, out), src in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{out}")
        if out.strip():
            msgs.append(out)
    tmp = LIB + ".tmp"
    # amd_comgr assembles the weights-in-code kernels at pack time
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs +
                   ["-L/opt/rocm/lib", "-lamd_comgr", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    if verbose and (msgs or out.strip()):
        print("\n".join(msgs + [out]))
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    rc, out = _run([HIPCC] + FLAGS + ["-shared", PROBE_SOURCE, "-o", tmp])
    if rc != 0:
        raise RuntimeError(f"hipcc failed on probes.hip ({rc}):\n{out}")
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
