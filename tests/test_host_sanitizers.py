"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The packer, plan chooser, schedule, kernel-stream encoder, weights-in-code generator and C
ABI (api.cpp, pack.cpp, bake.cpp) are index arithmetic over offsets, segments and schedules;
they are built with g++ -fsanitize=address,undefined (device launchers stubbed: host-only
handles never launch) and driven through the ABI by a seeded fuzz of host-only packs over
filters up to 11x11, strides to 4, pads to 3, up to 300 channels, every pack form and malformed
CSR.  The oracle is built the same way and run on small layers.  Any sanitizer report or
failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_weight_direct_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="no host compiler")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_packer_and_generator_under_sanitizers(tmp_path):
    objs = []
    for src in ("api.cpp", "pack.cpp", "bake.cpp"):
        o = str(tmp_path / (src + ".o"))
        _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + CSRC,
              "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", o] + SAN)
        objs.append(o)
    for src in ("stubs.cpp", "fuzz_pack.cpp"):
        o = str(tmp_path / (src + ".o"))
        _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + CSRC,
              "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(HERE, src), "-o", o] + SAN)
        objs.append(o)
    exe = str(tmp_path / "fuzz_pack")
    _run(["g++", "-o", exe] + objs + SAN + ["-L/opt/rocm/lib", "-lamdhip64", "-lamd_comgr",
                                               "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([exe, "60"], env=env)
    assert "failed checks 0" in r.stdout, r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_run")
    _run(["gcc", "-std=c11", "-o", exe, os.path.join(HERE, "oracle_run.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-lm"] + SAN)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = _run([exe], env=env)
    assert "disagree on 0 outputs" in r.stdout, r.stdout
