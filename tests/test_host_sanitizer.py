"""Host code of liblla under AddressSanitizer + UndefinedBehaviorSanitizer, and under
ThreadSanitizer.

For each of the two sanitizer sets, builds every ``csrc/*.hip`` file with the sanitizers on
its host half only (``-Xarch_host`` before each sanitizer flag; the device code is compiled
as for the library and never launched), links the objects with
``tests/host/lla_host_checks.c`` into one executable, and runs it.  The program drives every C-ABI entry point through the calls the header promises
to reject or answer on the host (validation order, size arithmetic at the index limits,
path resolution, workspace and alias checks, status strings, the timing record from
several threads), over a sweep of extreme shapes; a sanitizer report aborts it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

import pytest

from local_linear_attention_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host", "lla_host_checks.c")
ROCM = "/opt/rocm"
SANITIZER_SETS = {"address+undefined": ["address", "undefined"], "thread": ["thread"]}


def build_host_checks(out_dir: str, sanitize: list[str]) -> str:
    host_flags = [f for s in sanitize for f in ("-Xarch_host", f"-fsanitize={s}")] + [
        "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
        "-Xarch_host", "-O1", "-Xarch_host", "-g"]
    cc = _build.hipcc()
    srcs = sorted(glob.glob(os.path.join(_build.CSRC, "*.hip")))

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [cc, *[f for f in _build.HIPFLAGS if f != "-fPIC"], *_build.FILE_FLAGS.get(os.path.basename(src), []),
               *host_flags, "-I", _build.INCLUDE, "-I", _build.CSRC, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    drv = os.path.join(out_dir, "lla_host_checks.o")
    san = [f"-fsanitize={','.join(sanitize)}", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    cmd = [clang, "-std=c11", "-O1", "-g", "-Wall", "-Werror", *san, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", _build.INCLUDE, "-c", DRIVER, "-o", drv]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    exe = os.path.join(out_dir, "lla_host_checks")
    # The objects carry their device code already: the host linker and the HIP runtime suffice.
    cmd = [clang + "++", *san, drv, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-lpthread", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return exe


@pytest.mark.parametrize("name", sorted(SANITIZER_SETS))
def test_host_code_under_sanitizers(tmp_path, name):
    exe = build_host_checks(str(tmp_path), SANITIZER_SETS[name])
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1:exitcode=66"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    if res.returncode == 77:
        pytest.skip(res.stdout.strip())
    assert res.returncode == 0, f"exit {res.returncode}\n{res.stdout}\n{res.stderr[-6000:]}"
    assert "0 failed checks" in res.stdout, res.stdout
