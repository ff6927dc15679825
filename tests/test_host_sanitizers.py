"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with the sanitizers on the host side only (each
``-fsanitize=`` follows ``-Xarch_host``; device code is compiled as usual),
links ``tests/abi_host_check.c`` against it with the sanitizer runtimes, and
runs it. The checker only makes calls that fail validation or are pure host
arithmetic, so it needs no GPU. Skipped when hipcc or clang is missing.

The units that hold the ABI's host logic (argument checks, geometry, the
config tables) are rebuilt sanitized. The kernel-heavy units hold no host
code beyond launch switches that the checker never reaches, so their in-tree
objects are linked as they are when newer than every source; otherwise they
are compiled here without sanitizers.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests.conftest import ROOT

sys.path.insert(0, ROOT)
from async_stage_tile_amd import build as B  # noqa: E402

HOST_UNITS = {"pipe_api.hip", "pipe_stream_aux.hip"}
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
       "-Xarch_host", "-g"]


def _newest_source_mtime():
    newest = 0.0
    for d in (os.path.join(ROOT, "async_stage_tile_amd", "csrc"), os.path.join(ROOT, "include")):
        for name in os.listdir(d):
            newest = max(newest, os.path.getmtime(os.path.join(d, name)))
    return newest


def _clang():
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(900)
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    clang = _clang()
    if clang is None:
        pytest.skip("clang not available")
    objs = []
    cmds = []
    newest = _newest_source_mtime()
    for (src, obj, defines) in B.UNITS:
        built = os.path.join(B.OBJ, obj)
        if src not in HOST_UNITS and os.path.exists(built) and os.path.getmtime(built) > newest:
            objs.append(built)
            continue
        o = str(tmp_path / obj)
        cmd = B.compile_command(src, o, defines)
        if src in HOST_UNITS:
            cmd[1:1] = SAN
        cmds.append(cmd)
        objs.append(o)
    assert any(src in HOST_UNITS for (src, _, _) in B.UNITS)

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(run, cmds))
    lib = str(tmp_path / "libpipetile.so")
    run([hipcc, f"--offload-arch={B.ARCH}", "-fPIC", "-shared", *objs, "-o", lib])
    exe = str(tmp_path / "abi_host_check")
    run([clang, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-g", "-I", os.path.join(ROOT, "include"),
         "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
         os.path.join(ROOT, "tests", "abi_host_check.c"), lib,
         f"-Wl,-rpath,{tmp_path}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi host check ok" in r.stdout
