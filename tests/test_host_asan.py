"""The C ABI's host layer under AddressSanitizer (CPU only).

The library's host code is built with -fsanitize=address (device code as usual), and a
plain C program drives every entry point's argument checks, the empty-batch paths and
the workspace queries; none of them reaches a launch.  Any out-of-bounds access or
use-after-free in argument validation, planning or error reporting fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["lcs_api.hip", "attn.hip", "select.hip"]


@pytest.fixture(scope="module")
def asan_binary(tmp_path_factory):
    if not os.path.exists(HIPCC) or shutil.which("gcc") is None:
        pytest.skip("hipcc or gcc not available")
    d = tmp_path_factory.mktemp("asan")
    inc = os.path.join(ROOT, "include")
    objs = []
    procs = []
    for src in SOURCES:
        o = str(d / src.replace(".hip", ".o"))
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
               "-Wno-unused-function", "-Wno-inline-asm",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", inc, "-c", os.path.join(ROOT, "long_context_self_amd", "csrc", src), "-o", o]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE))
        objs.append(o)
    for p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, err.decode()[-2000:]
    main_o = str(d / "main.o")
    r = subprocess.run(["gcc", "-fsanitize=address", "-g", "-I", inc, "-c",
                        os.path.join(ROOT, "tests", "asan_abi_main.c"), "-o", main_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(d / "asan_abi")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-o", exe, main_o,
                        *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return exe


def test_host_error_paths_under_asan(asan_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99")
    r = subprocess.run([asan_binary], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert "0 failures" in r.stdout
