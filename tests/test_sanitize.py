"""Sanitizer builds on the CPU (no GPU involved):

- the oracle, driven over random and edge-case inputs with exactly sized
  buffers (gcc, -fsanitize=address,undefined);
- the host side of libepget (validation, capacity and workspace sizing,
  error paths) driven with 200,000 random and extreme descriptors, in a build
  whose host code carries the same sanitizers (device code is compiled as
  usual; no call reaches a device).
"""
import os
import shutil
import subprocess

import pytest

from combine_ep_get_amd import build as libbuild
from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    r = _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              os.path.join(HERE, "c", "oracle_driver.c"), obuild.SRC, "-lm", "-o", exe])
    assert r.returncode == 0, r.stderr
    r = _run([exe, "300"], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"), timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "clean" in r.stdout


@pytest.mark.skipif(not (os.path.exists(libbuild.HIPCC) and os.path.exists(CLANG)),
                    reason="hipcc / clang not available")
def test_library_host_code_under_address_and_ub_sanitizers(tmp_path):
    so = str(tmp_path / "libepget_san.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    r = _run([libbuild.HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-shared", *san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", libbuild.INCLUDE, libbuild.SRC, "-o", so])
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "abi_host_driver")
    r = _run([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all", "-I", libbuild.INCLUDE,
              os.path.join(HERE, "c", "abi_host_driver.c"), "-L", str(tmp_path),
              "-lepget_san", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    assert r.returncode == 0, r.stderr[-4000:]
    # the HIP runtime itself is not built with the sanitizer: leaks it keeps
    # until exit are not this library's
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"), timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "clean" in r.stdout
