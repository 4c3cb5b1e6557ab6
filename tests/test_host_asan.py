"""The library's host code (argument checks, workspace sizing, launch
planning) under AddressSanitizer: a host-ASan build of libcsa2 and a C
driver (tests/asan_host_check.c) that walks workspace sizing over a grid of
shapes and every validation error path.  No call reaches device work, so
this runs on the CPU."""
import os
import subprocess

import pytest

from compressed_sparse_attention_decode_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
CLANG = "/opt/rocm/llvm/bin/clang"


def test_host_paths_clean_under_asan():
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    lib = _build.build_host_asan()
    d = os.path.dirname(lib)
    exe = os.path.join(d, "asan_host_check")
    subprocess.run([CLANG, "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-O1",
                    os.path.join(HERE, "asan_host_check.c"), "-o", exe, f"-L{d}", "-lcsa2_asan",
                    f"-Wl,-rpath,{d}", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr, r.stderr
    assert "host checks passed" in r.stdout
