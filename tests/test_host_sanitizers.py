"""The host layer (absa.cpp) built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; the kernels are the ordinary
build), driven through every entry point's validation paths by a C program
(tests/sanitize_driver.c). No call reaches the device, so this runs on the
CPU; a sanitizer report or a wrong status fails it."""
import os
import subprocess

import pytest

from tests.conftest import ROOT

PKG = os.path.join(ROOT, "sampled_block_sparse_amd")
OUT = os.path.join(PKG, "_build", "sanitize")


@pytest.mark.slow
def test_host_layer_under_sanitizers():
    from sampled_block_sparse_amd.build import BUILD, hipcc, source_flags
    objs = [os.path.join(BUILD, "plan_kernels.hip.o"), os.path.join(BUILD, "attn_kernels.hip.o")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run python -m sampled_block_sparse_amd.build)")
    os.makedirs(OUT, exist_ok=True)
    cc = hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-g"]
    host_obj = os.path.join(OUT, "absa_san.o")
    subprocess.run([cc, *source_flags("absa.cpp"), *san, "-c",
                    os.path.join(PKG, "csrc", "absa.cpp"), "-o", host_obj],
                   check=True, capture_output=True, text=True)
    drv_obj = os.path.join(OUT, "driver.o")
    subprocess.run(["gcc", "-std=c99", "-g", "-fsanitize=address,undefined", "-I",
                    os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "sanitize_driver.c"), "-o", drv_obj],
                   check=True, capture_output=True, text=True)
    exe = os.path.join(OUT, "driver")
    subprocess.run([cc, "--offload-arch=gfx950", "-fsanitize=address,undefined", drv_obj,
                    host_obj, *objs, "-o", exe], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr
    assert "0 failure(s)" in res.stdout
