"""Host AddressSanitizer build of the C-ABI validation layer (CPU, no GPU needed).

dg_api.cpp -- argument, configuration, capacity and handle checks, error
text, handle bookkeeping -- is compiled with AddressSanitizer on its host pass
only (each sanitizer flag behind -Xarch_host; device code is built as usual)
and linked with the kernels' objects of the regular build into a library of
its own.  tests/asan_abi_driver.c, built with AddressSanitizer, calls every
entry point on the paths that fail before any device work and checks each
status; a heap overflow, use after free or double free there aborts it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "discrete_text_diffusion_dg_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
KERNEL_OBJS = ["k_gemm.o", "k_expert.o", "k_attn.o", "k_misc.o", "k_sampler.o"]

ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _tool(name):
    p = os.path.join("/opt/rocm/llvm/bin", name)
    return p if os.path.exists(p) else shutil.which(name)


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


def test_validation_layer_under_address_sanitizer(tmp_path):
    from discrete_text_diffusion_dg_amd import build as B
    hipcc, clang = _tool("hipcc") or "/opt/rocm/bin/hipcc", _tool("clang")
    if not os.path.exists(hipcc) or clang is None:
        pytest.skip("hipcc / clang not found")
    objs = [os.path.join(B.BUILD, o) for o in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        B.build()                      # the regular objects the library is linked from
    api = str(tmp_path / "dg_api_asan.o")
    _run([hipcc] + B.flags() + ["-O1", "-g"] + ASAN_HOST + ["-x", "hip", "-c", os.path.join(CSRC, "dg_api.cpp"),
                                                           "-o", api])
    lib = str(tmp_path / "libdg_asan.so")
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={B.ARCH}", "-o", lib, api] + objs)
    drv = str(tmp_path / "asan_abi_driver")
    _run([clang, "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-I", INCLUDE,
          os.path.join(ROOT, "tests", "asan_abi_driver.c"), lib, f"-Wl,-rpath,{tmp_path}", "-o", drv])
    env = dict(os.environ)
    # leak checking stays off: the HIP runtime's own start-up allocations are not ours to free
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    out = _run([drv], env=env, timeout=300)
    assert "ASAN_DRIVER_OK" in out and "AddressSanitizer" not in out, out[-4000:]
