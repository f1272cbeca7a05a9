"""Sanitizer builds of the CPU-side code (no GPU needed).

* The oracle's C (``oracle/moe_oracle.c``) with AddressSanitizer and UndefinedBehaviorSanitizer,
  driven by ``tests/sanitize/oracle_driver.c`` over every exported function and its edge cases.
* The library's host-only C++ -- status strings, ``moe_gather_layout`` and the EPLB placement
  (``moe_eplb_balancedness``, ``moe_eplb_rebalance``, ``moe_eplb_logical_to_physical``) --
  with the same sanitizers on the host side of the HIP compile (``-Xarch_host``), driven by
  ``tests/sanitize/host_driver.cpp`` through every argument check and over placements up to
  256 experts on 288 slots.  No GPU call is made.
* ``include/moe.h`` compiled as C11, with its enums 32 bits wide.

Any sanitizer report aborts the driver (``-fno-sanitize-recover=all``), which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_dp_gather_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVERS = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = "/opt/rocm/include"

# Host-side sanitizers for hipcc: each flag behind -Xarch_host, so device code is built as usual.
HOST_SANITIZE = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                 "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer").split()
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nexit {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _env():
    env = dict(os.environ)
    env.update(SAN_ENV)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(DRIVERS, "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=_env(), timeout=120)
    assert "oracle sanitizer driver: ok" in r.stdout


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_cxx_under_asan_ubsan(tmp_path):
    inc = ["-I", INCLUDE, "-I", CSRC]
    objs = []
    # capi.hip holds no kernels: host pass only.  eplb.hip holds kernels, so it is built for
    # gfx950 as usual (the sanitizers apply to its host pass only) and links its device image.
    capi = str(tmp_path / "capi.o")
    _run([HIPCC, "--cuda-host-only", "-O1", "-g", "-std=c++17", *HOST_SANITIZE, *inc,
          "-c", os.path.join(CSRC, "capi.hip"), "-o", capi])
    objs.append(capi)
    eplb = str(tmp_path / "eplb.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SANITIZE, *inc,
          "-c", os.path.join(CSRC, "eplb.hip"), "-o", eplb])
    objs.append(eplb)
    drv = str(tmp_path / "host_driver.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", *HOST_SANITIZE, *inc,
          "-c", os.path.join(DRIVERS, "host_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "host_driver")
    _run([HIPCC, *HOST_SANITIZE, drv, *objs, "-o", exe])
    r = _run([exe], env=_env(), timeout=120)
    assert "host sanitizer driver: ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="gcc or the HIP headers not found")
def test_header_is_c11_with_32_bit_enums(tmp_path):
    src = tmp_path / "header_as_c.c"
    src.write_text('#include "moe.h"\n'
                   '_Static_assert(sizeof(moe_status) == 4, "status is 32 bits");\n'
                   '_Static_assert(sizeof(moe_dtype) == 4, "dtype is 32 bits");\n'
                   '_Static_assert(sizeof(moe_pad_mode) == 4, "pad mode is 32 bits");\n'
                   '_Static_assert(sizeof(moe_route_kind) == 4, "route kind is 32 bits");\n'
                   '_Static_assert(sizeof(moe_gate_mode) == 4, "gate mode is 32 bits");\n'
                   '_Static_assert(sizeof(moe_fp8_act) == 4, "fp8 act is 32 bits");\n'
                   'int main(void) { return 0; }\n')
    _run(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
          "-I", INCLUDE, "-fsyntax-only", str(src)])
