"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:

- the library's planner and argument validation (dg_api.hip, dg_shapes.hip,
  dg_noalloc.hip built for the host with the sanitizers, kernel launches
  replaced by stubs that are never reached): dg_select_config over a grid of
  kinds and shapes with the plan's invariants, and every entry point's
  rejection of bad arguments;
- the oracle (oracle/*.c): every entry point on small ragged inputs;
- the GEMM kernel's buffer-resource range arithmetic (csrc/dg_rsrc.h): its
  boundary cases pinned (an empty range never wraps, a range moved along a
  row ends where it did).

Each driver exits non-zero on a failed check, and the sanitizers abort on the
first report (-fno-sanitize-recover=all)."""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "moe_grouped_gemm_x128_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _check_clean(r):
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "bad=0" in out, out


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_planner_and_validation_under_sanitizers(workdir):
    lib = os.path.join(workdir, "libdg_plan_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared", *HOST_SAN,
          "-I", os.path.join(ROOT, "include"), "-o", lib,
          os.path.join(CSRC, "dg_api.hip"), os.path.join(CSRC, "dg_shapes.hip"),
          os.path.join(CSRC, "dg_noalloc.hip"), os.path.join(SAN, "launch_stubs.hip")])
    exe = os.path.join(workdir, "planner_driver")
    _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
          os.path.join(SAN, "planner_driver.c"), "-o", exe, "-L", workdir, "-ldg_plan_san",
          f"-Wl,-rpath,{workdir}", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    _check_clean(_run([exe], timeout=120))


def test_oracle_under_sanitizers(workdir):
    exe = os.path.join(workdir, "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "dg_oracle.c"), os.path.join(ROOT, "oracle", "dg_quant_oracle.c"),
          "-lm", "-o", exe])
    _check_clean(_run([exe], timeout=120, env=dict(os.environ, OMP_NUM_THREADS="4")))


def test_resource_range_pins_under_sanitizers(workdir):
    exe = os.path.join(workdir, "rsrc_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", *HOST_SAN, "-o", exe,
          os.path.join(SAN, "rsrc_driver.hip")])
    _check_clean(_run([exe], timeout=120))
