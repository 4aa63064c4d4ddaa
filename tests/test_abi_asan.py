"""The C ABI's argument validation under AddressSanitizer, on the CPU.

Every library source is compiled with AddressSanitizer on its host code only
(device code is built as usual and never runs here), linked with the driver
``tests/asan/abi_validation.cpp``, and run: each entry point is called with
arguments it must reject before any device work (invalid problems, null or
misaligned pointers, short workspaces, out-of-range parameters), the statuses
are checked, and AddressSanitizer reports any invalid memory access in the
validation code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_sampling_verification_markov_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "asan", "abi_validation.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# AddressSanitizer on the host pass only (-Xarch_host right before the flag)
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr[-3000:]}")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC) or shutil.which("nm") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("abi_asan")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [str(out / (os.path.basename(s)[:-4] + ".o")) for s in srcs]
    cmds = [[HIPCC, *FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    drv = str(out / "driver.o")
    cmds.append([HIPCC, *FLAGS, "-x", "hip", "-c", DRIVER, "-o", drv])
    with ThreadPoolExecutor(min(8, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    exe = str(out / "abi_validation")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-o", exe, drv, *objs,
          "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"])
    return exe


def test_validation_paths_under_address_sanitizer(driver):
    # the objects really are instrumented
    syms = subprocess.run(["nm", driver], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:], r.stderr[-2000:])
