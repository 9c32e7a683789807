"""The library's host code (argument validation, workspace sizing and carving, the tile and split
planners) built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side only, and
driven by tests/host_sanitize_driver.cpp: thousands of workspace queries over the workload shapes
and every validation path, all of which return before any HIP call.  CPU only."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_drafter_draft_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# each -fsanitize= applies to the host compilation only (-Xarch_host right before it)
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
SOURCES = {"runtime.hip": [], "k_gemm.hip": [], "k_rowops.hip": [],
           "k_vocab.hip": ["-ffp-contract=off"],
           "k_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
           "k_gemm_deep.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    if not os.path.exists(HIPCC) or shutil.which("g++") is None:
        pytest.skip("hipcc not available")
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang",
              "-target-feature", "-Xclang", "-packed-fp32-ops", "-I",
              os.path.join(ROOT, "include"), *SAN]

    def compile_one(item):
        src, extra = item
        obj = str(tmp_path / (src + ".o"))
        r = subprocess.run([HIPCC, *common, *extra, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 2)) as ex:
        objs = list(ex.map(compile_one, SOURCES.items()))
    drv = str(tmp_path / "driver.o")
    r = subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                        *SAN, "-c", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
                        "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, drv, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
