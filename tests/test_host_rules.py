"""Host-side shape rules of the launchers (csrc/host_rules.h), compiled with the system C++
compiler and checked on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RULES = os.path.join(ROOT, "block_diffusion_drafter_draft_amd", "csrc", "host_rules.h")


def test_resid_norm_fusion_predicate(tmp_path):
    """The split-K reduction fuses the next RMSNorm only for rows one 1,024-thread workgroup
    covers with whole four-float vectors, stored densely: up to 8,192 columns, a multiple of 4,
    row stride equal to the width.  Wider, ragged or strided rows fall back to the plain
    reduction plus a separate norm."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    cases = [(4096, 4096, 1), (8192, 8192, 1), (8196, 8196, 0), (16384, 16384, 0),
             (4094, 4094, 0), (4, 4, 1), (0, 0, 0), (-4, -4, 0), (4096, 4160, 0),
             (2880, 2880, 1), (3584, 3584, 1)]
    src = [f'#include "{RULES}"', "#include <cstdio>", "int main() {"]
    src.append("  static_assert(dbd::kResidNormMaxCols == 8192, \"coverage\");")
    for n, ld, _ in cases:
        src.append(f'  std::printf("%d\\n", (int)dbd::resid_norm_fits({n}, {ld}));')
    src.append("  return 0;\n}")
    f = tmp_path / "probe.cpp"
    f.write_text("\n".join(src))
    exe = tmp_path / "probe"
    subprocess.run([cxx, "-std=c++17", str(f), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert [int(x) for x in out] == [c[2] for c in cases]
