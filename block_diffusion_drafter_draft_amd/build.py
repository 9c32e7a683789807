"""Build libdbd.so (HIP, gfx950 only) in-tree with hipcc.

python -m block_diffusion_drafter_draft_amd.build   # or build() from Python
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdbd.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# Translation units and their extra flags.  The vocabulary kernels carry the integer-exact
# weights and must not contract multiply-add pairs.
SOURCES = {
    "k_rowops.hip": [],
    "k_gemm.hip": [],
    # the deep-ring tiles keep their MFMA accumulators in VGPRs (see the file's header)
    "k_gemm_deep.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the attention accumulators are rescaled by the online softmax: keep them in VGPRs
    "k_attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "k_vocab.hip": ["-ffp-contract=off"],
    "runtime.hip": [],
}


def _compile(src, extra, verbose):
    obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


# Translation units whose kernels issue LDS reads as inline assembly: their device assembly is
# kept in _build/ so that tests/test_asm_lds_reads.py can check every such read is waited for
# before its registers are touched.
ASM_LISTED = ["k_gemm_deep.hip"]


def _device_asm(src, extra):
    out = os.path.join(OBJ_DIR, src.replace(".hip", ".s"))
    cmd = [HIPCC, *COMMON, *extra, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stdout}{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdbd.so next to this file."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(ASM_LISTED),
                                            os.cpu_count() or 4)) as ex:
        asm = [ex.submit(_device_asm, s, SOURCES[s]) for s in ASM_LISTED]
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
        for f in asm:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
