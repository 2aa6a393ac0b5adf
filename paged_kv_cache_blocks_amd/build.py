"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_blocks_amd.build      (or build() from Python)

Objects are compiled in parallel into paged_kv_cache_blocks_amd/_build/ and
linked into paged_kv_cache_blocks_amd/libpkv.so.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")
SOURCES = ["kv_ops.hip", "decode.hip", "decode_mfma.hip", "prefill.hip", "prefill_fp8.hip", "device_check.hip", "pkv_api.cpp"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

# Packed FP32 instructions are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
# The prefill and matrix-core decode kernels keep their MFMA accumulators in
# ordinary VGPRs: they need fewer than 256 registers that way, which leaves
# room for two waves per SIMD, and the softmax and the output rescale read the
# tiles without accumulator-register copies (about 100 copy instructions per
# 32-token decode chunk otherwise).
# The prefill kernels are also built without NaN semantics: their softmax
# sees no NaN (masked scores are -inf, V rows past the keys are zeroed, block
# scales of dead halves are 0), so the row maxima need not canonicalise each
# score before v_max (12-16 instructions per 16-row tile; 1.5-2 % faster).
EXTRA = {"prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "prefill_fp8.hip": ["-fno-honor-nans"],
         "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [_hipcc()] + FLAGS + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj, msg


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, msg in results:
            if msg.strip():
                print(msg)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
