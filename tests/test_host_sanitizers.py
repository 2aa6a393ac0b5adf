"""The host code of the C-ABI (pkv_api.cpp: argument checks, plans, caches,
the block pool) under AddressSanitizer and UndefinedBehaviorSanitizer: a copy
of libpkv.so whose pkv_api.cpp is built with both (host side only; the kernels
are the ordinary objects), loaded by a Python interpreter that carries the
sanitizer runtimes, runs test_abi.py and test_block_pool.py.  Any report
fails the run.  CPU only."""
import glob
import os
import subprocess
import sysconfig

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_blocks_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
HIPCC = os.path.join(ROCM, "bin", "hipcc")


def _objects():
    # the kernels' objects of the ordinary build (build() made them)
    objs = sorted(glob.glob(os.path.join(PKG, "_build", "*.o")))
    return [o for o in objs if not os.path.basename(o).startswith("pkv_api")]


def _have_toolchain():
    rt = glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.a"))
    inc = sysconfig.get_paths()["include"]
    return bool(rt) and os.path.exists(CLANG) and os.path.exists(HIPCC) and os.path.exists(os.path.join(inc, "Python.h"))


@pytest.mark.skipif(not _have_toolchain(), reason="no clang sanitizer runtime, hipcc or Python headers")
@pytest.mark.skipif(not _objects(), reason="kernel objects not built (run __graft_entry__.build())")
def test_abi_and_pool_under_asan_and_ubsan(tmp_path):
    sys_flags = ["-O1", "-g", "-fno-omit-frame-pointer"]
    api_obj = str(tmp_path / "pkv_api_san.o")
    # host-side instrumentation only: each -fsanitize= goes to the host pass
    cmd = [HIPCC, "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops"] + sys_flags + ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                              "-fsanitize=undefined", "-x", "hip", "-c",
                                              os.path.join(PKG, "csrc", "pkv_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libpkv_san.so")
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", lib] + _objects() + [api_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    py = str(tmp_path / "python_san")
    libdir = sysconfig.get_config_var("LIBDIR")
    ver = sysconfig.get_config_var("LDVERSION")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined"] + sys_flags +
                       ["-I", sysconfig.get_paths()["include"], "-x", "c",
                        os.path.join(ROOT, "tests", "host_sanitize", "python_main.c"), "-o", py, "-L", libdir,
                        f"-lpython{ver}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env.update(PKV_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([py, "-m", "pytest", "tests/test_abi.py", "tests/test_block_pool.py", "-q", "-s", "-p",
                        "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error:" not in out and "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out and "failed" not in out, out[-3000:]
