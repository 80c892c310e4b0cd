"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The CPU oracle (oracle/moba_oracle.c) with a driver that runs every entry
  point on small shapes (bf16 and fp32, GQA, a short last block, top-k 1 and
  top-k above the block count, a refused selection entry, argument errors).
* The GPU library's host side: every source is built with the sanitizers on
  the host pass (the device pass is built without optimisation: it is never
  run here), linked with a driver that calls the workspace sizing over many
  shapes and every argument check that must refuse a call before any HIP
  call.  Leak checking is off for this one: the HIP runtime keeps its own
  allocations until exit.
"""
import glob
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_sparse_attention_moba_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    d = tmp_path_factory.mktemp("sanitize")
    yield str(d)
    shutil.rmtree(str(d), ignore_errors=True)


def test_oracle_under_asan_ubsan(build_dir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = os.path.join(build_dir, "oracle_san")
    rc, log = run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                   "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                   "-o", exe, os.path.join(ROOT, "oracle", "moba_oracle.c"),
                   os.path.join(HERE, "oracle_driver.c"), "-lm"])
    assert rc == 0, log
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    rc, log = run([exe], env=env)
    assert rc == 0 and "ok" in log, log


def test_library_host_paths_under_asan_ubsan(build_dir):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    common = ["--offload-arch=gfx950", "-std=c++17", "-Xarch_host", "-O1", "-Xarch_device", "-O0",
              "-g", "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", *HOST_SAN, "-I", INCLUDE, "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        extra = ["-x", "hip"] if src.endswith(".cpp") else []
        rc, log = run([HIPCC, *common, *extra, "-c", src, "-o", obj])
        assert rc == 0, log
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(HERE, "abi_driver.cpp")]
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(build_dir, "abi_san")
    rc, log = run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, "-o", exe, *objs])
    assert rc == 0, log
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    rc, log = run([exe], env=env)
    assert rc == 0 and "ok" in log, log
