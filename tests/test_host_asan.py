"""Host-side memory safety of the C ABI: the library's sources are built
with AddressSanitizer on the host half only (the device code is compiled as
usual and never run here), and a plain C driver (tests/host_asan/) calls
every host-only path: geometry and placement queries, tile offsets,
argument checks that return before a launch, and the block-pool allocator
under a seeded random sequence of reservations and releases.  Any invalid
access or leak on the host side fails the test."""

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

from tests.helpers import ROOT

CSRC = os.path.join(ROOT, "long_context_decode_split_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_asan", "abi_host_driver.c")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_host_paths_under_address_sanitizer(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address",
               f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libhelixdecode_asan.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-o", lib, *objs], check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_host_driver")
    subprocess.run([CLANG, "-std=c99", "-Wall", "-Werror", "-g", "-fsanitize=address", f"-I{INCLUDE}", DRIVER,
                    "-o", exe, f"-L{tmp_path}", "-lhelixdecode_asan", f"-Wl,-rpath,{tmp_path}"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr[-4000:]
