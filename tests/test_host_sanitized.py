"""The library's host code (schedule generator and executor) under the address
and undefined-behaviour sanitizers: `tests/native/fuzz_abi.cpp` drives the C
ABI with random, often invalid, calls on bookkeeping-only handles (no device is
touched) and checks statuses, the op log and the handle's state after every
rejected call.  The kernel objects come from the in-tree build
(`pipeline_schedules_amd/_build`), unsanitized; they are linked, not run."""

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "pipeline_schedules_amd", "csrc")
BUILD = os.path.join(ROOT, "pipeline_schedules_amd", "_build")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no C++ compiler")
    kobjs = sorted(glob.glob(os.path.join(BUILD, "*.hip.o")))
    if not kobjs:
        pytest.skip("kernel objects not built (pipeline_schedules_amd/_build)")
    if not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")):
        pytest.skip("HIP runtime library not found")
    d = tmp_path_factory.mktemp("san")
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN
    objs = []
    for src in (os.path.join(CSRC, "schedule.cpp"), os.path.join(CSRC, "stage.cpp"),
                os.path.join(ROOT, "tests", "native", "fuzz_abi.cpp")):
        obj = str(d / (os.path.basename(src) + ".o"))
        r = subprocess.run([gxx] + flags + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(d / "fuzz_abi")
    r = subprocess.run([gxx] + SAN + objs + kobjs + ["-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                                                     "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("seed", range(1, 7))
def test_abi_fuzz_under_sanitizers(fuzz_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_exe, str(seed), "300"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
