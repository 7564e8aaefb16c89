"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI layer (argument checks, the planner, the workspace layout, error
reporting) is rebuilt with both sanitizers on its host code, linked with the
kernel objects of a normal build, and the CPU tests of the planner and of the
ABI run against it in a child process that preloads the sanitizer runtime.
A control library with a planted heap overflow must make the same harness
fail, so that a harness whose sanitizer is not active cannot pass."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_fp32_amd", "csrc")
BUILD = os.path.join(ROOT, "linear_cross_entropy_fp32_amd", "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
# sanitizers on the host side only: each flag applies to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
LINK_SAN = ["-fsanitize=address,undefined", "-shared-libasan"]
HIP_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def _asan_runtime():
    hits = glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _env(runtime):
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def _kernel_objects(tmp):
    objs = [os.path.join(BUILD, f) for f in ("flce_kernels.hip.o", "ce_kernels.hip.o")]
    if all(os.path.exists(o) for o in objs):
        return objs
    objs = []
    for src in ("flce_kernels.hip", "ce_kernels.hip"):
        obj = os.path.join(tmp, src + ".o")
        subprocess.run([HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
                        os.path.join(CSRC, src), "-o", obj], check=True)
        objs.append(obj)
    return objs


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    runtime = _asan_runtime()
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and runtime and shutil.which("nm")):
        pytest.skip("ROCm clang with its sanitizer runtime is needed")
    tmp = str(tmp_path_factory.mktemp("san"))
    api = os.path.join(tmp, "flce_api.o")
    subprocess.run([HIPCC, *HIP_FLAGS, *HOST_SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    "-x", "hip", "-c", os.path.join(CSRC, "flce_api.cpp"), "-o", api], check=True)
    lib = os.path.join(tmp, "libflce_san.so")
    subprocess.run([CLANG, "-shared", "-fPIC", *LINK_SAN, api, *_kernel_objects(tmp),
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib],
                   check=True)
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "sanitizer hooks missing"
    return tmp, lib, runtime


def _child(tmp, code, runtime):
    script = os.path.join(tmp, "child.py")
    with open(script, "w") as fh:
        fh.write(code)
    return subprocess.run([sys.executable, script], capture_output=True, text=True,
                          env=_env(runtime), timeout=600)


def test_planner_and_abi_tests_pass_under_sanitizers(sanitized):
    tmp, lib, runtime = sanitized
    code = f"""
import sys
sys.path.insert(0, {ROOT!r})
from linear_cross_entropy_fp32_amd import _binding
_binding.LIB_PATH = {lib!r}
maps = open('/proc/self/maps').read()
assert 'libclang_rt.asan' in maps, 'sanitizer runtime not loaded'
import pytest
rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu',
                  {os.path.join(ROOT, 'tests', 'test_plan_cpu.py')!r},
                  {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}, '-k', 'not hazard'])
assert open('/proc/self/maps').read().count({os.path.basename(lib)!r}) > 0, 'library not loaded'
sys.exit(int(rc))
"""
    r = _child(tmp, code, runtime)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_harness_catches_a_planted_overflow(sanitized):
    tmp, _, runtime = sanitized
    src = os.path.join(tmp, "control.cpp")
    with open(src, "w") as fh:
        fh.write('extern "C" int control_read(int i) {\n'
                 '  int* p = new int[4]();\n  int v = p[i];\n  delete[] p;\n  return v;\n}\n')
    lib = os.path.join(tmp, "libcontrol.so")
    subprocess.run([CLANG, "-shared", "-fPIC", "-g", *LINK_SAN, src, "-o", lib], check=True)
    code = f"""
import ctypes
L = ctypes.CDLL({lib!r})
L.control_read(3)
L.control_read(4)
print('not caught')
"""
    r = _child(tmp, code, runtime)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stdout + r.stderr[-2000:]
