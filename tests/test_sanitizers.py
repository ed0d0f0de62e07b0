"""AddressSanitizer and UndefinedBehaviorSanitizer runs on the CPU.

* The C++ oracle (oracle/nanospec_oracle.cpp) is built with g++ and both
  sanitizers together with tests/native/oracle_checks.cpp, which drives every
  exported function over edge sizes.
* The library's host code (argument checks, launch planning, workspace
  layout) is built from the HIP sources with the sanitizers on the host side
  only (device code unoptimised: it is never run here), and driven by
  tests/native/abi_host_checks.cpp: size queries at and past every limit,
  argument errors, and calls that pass the checks with placeholder device
  addresses, which plan the launch and stop at the first HIP call for want
  of a device.

Any report from either sanitizer fails the run.  Both builds take about
15 s.  The host-library run needs a machine without a GPU (the placeholder
addresses must never reach a device), so it is skipped where /dev/kfd exists.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "dynamic_vocab_draft_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SOURCES = ["state.hip", "gather.hip", "packed.hip", "draft.hip", "tree.hip", "prefill.hip"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=timeout)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{p.stdout[-6000:]}"
    return p.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["g++", "-O1", "-g", "-std=c++17", "-fopenmp", *SAN,
          os.path.join(ROOT, "oracle", "nanospec_oracle.cpp"), os.path.join(NATIVE, "oracle_checks.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    assert "oracle checks passed" in _run([exe], env=env)


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="placeholder device addresses: run only without a GPU")
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_host_library_under_asan_ubsan(tmp_path):
    host = [f for flag in ["-O1", "-g", *SAN] for f in ("-Xarch_host", flag)]
    common = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-Xarch_device", "-O0", *host, f"-I{INCLUDE}", f"-I{CSRC}"]
    objs = [str(tmp_path / (s[:-4] + ".o")) for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda i: _run([HIPCC, *common, "-c", os.path.join(CSRC, SOURCES[i]), "-o", objs[i]]),
                    range(len(SOURCES))))
    lib = str(tmp_path / "libnanospec_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", lib])
    exe = str(tmp_path / "abi_host_checks")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
          f"-I{ROCM}/include", os.path.join(NATIVE, "abi_host_checks.cpp"), lib, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{ROCM}/lib", "-o", exe])
    # The HIP runtime keeps allocations until exit, so leak checking is off.
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    assert "host checks passed" in _run([exe], env=env, timeout=300)
