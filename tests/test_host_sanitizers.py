"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two builds in a temporary directory:
- the C ABI library with its host code instrumented (the device code is built too, unoptimised,
  because the host part registers it; it never runs here), loaded into a child process beside
  LLVM's sanitizer runtime, which then runs every host-side test of the ABI: symbol exports, the
  argument checks in their fixed order, the launch planners and their refusals;
- the CPU oracle built with gcc's sanitizers, loaded into a child process beside gcc's runtimes,
  which then runs every oracle pin (unpacking, conversions, exhaustive dequantisation, the
  matmuls, the picks, the affine codes, the hand goldens).

Any sanitizer report ends the child with an error and fails the test. Leak checking is off: the
Python interpreter and the HIP runtime keep allocations until exit by design.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "verify_matmul_amd", "csrc")
SOURCES = ["w4a16_api", "w4a16_gemm", "w4a16_decode", "w4a16_prefill", "w4a16_aux"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


def _run_child(code, preload, timeout):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = _hipcc()
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if hipcc is None or not rts:
        pytest.skip("hipcc or LLVM's sanitizer runtime not found")
    from verify_matmul_amd import _build
    defs = f'-DW4A16_SOURCE_HASH="{_build.source_hash()}"'
    procs = []
    for s in SOURCES:   # one translation unit per process
        cmd = [hipcc, "--offload-arch=gfx950", "-c", "-O1", "-g", "-std=c++17", "-fPIC", "-Xarch_device", "-O0",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-omit-frame-pointer", f"-I{os.path.join(ROOT, 'include')}", defs,
               os.path.join(CSRC, s + ".hip"), "-o", str(tmp_path / (s + ".o"))]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        _, err = p.communicate(timeout=900)
        assert p.returncode == 0, err[-3000:]
    lib = str(tmp_path / "libw4a16_san.so")
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            *[str(tmp_path / (s + ".o")) for s in SOURCES], "-o", lib]
    r = subprocess.run(link, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm   # the host code is instrumented
    code = (f"import sys\nsys.path.insert(0, {ROOT!r})\n"
            "import verify_matmul_amd as vm\n"
            f"vm.lib_path = {lib!r}\n"
            "import pytest\n"
            f"sys.exit(pytest.main([{os.path.join(ROOT, 'tests', 'test_library_cpu.py')!r}, "
            f"{os.path.join(ROOT, 'tests', 'test_library_cpu_decode.py')!r}, '-q', '-x', '-p', 'no:cacheprovider']))\n")
    out = _run_child(code, rts[0], 600)
    assert " passed" in out and "failed" not in out and "error" not in out.lower()


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gcc, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(asan) and os.path.exists(asan) and os.path.isabs(ubsan) and os.path.exists(ubsan)):
        pytest.skip("gcc's sanitizer runtimes not found")
    lib = str(tmp_path / "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "w4a16_oracle.c")
    r = subprocess.run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", src, "-o", lib, "-lm"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_oracle_pins.py", "test_oracle_affine_pins.py",
                                                      "test_golden.py")]
    code = (f"import sys\nsys.path.insert(0, {ROOT!r})\n"
            "import oracle\n"
            f"oracle._LIB_PATH = {lib!r}\n"
            "import pytest\n"
            f"sys.exit(pytest.main({tests!r} + ['-q', '-x', '-p', 'no:cacheprovider']))\n")
    out = _run_child(code, f"{asan} {ubsan}", 900)
    assert " passed" in out and "failed" not in out and "error" not in out.lower()
