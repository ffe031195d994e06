"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU.

1. The oracle is rebuilt with gcc's ASan and UBSan (UB aborts) and its pin
   suites run against that build in a child process with gcc's ASan runtime
   preloaded (Python itself is not instrumented).
2. The NVFP4 library is rebuilt with the sanitizers on its host code only
   (every hipcc sanitizer flag sits behind -Xarch_host; the device code is
   compiled as usual but never launched here), and tests/test_abi.py -- every
   declared symbol exported, every invalid-argument path returning its status
   before any HIP call -- runs against it with clang's ASan runtime (which
   carries the UBSan handlers) preloaded.

Both builds go to a temporary directory; neither touches the in-tree
libraries.  A child process that hits a sanitizer report exits non-zero."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def _gcc_asan_runtime():
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    path = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run_child(code, preload, timeout):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    rt = _gcc_asan_runtime()
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "nvfp4_oracle.c"),
                    "-o", lib, "-lm"], check=True)
    suites = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    code = (
        "import sys; sys.path[:0] = ['.', 'tests']\n"
        "import oracle\n"
        f"oracle._LIB_PATH = {lib!r}\n"
        "import pytest\n"
        f"rc = pytest.main(['-x', '-q', '-s', '-p', 'no:cacheprovider', *{suites!r}])\n"
        "assert oracle.lib()._name == oracle._LIB_PATH\n"
        "sys.exit(int(rc))\n")
    out = _run_child(code, rt, timeout=600)
    assert " passed" in out


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang",
             "-target-feature", "-Xclang", "-packed-fp32-ops", *san, "-Xarch_host",
             "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-I",
             os.path.join(ROOT, "include")]
    srcs = sorted(glob.glob(os.path.join(ROOT, "bit_quantized_gemm_nvfp4_amd", "csrc", "*.hip")))
    procs = []
    objs = []
    for s in srcs:
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        objs.append(o)
        procs.append(subprocess.Popen([HIPCC, *flags, "-c", s, "-o", o], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT))
    for p in procs:
        out, _ = p.communicate(timeout=900)
        assert p.returncode == 0, out.decode(errors="replace")[-3000:]
    lib = str(tmp_path / "libnvfp4_san.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-Xarch_host",
                    "-shared-libsan", *objs, "-o", lib], check=True, capture_output=True)
    code = (
        "import sys; sys.path[:0] = ['.', 'tests']\n"
        "import bit_quantized_gemm_nvfp4_amd as nv\n"
        f"nv._LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "rc = pytest.main(['-x', '-q', '-s', '-p', 'no:cacheprovider', 'tests/test_abi.py'])\n"
        "assert nv.lib()._name == nv._LIB_PATH\n"
        "sys.exit(int(rc))\n")
    out = _run_child(code, rt, timeout=600)
    assert " passed" in out
