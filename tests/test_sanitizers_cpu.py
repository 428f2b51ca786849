"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only), and its pins run against that build in a subprocess with the
sanitizer runtimes preloaded: an out-of-bounds access, a use after free or an
undefined operation anywhere the pins reach ends the run with a report."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvc_oracle.c")


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
                        "-o", lib, SRC, "-lm"], check=True)
        env = dict(os.environ, KVC_ORACLE_LIB=lib, LD_PRELOAD=asan + ":" + ubsan,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                       if f.startswith("test_oracle_")) + ["tests/test_golden.py"]
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                            *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        out = r.stdout[-3000:] + r.stderr[-3000:]
        assert r.returncode == 0, out
        assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
        assert " passed" in r.stdout


def _clang_asan_runtime():
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_library_host_code_under_asan_and_ubsan():
    # every libkvc source compiled with AddressSanitizer and UBSan on its host code only
    # (the GPU code is built as usual), then the CPU-only checks of the C ABI -- argument
    # validation of every entry point, options, workspace sizing, the host budget
    # function -- run against it in a subprocess with clang's sanitizer runtime preloaded
    from token_scoring_eviction_amd import build
    runtime = _clang_asan_runtime()
    if runtime is None or (shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC)):
        pytest.skip("hipcc or clang's sanitizer runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=" + build.ARCH, "-I", build.INCLUDE,
             "-I", build.CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    import concurrent.futures as cf
    import glob
    with tempfile.TemporaryDirectory() as tmp:
        srcs = sorted(glob.glob(os.path.join(build.CSRC, "*.hip")))

        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            subprocess.run([build.HIPCC, *flags, *san, "-c", src, "-o", obj], check=True, capture_output=True)
            return obj

        with cf.ThreadPoolExecutor(max_workers=8) as ex:
            objs = list(ex.map(compile_one, srcs))
        lib = os.path.join(tmp, "libkvc_san.so")
        subprocess.run([build.HIPCC, "-shared", "-fPIC", "--offload-arch=" + build.ARCH, *san, "-o", lib, *objs],
                       check=True, capture_output=True)
        runner = ("import sys; sys.path.insert(0, %r)\n"
                  "from token_scoring_eviction_amd import kvc\n"
                  "kvc.LIB_PATH = %r; kvc.load(kvc.LIB_PATH)\n"
                  "import pytest\n"
                  "sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider', "
                  "'tests/test_abi_cpu.py', 'tests/test_abi_errors_cpu.py', 'tests/test_budgets_host.py']))\n"
                  % (ROOT, lib))
        env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
        out = r.stdout[-3000:] + r.stderr[-3000:]
        assert r.returncode == 0, out
        assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out
        assert " passed" in r.stdout
