"""Host-code sanitizer tier (CPU only, no GPU needed).

Two builds with AddressSanitizer and UndefinedBehaviorSanitizer on host code:

- the oracle's C sources (gcc), exercised by every oracle pin test;
- the library's host layer (sma_host.cpp: argument checks, size arithmetic,
  planner, workspace sizes; hipcc with the sanitizers on the host pass only),
  linked with the ordinary device objects and exercised by the ABI tests.

Each runs in a child process with the sanitizer runtime preloaded, since the
test runner itself is not instrumented. A positive control shows that the same
set-up reports an out-of-bounds read, so that a clean run means something.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "scaled_masked_attention_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PIN_TESTS = ["tests/test_oracle_pins.py", "tests/test_rows_oracle_pins.py",
             "tests/test_masked_oracle_pins.py", "tests/test_bwd_oracle_pins.py",
             "tests/test_bwd_masked_oracle_pins.py"]


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run_child(code, preload, extra_env=None, timeout=900):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra_env or {})
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def _assert_clean(r, what):
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, f"{what}: AddressSanitizer report\n{out[-4000:]}"
    assert "runtime error:" not in out, f"{what}: UndefinedBehaviorSanitizer report\n{out[-4000:]}"
    assert r.returncode == 0, f"{what}: exit {r.returncode}\n{out[-4000:]}"


@pytest.fixture(scope="module")
def sandir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    return tmp_path_factory.mktemp("sanitize")


def test_sanitizer_setup_reports_a_planted_overflow(sandir):
    """Positive control: a one-past-the-end read in a gcc-built library, loaded the same way
    as the oracle, is reported."""
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is missing")
    src = sandir / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int n) { int* a = (int*)malloc(n * sizeof(int));\n"
                   "  for (int i = 0; i < n; ++i) a[i] = i;\n"
                   "  int s = a[n]; free(a); return s; }\n")
    lib = sandir / "libplanted.so"
    subprocess.check_call(["gcc", "-O0", "-g", "-fsanitize=address", "-fPIC", "-shared", str(src),
                           "-o", str(lib)])
    r = _run_child(f"import ctypes; ctypes.CDLL({str(lib)!r}).planted(8)", asan)
    assert "heap-buffer-overflow" in r.stdout + r.stderr


def test_oracle_pins_under_asan_and_ubsan(sandir):
    asan = _gcc_runtime("libasan.so")
    if asan is None or _gcc_runtime("libubsan.so") is None:
        pytest.skip("gcc's sanitizer runtimes are missing")
    lib = sandir / "liboracle_san.so"
    srcs = sorted(glob.glob(os.path.join(ROOT, "oracle", "*.c")))
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
                           "-fPIC", "-shared"] + srcs + ["-o", str(lib), "-lm"])
    code = ("import sys; sys.path[:0] = ['.', 'tests']\n"
            "import oracle\n"
            f"oracle._lib = oracle.load({str(lib)!r})\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-p', 'no:xdist'] + {PIN_TESTS!r}))\n")
    r = _run_child(code, asan)
    _assert_clean(r, "oracle pins")
    assert " passed" in r.stdout


def test_host_layer_abi_tests_under_asan_and_ubsan(sandir):
    """sma_host.cpp built with the sanitizers on its host pass (undefined behaviour traps),
    linked with the library's device objects, then the ABI tests load it."""
    asan = _clang_asan_runtime()
    if asan is None or not os.path.exists(HIPCC):
        pytest.skip("hipcc or clang's AddressSanitizer runtime is missing")
    from scaled_masked_attention_amd import build as sma_build

    objs = [os.path.join(sma_build.BUILD, os.path.splitext(s)[0] + ".o")
            for s in sma_build.SOURCES if s != "sma_host.cpp"]
    if not all(os.path.exists(o) for o in objs):
        sma_build.build()
    host_obj = sandir / "sma_host_san.o"
    subprocess.check_call([HIPCC, "--offload-arch=" + sma_build.ARCH, "-O1", "-g", "-std=c++17",
                           "-fPIC", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-I", sma_build.INCLUDE, "-I", sma_build.CSRC,
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fsanitize-trap=undefined",
                           "-Xarch_host", "-fno-omit-frame-pointer",
                           "-x", "hip", "-c", os.path.join(sma_build.CSRC, "sma_host.cpp"),
                           "-o", str(host_obj)], stderr=subprocess.DEVNULL)
    lib = sandir / "libsma_san.so"
    subprocess.check_call([HIPCC, "--offload-arch=" + sma_build.ARCH, "-shared", "-fPIC",
                           "-shared-libsan", "-Xarch_host", "-fsanitize=address", "-o", str(lib),
                           str(host_obj)] + objs)
    nm = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm, "the host layer is not instrumented"
    code = ("import sys; sys.path[:0] = ['.', 'tests']\n"
            "import scaled_masked_attention_amd as sma\n"
            f"sma.LIB_PATH = {str(lib)!r}\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-p', 'no:xdist', "
            "'tests/test_abi.py']))\n")
    r = _run_child(code, asan)
    _assert_clean(r, "ABI tests")
    assert " passed" in r.stdout
