"""CPU: the host-side code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds, into a temporary directory, the fp64 oracle and the input generator
with clang and -fsanitize=address,undefined, and libfr with its host code
sanitized (-Xarch_host before each flag, so device code is built as usual:
GPU sanitizers are not used). Then runs the CPU tests that exercise that
code - the oracle's pins, the planner and argument checks of the C ABI, the
configuration search, the comparison rules and the byte formulas - in a
child process with the sanitizer runtime preloaded and the three libraries
swapped in (FR_LIB, ORACLE_LIB, SYNTH_LIB). Any sanitizer report fails it.
"""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/lib/llvm/bin/clang"
TESTS = ["tests/test_oracle_pins.py", "tests/test_host.py", "tests/test_tune_search.py",
         "tests/test_check_rules.py", "tests/test_bench_bytes.py"]


def asan_runtime():
    found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(not os.path.exists(CLANG) or asan_runtime() is None, reason="clang sanitizer runtime not found")
def test_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    import synth
    spec = importlib.util.spec_from_file_location("fr_build", os.path.join(ROOT, "pointwise_reduction_amd", "build.py"))
    fr_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(fr_build)

    lib_oracle = str(tmp_path / "liboracle_san.so")
    lib_synth = str(tmp_path / "libsynth_san.so")
    lib_fr = str(tmp_path / "libfr_san.so")
    oracle.build(out=lib_oracle, cc=CLANG, extra=oracle.SANITIZE_FLAGS)
    synth.build(out=lib_synth, cc=CLANG, extra=oracle.SANITIZE_FLAGS)
    fr_build.build(lib=lib_fr, build_dir=str(tmp_path / "fr"), host_extra=fr_build.HOST_SANITIZE_FLAGS)

    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "FR_LIB": lib_fr, "ORACLE_LIB": lib_oracle, "SYNTH_LIB": lib_synth,
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"] + TESTS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
