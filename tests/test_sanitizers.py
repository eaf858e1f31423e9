"""CPU sanitizer builds: the C oracle and the C ABI's host-side validation.

* The oracle is compiled with AddressSanitizer and UndefinedBehaviorSanitizer
  (gcc) and every pin of tests/oracle_pins.py runs against it; two copies with
  a planted heap overflow and a planted signed overflow must be stopped by the
  sanitizers, which shows they are live in this set-up.
* gqa_api.hip (argument validation, work map, workspace layout) is compiled
  with both sanitizers on its host code only, linked against stub launchers
  (no kernel runs without a GPU), and tests/test_abi_cpu.py runs against it.

The instrumented libraries are loaded into an uninstrumented Python, so each
run preloads its compiler's AddressSanitizer runtime; leak detection is off
(the interpreter keeps its memory to the end).
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE_SRC = os.path.join(ROOT, "oracle", "gqa_oracle.c")
CSRC = os.path.join(ROOT, "grouped_query_attention_03_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"

GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "OMP_NUM_THREADS": "2"}


def _runtime(cmd):
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout.strip()


def _build_oracle(tmp_path, source, name):
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(source)
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-ffp-contract=off", *GCC_SAN, str(src), "-o", str(lib), "-lm"], check=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, LD_PRELOAD=_runtime(["gcc", "-print-file-name=libasan.so"]), **ENV_SAN)
    return subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), str(lib)],
                          capture_output=True, text=True, env=env, timeout=600)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    r = _run_pins(_build_oracle(tmp_path, open(ORACLE_SRC).read(), "oracle_san"))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "pins failed: 0 of" in r.stdout


PLANTED = {
    # one score written past the end of its scratch row
    "heap_overflow": ("    double z = 0.0;\n    for (int j = 0; j < n_vis; ++j) {",
                      "    double z = 0.0;\n    scores[n_vis] = 0.0;\n"
                      "    for (int j = 0; j < n_vis; ++j) {",
                      "AddressSanitizer"),
    # a signed int pushed past INT_MAX
    "signed_overflow": ("    if (n_vis <= 0) return;\n",
                        "    if (n_vis <= 0) return;\n"
                        "    { volatile int big = 2147483647; big = big + (n_vis > 0); }\n",
                        "runtime error"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(PLANTED))
def test_sanitizers_stop_a_planted_error(tmp_path, name):
    text = open(ORACLE_SRC).read()
    old, new, marker = PLANTED[name]
    assert text.count(old) == 1
    r = _run_pins(_build_oracle(tmp_path, text.replace(old, new), name))
    assert r.returncode != 0 and marker in r.stdout + r.stderr, r.stdout[-2000:] + r.stderr[-2000:]


STUBS = """#include "gqa_kernels.h"
namespace gqa {
int launch_prefill_bf16(const PrefillArgs &, int, bool, hipStream_t) { return -1; }
int launch_prefill_f32(const PrefillArgs &, int, bool, hipStream_t) { return -1; }
int launch_rope_k_bf16(const RopeArgs &, int, hipStream_t) { return -1; }
int launch_decode_bf16(const DecodeArgs &, int, hipStream_t) { return -1; }
}
"""

RUN_ABI = """import sys
sys.path.insert(0, {root!r})
import grouped_query_attention_03_amd as gqa
gqa.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {tests!r}]))
"""


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs hipcc")
def test_abi_validation_under_address_and_undefined_sanitizers(tmp_path):
    stubs = tmp_path / "stubs.hip"
    stubs.write_text(STUBS)
    lib = tmp_path / "libgqa_san.so"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
                        "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                        "-I", CSRC, "-shared", os.path.join(CSRC, "gqa_api.hip"), str(stubs),
                        "-o", str(lib)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    script = tmp_path / "run_abi.py"
    script.write_text(RUN_ABI.format(root=ROOT, tests=os.path.join(HERE, "test_abi_cpu.py")))
    env = dict(os.environ,
               LD_PRELOAD=_runtime([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"]),
               **ENV_SAN)
    r = subprocess.run([sys.executable, str(script), str(lib)], capture_output=True, text=True,
                       env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
