"""The oracle and the library's host side (argument validation, planning and
workspace sizing of every entry point) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.  Both are rebuilt with clang's
sanitizers into a temporary directory -- the oracle from oracle.c, the host
code of dattn.hip (linked with the library's kernel objects, whose device code
is not instrumented) -- and the oracle's pin tests and the C-ABI tests run
against those builds in a child process with the sanitizer runtime preloaded.
The first sanitizer report aborts the child, which fails this test (the child
runs pytest with -s, so a report of a child that dies inside a test reaches its
stderr).  No GPU is touched: every ABI test stops in host-side validation or
sizing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
CHILD_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_append_pins.py", "tests/test_oracle_tiered_f16_pins.py",
               "tests/test_oracle_ring_pins.py", "tests/test_oracle_multi_query_pins.py", "tests/test_abi_cpu.py"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("clang from ROCm is not installed")
    from int8_quantized_kv_amd import build as B
    tmp = tmp_path_factory.mktemp("san")
    kernel_objs = [os.path.join(B.OBJDIR, name + ".o") for name, _, _ in B.UNITS if name != "dattn"]
    if not all(os.path.exists(o) for o in kernel_objs):
        B.build()
    oracle_so = str(tmp / "liboracle_san.so")
    _run([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-shared-libsan", "-fopenmp", "-std=c11", "-shared", "-fPIC",
          os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_so, "-lm"])
    host_obj = str(tmp / "dattn_san.o")
    # host-only instrumentation: each sanitizer flag applies to the host pass alone
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan"]
    _run([B.hipcc(), f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-c", *san,
          "-I", B.INCLUDE, "-I", B.CSRC, os.path.join(B.CSRC, "dattn.hip"), "-o", host_obj])
    lib_so = str(tmp / "libdattn_san.so")
    _run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *san, host_obj, *kernel_objs, "-o", lib_so])
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    return dict(oracle=oracle_so, lib=lib_so, runtime=rt)


def test_oracle_and_host_code_under_asan_and_ubsan(sanitized):
    env = dict(os.environ, LD_PRELOAD=sanitized["runtime"], ORACLE_LIB_OVERRIDE=sanitized["oracle"],
               DATTN_LIBRARY_OVERRIDE=sanitized["lib"], OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *CHILD_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out


def test_planted_overflow_in_the_oracle_is_reported(sanitized, tmp_path):
    """Negative control: a copy of oracle.c whose Q copy runs one element past
    its buffer must make the same child run fail with an AddressSanitizer
    report, so a pass above means the instrumentation was live."""
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "for (int32_t d = 0; d < D; ++d) qv[d] = (double)q[qrow * D + d];"
    assert src.count(good) == 1
    bad_c = tmp_path / "oracle_bad.c"
    bad_c.write_text(src.replace(good, "for (int32_t d = 0; d <= D; ++d) qv[d] = (double)q[qrow * D + (d % D)];"))
    bad_so = str(tmp_path / "liboracle_bad.so")
    _run([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-shared-libsan", "-fopenmp",
          "-std=c11", "-shared", "-fPIC", str(bad_c), "-o", bad_so, "-lm"])
    env = dict(os.environ, LD_PRELOAD=sanitized["runtime"], ORACLE_LIB_OVERRIDE=bad_so, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stdout + r.stderr
