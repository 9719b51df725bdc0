"""The oracle's self-tests (the pins) against an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c, in a child process with the ASan runtime preloaded (Python itself is not
instrumented; leak checks are off; the child runs without pytest's output capture, which
would swallow a sanitizer report written just before the process exits).  Any out-of-bounds
access or undefined behaviour in the oracle fails the run."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_pins_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no ASan runtime")
    lib = str(tmp_path / "liboracle_asan.so")
    oracle.build(extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                              "-fno-omit-frame-pointer", "-g"), out=lib)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan" in syms and "__ubsan" in syms
    env = dict(os.environ, LD_PRELOAD=asan, BSA_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    root = os.path.dirname(HERE)
    # the child really loads the instrumented build
    probe = subprocess.run([sys.executable, "-c",
                            "import oracle; oracle.load(); "
                            "print(open('/proc/self/maps').read())"],
                           env=env, cwd=root, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert lib in probe.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       env=env, cwd=root, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout

    # negative control: a copy of oracle.c with a planted heap over-read in
    # oracle_num_blocks must make the same run fail under the sanitizer
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    head = "int32_t oracle_num_blocks(int32_t n, int32_t m) {"
    assert head in src
    planted = head + " { int* p = (int*)malloc(4 * sizeof(int)); volatile int z = p[4]; (void)z; free(p); }"
    bad_c = tmp_path / "oracle.c"
    bad_c.write_text(src.replace(head, planted))
    shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "oracle.h"), tmp_path / "oracle.h")
    bad = str(tmp_path / "liboracle_bad.so")
    subprocess.run([gcc, *oracle._CFLAGS, "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-g", str(bad_c), "-o", bad, "-lm"], check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py"), "-k", "entry_counts"],
                       env=dict(env, BSA_ORACLE_LIB=bad), cwd=root, capture_output=True, text=True,
                       timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode != 0 and ("heap-buffer-overflow" in out or "runtime error:" in out), out[-2000:]
    assert "oracle.c:" in out  # the report points into the planted copy
