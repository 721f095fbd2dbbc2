"""The host block manager under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

``csrc/block_manager.cpp`` indexes caller-supplied token arrays and block
tables through raw pointers.  Here the same source is built a second time with
g++ and ``-fsanitize=address,undefined`` (host code only; nothing of the GPU
path is involved) and every test of ``test_block_manager.py`` runs against
that build in a child process (``PA_BM_LIBRARY`` points the binding at it, the
sanitizer runtimes are preloaded).  Any invalid access or undefined operation
aborts the child with the sanitizer's report.  A second test plants an
out-of-bounds table write in a copy of the source and checks that the harness
reports it, so a silent sanitizer setup cannot pass.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "paged_kv_attention_27_amd", "csrc", "block_manager.cpp")
SANITIZERS = "address,undefined"


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _need_toolchain():
    if shutil.which("g++") is None or _runtime("libasan.so") is None or _runtime("libubsan.so") is None:
        pytest.skip("g++ with the AddressSanitizer / UBSan runtimes is not available")


def _build(src, out):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", f"-fsanitize={SANITIZERS}",
           "-fno-sanitize-recover=all", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def _run_tests(lib):
    env = dict(os.environ)
    env["PA_BM_LIBRARY"] = lib
    env["LD_PRELOAD"] = f"{_runtime('libasan.so')} {_runtime('libubsan.so')}"
    # the interpreter's own allocations are not instrumented, so leaks are not checked;
    # pytest runs with -s so that a report printed just before the child exits is kept
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_block_manager.py"),
                           "-q", "-x", "-s", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_block_manager_tests_clean_under_sanitizers(tmp_path):
    _need_toolchain()
    lib = _build(SRC, str(tmp_path / "libpa_bm_asan.so"))
    r = _run_tests(lib)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout


def test_sanitizer_harness_reports_a_planted_overflow(tmp_path):
    """Planted mistake (CPU only): pa_bm_allocate pads one entry past the table."""
    _need_toolchain()
    text = open(SRC).read()
    needle = "for (int32_t b = nb; b < max_blocks; ++b)"
    assert text.count(needle) == 1
    bad = tmp_path / "block_manager_overflow.cpp"
    bad.write_text(text.replace(needle, "for (int32_t b = nb; b <= max_blocks; ++b)"))
    lib = _build(str(bad), str(tmp_path / "libpa_bm_bad.so"))
    r = _run_tests(lib)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stdout + r.stderr
