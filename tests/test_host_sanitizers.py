"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only;
no GPU code runs). The C ABI's host layer (api.cpp: recipe, shape, pointer,
alignment and workspace checks, the split plan, the tau choice) is built with
ASan and UBSan into lib/libbdfp4_san.so (build.build_sanitized, device code
as usual) and the host ABI tests run against it with the sanitizer runtime
preloaded; the oracle's C checker of the quotient correction runs under the
same sanitizers (gcc)."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))


def _sanitized_env(runtime: str) -> dict:
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def test_host_abi_under_asan_and_ubsan():
    from fp4_kv_cache_nvfp4_amd import build as B
    try:
        lib = B.build_sanitized(verbose=False)
        runtime = B.sanitizer_runtime()
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"no hipcc / clang sanitizer runtime here: {e}")
    code = ("import sys; sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r}); "
            "import fp4_kv_cache_nvfp4_amd as bd; bd.LIB_PATH = {lib!r}; import pytest; "
            "sys.exit(pytest.main([{t!r}, '-q', '-p', 'no:cacheprovider', '-m', 'not gpu']))"
            ).format(root=ROOT, tests=HERE, lib=lib, t=os.path.join(HERE, "test_abi_host.py"))
    r = subprocess.run([sys.executable, "-c", code], env=_sanitized_env(runtime), capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quotient_checker_under_asan_and_ubsan():
    src = os.path.join(HERE, "arith", "quotient_check.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "qc")
        subprocess.run(["gcc", "-O2", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-o", exe,
                        src, "-lm"], check=True)
        r = subprocess.run([exe, "-122", "0"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout and "runtime error:" not in r.stderr
