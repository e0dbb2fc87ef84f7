"""The C ABI's host-side checks under AddressSanitizer and UndefinedBehaviorSanitizer.

A second build of the library compiles its host code with ASan and UBSan (the
device code as usual) into a temporary directory; the host-only ABI tests then
run against it in a child process that preloads the sanitizer runtime.  Any
invalid host access or undefined behaviour in argument checking, workspace
sizing or status reporting aborts the child.  No GPU is touched."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    from sparse_long_context_relu_amd.build import build
    runtime = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtime:
        pytest.skip("the clang ASan runtime is not installed")
    lib = build(out_path=str(tmp_path / "libdsa_san.so"), build_dir=str(tmp_path / "obj"), sanitize_host=True, jobs=8)
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in undefined and "__ubsan_handle" in undefined, "host code not instrumented"
    env = dict(os.environ, DSA_LIBRARY_PATH=lib, LD_PRELOAD=runtime[-1],
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_abi.py"), "-q", "-p",
                        "no:cacheprovider", "-k", "validation or workspace or status or noalloc or exports"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-4000:] + "\n" + r.stderr[-4000:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    passed = [l for l in r.stdout.splitlines() if " passed" in l]
    assert passed and int(passed[-1].split()[0]) >= 10, tail
