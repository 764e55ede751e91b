"""The C ABI's host code (argument checks, workspace sizing, error paths) under
AddressSanitizer and UndefinedBehaviorSanitizer.

Runs the CPU ABI tests (tests/test_abi_cpu.py) in a child process against
libsad_hostsan.so, the library with sanitized host code
(`python -m sparse_attention_decode_build_amd.build --host-sanitize`), with the clang
ASan runtime preloaded.  Skipped when that library has not been built (it is not part of
the default build)."""

import os
import subprocess
import sys

import pytest

from sparse_attention_decode_build_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    clang = os.path.join(os.path.dirname(os.path.realpath(B._hipcc())), "..", "lib", "llvm", "bin", "clang")
    for exe in (clang, "/opt/rocm/lib/llvm/bin/clang"):
        if os.path.exists(exe):
            d = subprocess.run([exe, "--print-runtime-dir"], capture_output=True, text=True).stdout.strip()
            for cand in (os.path.join(d, "libclang_rt.asan.so"),
                         os.path.join(os.path.dirname(d), "linux", "libclang_rt.asan-x86_64.so")):
                if os.path.exists(cand):
                    return cand
    return None


@pytest.mark.skipif(not os.path.exists(B.HOST_SANITIZED_LIB), reason="libsad_hostsan.so not built")
def test_abi_host_code_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    code = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "from sparse_attention_decode_build_amd import _lib as L\n"
        "L.load(%r)\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), B.HOST_SANITIZED_LIB, os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    # the ASan runtime goes first; anything already preloaded stays after it
    pre = ":".join(x for x in (rt, os.environ.get("LD_PRELOAD", "")) if x)
    env = dict(os.environ, LD_PRELOAD=pre, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr
