"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with host-side ASan/UBSan (device code unchanged) and
every C-ABI test of tests/test_abi.py -- argument validation, size limits,
workspace queries, the symbol table -- runs against it in a child process with
the ASan runtime preloaded; any sanitizer report aborts the child.  No GPU is
needed: every call there returns before its first HIP call, or at it.
"""

import os
import subprocess
import sys

import pytest

from softmax_learnable_sink_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {root!r})
from softmax_learnable_sink_amd import binding
binding.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(['-q', '-p', 'no:cacheprovider', {tests!r}])
print('loaded', binding.lib()._name)
sys.exit(rc)
"""


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("san") / "libattn_sink_san.so")
    return build.build_sanitized(out)


def test_library_is_instrumented(sanitized_lib):
    syms = subprocess.run(["nm", "-D", "--undefined-only", sanitized_lib], capture_output=True,
                          text=True).stdout
    assert "__asan_report" in syms, "host code not built with AddressSanitizer"
    assert "__ubsan_handle" in syms, "host code not built with UndefinedBehaviorSanitizer"


def test_abi_checks_under_asan_and_ubsan(sanitized_lib):
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=ROOT, lib=sanitized_lib,
                        tests=os.path.join(ROOT, "tests", "test_abi.py"))
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         cwd=ROOT, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert f"loaded {sanitized_lib}" in out
