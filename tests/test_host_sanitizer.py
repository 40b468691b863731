"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

libgt_attn_san.so is the same library with its host code instrumented (argument
checks, workspace sizing, the breadth-first distance-code builder, launch set-up;
`python -m graph_transformer_attention_amd.build --sanitize`). The host tests run
against it in a child interpreter that preloads the sanitizer runtime; any report
aborts the child. A canary library with one planted heap overflow and one planted
oversized shift, loaded the same way, must be caught, so that a clean run means
something.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from graph_transformer_attention_amd import build as B  # noqa: E402

pytestmark = pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                                reason="a preload is already set; the sanitizer runtime is not stacked on it")


def _env():
    env = dict(os.environ)
    env.update(LD_PRELOAD=B.sanitizer_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", GT_ATTN_LIBRARY=B.SAN_LIB)
    return env


def test_host_tests_pass_under_sanitizers():
    assert os.path.exists(B.SAN_LIB), f"{B.SAN_LIB} is missing: python -m graph_transformer_attention_amd.build --sanitize"
    assert os.path.exists(B.sanitizer_runtime())
    # the full-size certificate at N = 32768 is left to the plain run (a minute under ASan)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py"), "-k", "not ba32768"],
                       cwd=ROOT, env=_env(), capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def test_canary_errors_are_caught(tmp_path):
    src = tmp_path / "canary.cpp"
    src.write_text(textwrap.dedent("""\
        #include <vector>
        extern "C" int heap_read(int i) { std::vector<int> v(8, 1); return v.data()[i]; }
        extern "C" int shift(int s) { return 1 << s; }
        """))
    so = tmp_path / "libcanary.so"
    subprocess.run([B.HIPCC, "-x", "c++", "-O1", "-fPIC", "-shared", "-shared-libasan", *B.SAN_FLAGS, str(src),
                    "-o", str(so)], check=True, capture_output=True)
    for call, report in (("heap_read(3); L.heap_read(9)", "heap-buffer-overflow"),
                         ("shift(3); L.shift(40)", "shift exponent 40")):
        code = f"import ctypes; L = ctypes.CDLL({str(so)!r}); L.{call}"
        r = subprocess.run([sys.executable, "-c", code], env=_env(), capture_output=True, text=True, timeout=120)
        assert r.returncode != 0 and report in r.stderr, r.stderr[-2000:]
