"""The C-ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The library is rebuilt with sanitized host code (the gfx950 code as usual)
and the C-ABI tests (argument validation before any HIP call, status and
error strings, workspace sizes, the allocation-free entry point's limits)
run against it in a child process with the ASan runtime preloaded; any
sanitizer report fails the run (UBSan does not recover).  The two binding
tests that build torch tensors are left out: torch is not instrumented and
its import under a preloaded ASan runtime only adds noise."""

import os
import subprocess
import sys

import pytest

from video_diffusion_transformer_vdit_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _toolchain():
    try:
        build._hipcc()
        return build.asan_runtime()
    except RuntimeError:
        return None


@pytest.mark.skipif(_toolchain() is None, reason="hipcc or its ASan runtime is missing")
def test_capi_checks_clean_under_asan_and_ubsan():
    lib = build.build_sanitized(os.path.join(ROOT, "_build", "sanitize"))
    env = dict(os.environ)
    env.update({
        "VDIT_ATTN_LIB": lib,
        "LD_PRELOAD": build.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           "tests/test_capi_cpu.py", "tests/test_zz_no_alloc.py::test_noalloc_scratch_size_and_limit",
           "-k", "not binding_rejects and not reject_block_v_means"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, out[-2000:]
