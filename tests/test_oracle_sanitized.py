"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_main.c calls every oracle entry point (prefill with taps, a
chained prefill, a failing over-capacity prefill, passes with every tap and
with injected routing, re-noise, the masked update, Philox and the format
conversions) for fp32, bf16, fp8 and MXFP4 expert weights on one and two
threads.  Any sanitizer report aborts the run.
"""
import os
import subprocess

from oracle.build import build_sanitized


def _run(path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    return subprocess.run([path], capture_output=True, text=True, env=env, timeout=300)


def test_oracle_is_clean_under_asan_and_ubsan():
    r = _run(build_sanitized())
    assert r.returncode == 0, r.stderr[-4000:]
    assert "ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_the_sanitized_build_is_instrumented():
    # a planted heap read past the end of an allocation must be caught
    r = _run(build_sanitized(selfcheck=True))
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
