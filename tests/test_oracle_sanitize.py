"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
oracle/sanitize_main.c calls every entry point on small seeded inputs and
their edge cases (ragged sequences, T = 0, rows with no ready entry, -1
padding, latent outputs, no sink); any out-of-bounds access, use after free,
leak, signed overflow or misaligned access ends the run with a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "oracle", "sanitize_main.c"), os.path.join(ROOT, "oracle", "csa_oracle.c")]
FLAGS = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build(tmp_path, extra=()):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "orc_san")
    r = subprocess.run(["gcc", *FLAGS, *extra, *SRC, "-lm", "-o", exe], capture_output=True,
                       text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower():
        pytest.skip("the sanitizer runtime is not installed")
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)


def test_oracle_is_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    r = _run(_build(tmp_path))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all cases clean" in r.stdout


def test_sanitizer_harness_reports_a_planted_overflow(tmp_path):
    # the same driver with one deliberate read past an allocation
    r = _run(_build(tmp_path, ["-DORC_SANITIZE_SELFTEST"]))
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr
