"""Memory-safety, undefined-behaviour and data-race checks of the CPU code the
tests rely on: the oracle (oracle/oracle.c) and the seeded input generator
(synth/synth.c), linked into tests/sanitize_driver.c, which calls every
function they export over small, ragged and degenerate shapes.

Two builds with gcc: AddressSanitizer + UndefinedBehaviorSanitizer (with the
float-to-integer and float-divide checks that -fsanitize=undefined leaves
out), and ThreadSanitizer for the threaded splits.  Any sanitizer report, or
a non-zero exit, fails the test.  Built and run on the CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "tests", "sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(ROOT, "synth", "synth.c")]
BASE = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off"]

BUILDS = {
    "asan_ubsan": ["-fsanitize=address,undefined,float-cast-overflow,float-divide-by-zero",
                   "-fno-sanitize-recover=all"],
    "tsan": ["-fsanitize=thread"],
}
ENV = {
    "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=86",
    "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=87",
    "TSAN_OPTIONS": "halt_on_error=1:exitcode=88",
}
REPORT_MARKS = ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer",
                "ERROR: LeakSanitizer")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
@pytest.mark.parametrize("build", sorted(BUILDS))
def test_oracle_and_generator_under_sanitizers(build, tmp_path):
    exe = str(tmp_path / f"sanitize_{build}")
    cmd = ["gcc", *BASE, *BUILDS[build], "-o", exe, *SOURCES, "-lm", "-lpthread"]
    cp = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if cp.returncode != 0 and "cannot find" in cp.stderr and "san" in cp.stderr:
        pytest.skip(f"the {build} runtime is not installed: {cp.stderr.strip()[:200]}")
    assert cp.returncode == 0, cp.stderr
    env = dict(os.environ, **ENV)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    reports = [m for m in REPORT_MARKS if m in run.stderr]
    assert run.returncode == 0 and not reports, (
        f"{build}: exit {run.returncode}, reports {reports}\n{run.stderr[-4000:]}")
    assert "sanitize_driver: done" in run.stdout
