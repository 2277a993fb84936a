"""Host logic without a GPU: the workspace layout (moe_groupgemm_amd/csrc/mk_common.h) is
compiled with g++ into tests/host_layout_check.cpp, which checks that the layout grows with
the capacity and that a workspace sized for cap tokens holds every array, task index, queue
slot and trace record of every batch B <= cap under adversarial routing histograms.  The
host checks and the CPU oracle are also built with AddressSanitizer and
UndefinedBehaviorSanitizer (and the threaded capacity check with ThreadSanitizer), so an
out-of-bounds access, a leak, undefined arithmetic or a data race fails the run."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "moe_groupgemm_amd", "csrc")


ASAN_UBSAN = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
TSAN = ["-g", "-fsanitize=thread"]
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")


def _build_and_run(compiler, std, src, exe, flags, extra=()):
    b = subprocess.run([compiler, std, "-O1", "-Wall", *flags, "-I", CSRC, src, *extra, "-o", exe],
                       capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=SAN_ENV)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert re.search(r"(^|\s)0 failures", r.stdout), r.stdout[-3000:]
    assert "runtime error" not in r.stderr, r.stderr[-3000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("san", [[], ASAN_UBSAN], ids=["plain", "asan_ubsan"])
def test_workspace_layout_holds_every_batch(tmp_path, san):
    _build_and_run("g++", "-std=c++17", os.path.join(HERE, "host_layout_check.cpp"),
                   str(tmp_path / "host_layout_check"), san)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
@pytest.mark.parametrize("san", [[], ASAN_UBSAN, TSAN], ids=["plain", "asan_ubsan", "tsan"])
def test_capacity_lookups_from_two_threads_on_one_plan(tmp_path, san):
    _build_and_run("g++", "-std=c++17", os.path.join(HERE, "host_capacity_check.cpp"),
                   str(tmp_path / "host_capacity_check"), san, ["-pthread"])


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    # every oracle entry point on small shapes (empty batch, k = E, ragged blocks, k = 1),
    # the routing invariants and the documented error returns, serial build (no OpenMP)
    _build_and_run("gcc", "-std=c11", os.path.join(HERE, "oracle_sanitize_check.c"),
                   str(tmp_path / "oracle_sanitize_check"), ASAN_UBSAN + ["-ffp-contract=off"], ["-lm"])
