"""The megakernel's task protocol (event counters, task numbering, static per-XCD claim lists,
dynamic ticket queue, rest state) restated in tests/protocol_sim.cpp and run by host threads
under random interleavings: every task exactly once, no deadlock, every read ordered after
its write (also under ThreadSanitizer), and a dropped notification ending the forward through
the watchdog.  Builds with a planted mistake show that the checks catch it."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "protocol_sim.cpp")
pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _build(tmp_path, name, flags):
    exe = str(tmp_path / name)
    b = subprocess.run(["g++", "-std=c++17", "-Wall", "-pthread", *flags, SRC, "-o", exe], capture_output=True,
                       text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    return exe


def _run(exe, *args, timeout=300):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    return subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout, env=env)


def test_protocol_random_interleavings(tmp_path):
    exe = _build(tmp_path, "protocol_sim", ["-O2"])
    for seed in (1, 2, 3):
        r = _run(exe, seed, 5)
        assert r.returncode == 0, r.stdout[-4000:]
        assert " 0 failures" in r.stdout


def test_protocol_under_thread_sanitizer(tmp_path):
    exe = _build(tmp_path, "protocol_sim_tsan", ["-O1", "-g", "-fsanitize=thread"])
    r = _run(exe, 7, 1)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and " 0 failures" in r.stdout, r.stdout[-4000:]


def test_checks_catch_a_planted_double_notify(tmp_path):
    exe = _build(tmp_path, "protocol_sim_plant2", ["-O2", "-DPLANT=2"])
    r = _run(exe, 1, 1, 200)
    assert r.returncode != 0 and "FAIL" in r.stdout


def test_thread_sanitizer_catches_a_planted_missing_wait(tmp_path):
    exe = _build(tmp_path, "protocol_sim_plant1", ["-O1", "-g", "-fsanitize=thread", "-DPLANT=1"])
    r = _run(exe, 1, 1, 200)
    assert "ThreadSanitizer: data race" in r.stderr
