"""Host checks of the persistent forward driver's work plan.

The plan (csrc/persist_plan.h: per-XCD queues, the ticket-to-item mapping,
the dependency targets of the waits) is compiled with g++ into a simulation
(tests/persist_sim.cpp) in which threads play the workgroups; it checks that
every gate/up and down item runs exactly once, that no wait can deadlock under
random interleavings, that the waits enforce the ring's slot reuse rule and
that the queues are balanced. Cited: [MoK clip] Key points bullets 3-5 and
How-to item 3 (minibatches through a reused ring of slots, completion
signalled through device counters).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("persist") / "persist_sim")
    subprocess.run([cxx, "-O2", "-std=c++17", "-pthread", "-Wall", "-Wextra", "-Werror", "-o", exe,
                    os.path.join(HERE, "persist_sim.cpp")], check=True)
    return exe


def test_plan_runs_every_item_once_without_deadlock(sim):
    out = subprocess.run([sim, "400"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok 405"
