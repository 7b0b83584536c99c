"""Host model of the completion protocol under ThreadSanitizer
(tests/cpu_model/election.cpp): the acquire-release election, the per-expert
release/acquire form, and the tile level (several workgroups per expert, each
handing its waves' rows to one counting thread through a fenced barrier, then
a per-expert tile counter) run clean and deliver every value; each negative
control, which drops one of those orderings (a relaxed election, a relaxed
tile counter, a barrier without workgroup fences), must draw a data-race
report (a missing happens-before edge that hardware runs cannot be relied on
to show)."""
import shutil
import subprocess
from pathlib import Path

import pytest

SRC = Path(__file__).parent / "cpu_model" / "election.cpp"


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path_factory.mktemp("model") / "election_tsan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", str(SRC), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        pytest.skip(f"ThreadSanitizer build unavailable: {r.stderr[-300:]}")
    return exe


def _run(exe, mode, rounds=200):
    return subprocess.run([str(exe), mode, str(rounds)], capture_output=True, text=True,
                          timeout=120)


@pytest.mark.parametrize("mode", ["acq_rel", "per_expert", "tiles"])
def test_release_acquire_forms_are_race_free(model, mode):
    r = _run(model, mode)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-2000:]
    assert r.returncode == 0 and "0 wrong values" in r.stdout, r.stdout + r.stderr[-500:]


@pytest.mark.parametrize("mode", ["relaxed", "tiles_relaxed_counter", "tiles_no_wg_fence"])
def test_dropped_ordering_is_reported_as_a_race(model, mode):
    r = _run(model, mode)
    assert "WARNING: ThreadSanitizer: data race" in r.stderr, r.stderr[-2000:]
