"""The library's host runtime on the CPU (no GPU): api.hip built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer against a fake HIP runtime
whose kernel launchers check every launch's read and write extents (from the
kernels' indexing) and the invariants the kernels rely on
(tests/hostsim/fake_hip.cpp).  The scenarios replay the call sequences of the
benchmark workloads at their real Dory-2B sizes (the batched workload's
64 x 8192-token set-up included), the dispatch edges of every entry point on
the tiny, pages and Dory-2B geometries, and the latch of failed calls
(kv_cache.rs `append`: a failed transition is terminal until the sequence is
cleared) with launch failures injected by the library's own test hook and by
the fake runtime."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, os.path.join(ROOT, "tests", "hostsim"))


@pytest.fixture(scope="module")
def hostsim():
    import build as hs_build
    return hs_build.build()


def _run(exe, name, timeout=300):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe, name], capture_output=True, text=True, timeout=timeout, env=env)
    return r.returncode, r.stdout + r.stderr


def test_checker_reports_planted_out_of_bounds_launches(hostsim):
    rc, out = _run(hostsim, "selftest")
    assert rc == 0, out
    assert "as planted" in out


@pytest.mark.parametrize("name", ["latch", "noalloc", "kvtap", "tiny", "tiny_q8", "pages", "shapes2b", "shapes2b_q8", "decode2b",
                                  "gate2b", "prefill2b", "q8_2b"])
def test_host_runtime_scenario(hostsim, name):
    rc, out = _run(hostsim, name)
    assert rc == 0, out
    assert "violations 0, failed expectations 0" in out, out


@pytest.mark.slow
def test_batched_workload_setup_and_steps(hostsim):
    """The batched benchmark's call sequence: 64 sequences prefilled to 8192 in
    512-row calls, then 132 batched steps with loop counts in 1..16 (about
    250k launches, every extent checked)."""
    rc, out = _run(hostsim, "batch2b", timeout=600)
    assert rc == 0, out
    assert "violations 0, failed expectations 0" in out, out
