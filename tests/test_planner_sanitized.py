"""The planner under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only, built with g++, no GPU): tests/fuzz/planner_fuzz.cpp plans
random layouts, replays every region on host buffers of exactly the size
each view needs, and checks that every destination element is written
exactly once with its own global index, and walks each copy launch's work
units as the kernels take them (thin sibling groups member-fastest) to check
that every unit of every region is taken exactly once; corrupted descriptors
must be rejected with a message.  Any sanitizer report fails the run.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rl_weight_refit_amd", "csrc")


def _build(tmp_path_factory, name, extra=()):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("fuzz") / name)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", *extra,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "fuzz", "planner_fuzz.cpp"), os.path.join(CSRC, "planner.cpp"),
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    return _build(tmp_path_factory, "planner_fuzz")


@pytest.fixture(scope="module")
def fuzz_exe_small_pool(tmp_path_factory):
    """The planner with a 40-entry pointer pool (the library's is 500), so
    that the fuzz's small layouts overflow it: their plans get the table form
    (one launch per kind, pointers from a device table), which the fuzz
    walks unit by unit and compares region by region with the pooled form."""
    return _build(tmp_path_factory, "planner_fuzz_pool40", ("-DRS_POOL=40",))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_planner_fuzz_sanitized(fuzz_exe, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_exe, "4000", str(seed)], capture_output=True, text=True, timeout=600,
                       env=env)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    assert "planned and replayed" in r.stdout
    groups = int(r.stdout.split("thin sibling groups")[1].split()[0].rstrip(";"))
    assert groups > 0, r.stdout
    whole = int(r.stdout.split("loaded whole")[1].split()[0].rstrip(");"))
    assert whole > 0, r.stdout
    two = int(r.stdout.split("two-piece MXFP8 regions")[1].split()[0].rstrip(";"))
    assert two > 0, r.stdout


def test_planner_fuzz_table_form(fuzz_exe_small_pool):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_exe_small_pool, "4000", "7"], capture_output=True, text=True, timeout=600,
                       env=env)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    tables = int(r.stdout.split("table forms")[1].split()[0])
    assert tables > 100, r.stdout
