"""Every global-memory access of every kernel launch and copy stays inside the
buffer it addresses: the library's real host pipeline (hcattn.cpp) linked
against a fake HIP runtime that replays each kernel's index arithmetic on the
host (tests/native/extent_check.cpp), built with the address and
undefined-behaviour sanitizers, over ~1400 shapes around tile, workgroup and
trunk edges with exactly sized user tensors and workspace regions.  A planted
copy of the dK/dV kernel's K/V row loads without their clamp to the last key
must be reported, as must its runs of unchecked full-tile Q / dO loads
replayed without their limit at a head's last full tile, and the forward's
K / V ring schedule with one V slot too few, and HIP
failures injected into copies and kernel launches must come back as
ATTN_EHIP without breaking the next call."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "head_chunked_context_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def extent_exe(tmp_path_factory):
    if shutil.which("g++") is None or not os.path.isdir(ROCM_INC):
        pytest.skip("needs g++ and the HIP headers")
    exe = tmp_path_factory.mktemp("extent") / "extent_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", CSRC,
           os.path.join(HERE, "native", "extent_check.cpp"), os.path.join(CSRC, "hcattn.cpp"),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(exe)


def _run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe, *args], capture_output=True, text=True, env=env, timeout=600)


def test_every_kernel_access_stays_in_its_region(extent_exe):
    r = _run(extent_exe)
    print(r.stdout, r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "failures: 0" in r.stdout


def test_planted_over_read_is_reported(extent_exe):
    r = _run(extent_exe, "--plant-dkdv-overread")
    assert r.returncode == 1
    assert "dkdv V row" in r.stderr and "failures: 0" not in r.stdout


def test_planted_fast_run_past_the_last_full_tile_is_reported(extent_exe):
    # the dK/dV kernel's runs of unchecked full-tile loads, replayed without
    # their limit at a head's last full tile, must show up as partial-tile loads
    r = _run(extent_exe, "--plant-dkdv-fast-run")
    assert r.returncode == 1
    assert "dkdv fast run" in r.stderr and "failures: 0" not in r.stdout


def test_planted_four_slot_forward_v_ring_is_reported(extent_exe):
    # with the forward's deferred P V products, a V ring of four slots lets
    # a wave load a tile into a slot another wave still reads
    r = _run(extent_exe, "--plant-fwd-v-ring4")
    assert r.returncode == 1
    assert "fwd V ring" in r.stderr and "failures: 0" not in r.stdout


def test_injected_copy_and_launch_failures_surface_and_leave_no_state(extent_exe):
    # a trunk copy or kernel launch that fails makes the call return
    # ATTN_EHIP naming it, and the same call right after succeeds
    r = _run(extent_exe, "--inject")
    print(r.stdout, r.stderr[-2000:])
    assert r.returncode == 0, r.stderr[-2000:]
    assert "failures: 0" in r.stdout
