"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, plans workspaces by the stated formula, and rejects bad arguments
before any GPU work (no compute call needs a GPU here)."""
import ctypes
import os
import re

import pytest

import head_chunked_context_amd as hc
from head_chunked_context_amd.hcattn import LIB_PATH, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hcattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    names = declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_fwd_workspace_bytes", "attn_bwd_workspace_bytes",
            "attn_last_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in hcattn.h but not exported"


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in (("ATTN_OK", 0), ("ATTN_EINVAL", -1), ("ATTN_EUNSUPPORTED", -2),
                      ("ATTN_EWORKSPACE", -3), ("ATTN_EPOINTER", -4), ("ATTN_EHIP", -5)):
        assert re.search(rf"{name}\s*=\s*{val}\b", text)


E = lambda S, D: S * D * 2  # one bf16 head slice
A = lambda x: (x + 255) // 256 * 256


@pytest.mark.parametrize("hc_", [1, 2, 4, 8, 32])
def test_forward_workspace_formula(hc_):
    S, Hq, Hkv, D = 262144, 32, 8, 128
    g = Hq // Hkv
    kvc = max(1, -(-hc_ // g))
    assert hc.fwd_workspace_bytes(S, Hq, Hkv, D, True, hc_, 0) == \
        A(hc_ * E(S, D)) + 2 * A(kvc * E(S, D))


def test_workspace_shrinks_with_head_chunk_by_one_over_hkv():
    # one GQA group per chunk vs all heads at once: exactly 1/Hkv = 1/8
    for S in (32768, 262144):
        for fn in (hc.fwd_workspace_bytes, hc.bwd_workspace_bytes):
            small = fn(S, 32, 8, 128, True, 4, 0)
            full = fn(S, 32, 8, 128, True, 32, 0)
            assert small * 8 == full


def test_backward_workspace_formula_aligned_chunks():
    S, Hq, Hkv, D = 32768, 32, 8, 128
    for hc_ in (4, 8, 32):
        kvc = hc_ // 4
        # Q, dO (bf16), -Delta and -LSE*log2(e) (fp32 rows), per-head fp32 dK/dV
        # partials, K, V (bf16)
        want = 2 * A(hc_ * E(S, D)) + 2 * A(hc_ * S * 4) + 2 * A(2 * hc_ * E(S, D)) + \
            2 * A(kvc * E(S, D))
        assert hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, hc_, 0) == want


def test_backward_workspace_formula_group_loop():
    # S >= 65536: the group-loop dK/dV schedule keeps no per-head fp32
    # partials; a group spanning chunks carries its fp32 sums
    S, Hq, Hkv, D = 262144, 32, 8, 128
    for hc_ in (4, 8, 32):
        kvc = hc_ // 4
        want = 2 * A(hc_ * E(S, D)) + 2 * A(hc_ * S * 4) + 2 * A(kvc * E(S, D))
        assert hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, hc_, 0) == want
    # hc = 1 and 2 (g = 4): one carry slot of [S][D] fp32 for dK and for dV
    for hc_ in (1, 2):
        want = 2 * A(hc_ * E(S, D)) + 2 * A(hc_ * S * 4) + 2 * A(E(S, D)) + 2 * A(2 * E(S, D))
        assert hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, hc_, 0) == want


def test_group_loop_threshold_switch():
    L = lib()
    L.attn_set_group_loop_min_s.argtypes = [ctypes.c_int64]
    L.attn_set_group_loop_min_s.restype = ctypes.c_int64
    S, Hq, Hkv, D = 4096, 8, 2, 128
    per_head = hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, 4, 0)
    prev = L.attn_set_group_loop_min_s(1)
    try:
        assert prev == 65536
        looped = hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, 4, 0)
    finally:
        assert L.attn_set_group_loop_min_s(prev) == 1
    assert per_head - looped == 2 * A(4 * E(S, D) * 2)  # the per-head partials
    assert hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, 4, 0) == per_head


def test_trunked_workspace_scales_with_trunk_not_sequence():
    a = hc.fwd_workspace_bytes(524288, 40, 8, 128, True, 5, 65536)
    b = hc.fwd_workspace_bytes(1048576, 40, 8, 128, True, 5, 65536)
    assert a == b  # forward trunked workspace does not depend on S
    c = hc.fwd_workspace_bytes(524288, 40, 8, 128, True, 5, 131072)
    assert c > a


def test_head_chunk_zero_means_all_heads():
    assert hc.fwd_workspace_bytes(4096, 8, 2, 128, True, 0, 0) == \
        hc.fwd_workspace_bytes(4096, 8, 2, 128, True, 8, 0)
    # kv_trunk >= S selects the untrunked path
    assert hc.fwd_workspace_bytes(4096, 8, 2, 128, True, 2, 4096) == \
        hc.fwd_workspace_bytes(4096, 8, 2, 128, True, 2, 0)


@pytest.mark.parametrize("args,code", [
    ((0, 4, 2, 128, 1, 0, 0), -1),       # S = 0
    ((64, 3, 2, 128, 1, 0, 0), -1),      # Hq % Hkv
    ((64, 4, 2, 96, 1, 0, 0), -2),       # D unsupported
    ((64, 4, 2, 128, 2, 0, 0), -1),      # causal flag
    ((64, 4, 2, 128, 1, 5, 0), -1),      # head_chunk > Hq
    ((4096, 4, 2, 128, 1, 0, 100), -1),  # trunk not a multiple of 256
    ((64, 4, 2, 128, 1, -1, 0), -1),
    (((1 << 30) + 1, 4, 2, 128, 1, 0, 0), -2),  # beyond 2^30 tokens
    ((1 << 30, 1 << 30, 1, 128, 1, 0, 0), -2),  # workspace bytes would wrap 64 bits
])
def test_invalid_arguments_return_status_before_any_gpu_work(args, code):
    L = lib()
    assert L.attn_fwd_workspace_bytes(*args) == 0
    assert L.attn_bwd_workspace_bytes(*args) == 0
    # the compute entry points fail the same way, with null pointers, before HIP
    rc = L.attn_fwd(None, None, None, None, None, *args, None, 0, None)
    assert rc == code, hc.last_error()
    rc = L.attn_bwd(None, None, None, None, None, None, None, None, None, *args, None, 0, None)
    assert rc == code, hc.last_error()
    assert hc.last_error() != ""


def test_workspace_and_pointer_checks_precede_gpu_work():
    L = lib()
    args = (256, 4, 2, 64, 1, 0, 0)
    assert L.attn_fwd(None, None, None, None, None, *args, None, 1 << 30, None) == -3
    assert L.attn_fwd(None, None, None, None, None, *args, 8, 1 << 30, None) == -3  # misaligned
    assert L.attn_fwd(None, None, None, None, None, *args, 4096, 16, None) == -3    # too small
    assert L.attn_fwd(None, None, None, None, None, *args, 4096, 1 << 30, None) == -4  # NULL q
    assert "q is NULL" in hc.last_error()


def test_version():
    assert re.match(r"\d+\.\d+\.\d+", hc.version())
