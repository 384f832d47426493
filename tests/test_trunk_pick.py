"""Trunk-length selection (attn_pick_kv_trunk): host arithmetic only, no GPU.

The rule (FPDT summary, "Technical Deep Dive" and the trunk-size Q&A): the
copy of the next trunk should take about as long as computing on the current
one, and a longer trunk only costs memory.  Checked here: every pick fits the
budget and is accepted by the workspace planners; it is minimal (half of it
misses a criterion); slower links give longer trunks; device-resident K/V that
fit untrunked stay untrunked; and the picks for the two long workloads land in
the best band the trunk-size sweep measured on one MI355X (T >= 64K for
S = 524288, 40/8 heads, head_chunk 5 with K/V in pinned host memory).
"""
import ctypes

import pytest

import head_chunked_context_amd as hc
from head_chunked_context_amd.hcattn import HcAttnError, lib

GiB = 1 << 30


def need(S, Hq, Hkv, D, hc_, T, with_bwd=True):
    n = hc.fwd_workspace_bytes(S, Hq, Hkv, D, True, hc_, T)
    if with_bwd:
        n = max(n, hc.bwd_workspace_bytes(S, Hq, Hkv, D, True, hc_, T))
    return n


def kv_heads_in_widest_chunk(Hq, Hkv, hc_):
    g = Hq // Hkv
    return max((min(h0 + hc_, Hq) - 1) // g - h0 // g + 1 for h0 in range(0, Hq, hc_))


def test_long_workloads_pick_the_measured_balance():
    # measured sweep at S = 524288: T >= 64K within 0.3% of the best, 32K
    # loses 3% (2.5 rounds of forward workgroups), 16K 15%
    T4 = hc.pick_kv_trunk(524288, 40, 8, 128, True, 5, kv_on_host=True,
                          link_bytes_per_s=57e9, flops_per_s=1e15, num_cus=256)
    assert T4 == 65536
    T5 = hc.pick_kv_trunk(5242880, 4, 1, 128, True, 1, kv_on_host=True)
    assert T5 >= 262144 and T5 % 256 == 0 and T5 < 5242880


def test_device_resident_fitting_untrunked_stays_untrunked():
    assert hc.pick_kv_trunk(32768, 32, 8, 128, True, 4) == 0
    assert hc.pick_kv_trunk(262144, 32, 8, 128, True, 4,
                            budget_bytes=need(262144, 32, 8, 128, 4, 0)) == 0


@pytest.mark.parametrize("shape", [(262144, 32, 8, 128, 4), (524288, 40, 8, 128, 5),
                                   (100000, 8, 2, 64, 3), (5242880, 4, 1, 128, 1)])
@pytest.mark.parametrize("host", [False, True])
@pytest.mark.parametrize("with_bwd", [False, True])
def test_pick_fits_budget_and_is_minimal(shape, host, with_bwd):
    S, Hq, Hkv, D, hc_ = shape
    link, flops, cus = 20e9, 1e15, 256
    kvc = kv_heads_in_widest_chunk(Hq, Hkv, hc_)
    floor = need(S, Hq, Hkv, D, hc_, 256, with_bwd)
    for budget in (floor, int(floor * 1.3), floor * 2, floor * 5, floor * 40, 0):
        try:
            T = hc.pick_kv_trunk(S, Hq, Hkv, D, True, hc_, kv_on_host=host,
                                 with_backward=with_bwd, budget_bytes=budget,
                                 link_bytes_per_s=link, flops_per_s=flops, num_cus=cus)
        except HcAttnError as e:
            pytest.fail(f"budget {budget}: {e}")
        if T == 0:
            assert not host
            assert budget == 0 or need(S, Hq, Hkv, D, hc_, 0, with_bwd) <= budget
            continue
        assert T % 256 == 0 and 256 <= T < S and (T // 256) & (T // 256 - 1) == 0
        assert budget == 0 or need(S, Hq, Hkv, D, hc_, T, with_bwd) <= budget

        def ok(t):
            balanced = (not host) or t >= kvc * flops / (hc_ * link)
            fills = -(-t // 128) * hc_ >= 8 * cus
            return balanced and fills

        if ok(T):
            # smallest qualifying: half of it misses a criterion
            assert T == 256 or not ok(T // 2)
        else:
            # nothing qualified within the budget: the longest fitting trunk
            assert 2 * T >= S or (budget and need(S, Hq, Hkv, D, hc_, 2 * T, with_bwd) > budget)


def test_slower_link_never_shortens_the_trunk():
    prev = 0
    for link in (200e9, 57e9, 16e9, 4e9, 1e9, 0.25e9):
        T = hc.pick_kv_trunk(524288, 40, 8, 128, True, 5, kv_on_host=True,
                             link_bytes_per_s=link, flops_per_s=1e15, num_cus=256)
        assert T >= prev
        prev = T
    assert prev >= 131072


def test_budget_too_small_and_bad_arguments():
    S, Hq, Hkv, D, hc_ = 262144, 32, 8, 128, 4
    # the smallest workspace any choice needs: the shortest trunk, or no trunk
    # (the untrunked backward of a long sequence keeps no per-head partials and
    # needs less than a trunked one, which carries dQ in fp32)
    floor = min(need(S, Hq, Hkv, D, hc_, 256), need(S, Hq, Hkv, D, hc_, 0))
    with pytest.raises(HcAttnError, match="ATTN_EWORKSPACE"):
        hc.pick_kv_trunk(S, Hq, Hkv, D, True, hc_, budget_bytes=floor - 1)
    with pytest.raises(HcAttnError, match="ATTN_EINVAL"):
        hc.pick_kv_trunk(256, 4, 2, 128, True, 2, kv_on_host=True)  # too short to trunk
    with pytest.raises(HcAttnError, match="ATTN_EINVAL"):
        hc.pick_kv_trunk(S, 30, 8, 128, True, 4)  # Hq % Hkv != 0
    with pytest.raises(HcAttnError, match="ATTN_EUNSUPPORTED"):
        hc.pick_kv_trunk(S, Hq, Hkv, 96, True, 4)
    rc = lib().attn_pick_kv_trunk(S, Hq, Hkv, D, 1, hc_, 0, 1, 0, 0.0, 0.0, 0,
                                  ctypes.cast(None, ctypes.POINTER(ctypes.c_int64)))
    assert rc == -4
