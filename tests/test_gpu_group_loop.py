"""The group-loop dK/dV schedule (one workgroup per key tile and kv head walks
the chunk's heads of the group; an fp32 carry of its sums when a group spans
chunks; bf16 dK/dV written without partials or a reduce pass).  Long
sequences (S >= 65536) take it by default and are checked at full size in
test_gpu_large.py; here it is forced at small S (attn_set_group_loop_min_s)
so that every element can be compared with the oracle."""
import pytest
import torch

from head_chunked_context_amd import attn_bwd, attn_fwd, set_group_loop_min_s
from tests.gpu_util import DEV, check_bwd, check_fwd, gpu_bwd, gpu_fwd, inputs_cpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture
def group_loop():
    prev = set_group_loop_min_s(1)
    yield
    set_group_loop_min_s(prev)


@pytest.mark.parametrize("S,Hq,Hkv,D,hcs,causal", [
    (700, 8, 2, 128, [8, 3, 1, 2], True),   # g = 4: one and two carry slots
    (601, 8, 1, 64, [8, 3, 5], True),       # g = 8, ragged chunks, D = 64
    (333, 4, 1, 128, [4, 1], False),        # non-causal
    (1000, 4, 4, 128, [4, 1], True),        # g = 1: one head per kv head
    (2, 2, 1, 128, [2, 1], True),
])
def test_group_loop_matches_oracle_bitwise_across_head_chunk(group_loop, S, Hq, Hkv, D, hcs,
                                                              causal):
    inp = inputs_cpu(S, Hq, Hkv, D, 90 + S % 31)
    d = to_dev(inp)
    outs = []
    for hc in hcs:
        print(f"group loop S={S} Hq={Hq} Hkv={Hkv} D={D} hc={hc} causal={causal}", flush=True)
        o, lse = gpu_fwd(d, hc, causal=causal)
        outs.append((o, lse) + tuple(gpu_bwd(d, o, lse, hc, causal=causal)))
    for x in outs[1:]:
        for a, b, n in zip(outs[0], x, ("o", "lse", "dq", "dk", "dv")):
            assert torch.equal(a, b), f"{n} differs bitwise across head_chunk"
    check_fwd(inp, outs[0][0], outs[0][1], causal)
    check_bwd(inp, outs[0][2:], causal)


@pytest.mark.parametrize("kv_host,hc", [(False, 2), (True, 1), (True, 3)])
def test_group_loop_trunked_equals_untrunked(group_loop, kv_host, hc):
    S, Hq, Hkv, D, T = 1100, 6, 2, 128, 256  # g = 3: hc 1 and 2 split groups
    inp = inputs_cpu(S, Hq, Hkv, D, 97)
    d = to_dev(inp)
    dt = to_dev(inp, kv_host=kv_host)
    print(f"group loop trunked S={S} hc={hc} T={T} kv_host={kv_host}", flush=True)
    o, lse = gpu_fwd(d, hc)
    g = gpu_bwd(d, o, lse, hc)
    gt = gpu_bwd(dt, o, lse, hc, trunk=T)
    for a, b, n in zip(g, gt, ("dq", "dk", "dv")):
        assert torch.equal(a.cpu(), b.cpu()), f"trunked {n} differs bitwise from untrunked"
    check_bwd(inp, g)


def test_group_loop_and_per_head_schedules_agree_to_rounding():
    S, Hq, Hkv, D = 900, 8, 2, 128
    inp = inputs_cpu(S, Hq, Hkv, D, 98)
    d = to_dev(inp)
    o, lse = gpu_fwd(d, 2)
    per_head = gpu_bwd(d, o, lse, 2)
    prev = set_group_loop_min_s(1)
    try:
        looped = gpu_bwd(d, o, lse, 2)
    finally:
        set_group_loop_min_s(prev)
    # dQ does not depend on the dK/dV schedule; dK/dV differ only by the
    # order of fp32 additions over the group's heads
    assert torch.equal(per_head[0], looped[0])
    for a, b in zip(per_head[1:], looped[1:]):
        assert float((a.float() - b.float()).abs().max()) <= 2e-2
    check_bwd(inp, looped)


@pytest.mark.parametrize("trunk,kv_host,hc", [(0, False, 4), (0, False, 1), (256, True, 3)])
def test_group_loop_poisoned_workspace_and_guard_bytes(group_loop, trunk, kv_host, hc):
    # every workspace byte starts as 0xFF (NaN): the results equal those of a
    # zeroed workspace bit for bit, and the bytes around every output and the
    # workspace come back untouched
    from head_chunked_context_amd import hcattn as H
    from tests.test_gpu_parity import _guarded, _guards_intact
    S, Hq, Hkv, D = 900, 8, 2, 128
    inp = inputs_cpu(S, Hq, Hkv, D, 99)
    d = to_dev(inp, kv_host=kv_host)
    print(f"group loop poison S={S} hc={hc} T={trunk} kv_host={kv_host}", flush=True)
    o, lse = attn_fwd(d["q"], d["k"], d["v"], head_chunk=hc, kv_trunk=trunk)
    nb = H.bwd_workspace_bytes(S, Hq, Hkv, D, True, hc, trunk)
    zb = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    g_ref = attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, head_chunk=hc, kv_trunk=trunk,
                     workspace=zb)
    torch.cuda.synchronize()
    C = 0x5A
    wbb, wb = _guarded(nb, torch.uint8, DEV, 0xFF)
    dqb, dq = _guarded(S * Hq * D, torch.bfloat16, DEV, C)
    kdev = "cpu" if kv_host else DEV
    dkb, dk = _guarded(S * Hkv * D, torch.bfloat16, kdev, C, pin=kv_host)
    dvb, dv = _guarded(S * Hkv * D, torch.bfloat16, kdev, C, pin=kv_host)
    dq, dk, dv = dq.view(S, Hq, D), dk.view(S, Hkv, D), dv.view(S, Hkv, D)
    attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, head_chunk=hc, kv_trunk=trunk, dq=dq,
             dk=dk, dv=dv, workspace=wb)
    torch.cuda.synchronize()
    for a, b, n in zip((dq, dk, dv), g_ref, ("dq", "dk", "dv")):
        assert torch.equal(a, b), f"{n} depends on workspace contents"
    for buf, view, fill, n in ((dqb, dq, C, "dq"), (dkb, dk, C, "dk"), (dvb, dv, C, "dv"),
                               (wbb, wb, 0xFF, "backward workspace")):
        assert _guards_intact(buf, view, fill), f"bytes next to {n} were written"
