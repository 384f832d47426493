"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: max-abs 2e-2 for O, dQ, dK, dV and 1e-3 for LSE, on the same
seeded bf16 inputs (the oracle widens them exactly).  Results must also be
bitwise identical across head_chunk values and run to run.
"""
import math

import numpy as np
import pytest
import torch

from tests.gpu_util import (DEV, TOL, TOL_LSE, check_bwd, check_fwd, f64, gpu_bwd, gpu_fwd,
                            inputs_cpu, maxabs, to_dev)

pytestmark = pytest.mark.gpu


def _run_case(S, Hq, Hkv, D, hcs, seed, causal=True, q_scale=1.0, rel=False):
    inp = inputs_cpu(S, Hq, Hkv, D, seed, q_scale)
    d = to_dev(inp)
    outs = {}
    for hc in hcs:
        print(f"case S={S} Hq={Hq} Hkv={Hkv} D={D} hc={hc} causal={causal}", flush=True)
        o, lse = gpu_fwd(d, hc, causal=causal)
        g = gpu_bwd(d, o, lse, hc, causal=causal)
        outs[hc] = (o, lse) + tuple(g)
    ref = outs[hcs[0]]
    for hc in hcs[1:]:
        for a, b, n in zip(ref, outs[hc], ("o", "lse", "dq", "dk", "dv")):
            assert torch.equal(a, b), f"{n} differs bitwise between hc={hcs[0]} and hc={hc}"
    check_fwd(inp, ref[0], ref[1], causal)
    check_bwd(inp, ref[2:], causal, rel=rel)


def test_tiny_exactness_case_all_head_chunks():
    # S=256, Hq=4, Hkv=2, D=64, head_chunk in {1, 2, 4}
    _run_case(256, 4, 2, 64, [4, 1, 2], seed=1)


def test_tiny_case_fp32_variant_reports_input_rounding():
    # the tiny case's fp32 variant: the oracle on the fp32 draws themselves
    # against the GPU on their bf16 rounding.  The difference is the effect
    # of rounding the inputs to bf16 (the GPU path takes bf16 only); it is
    # reported, and only held to a loose bound that catches gross errors.
    from head_chunked_context_amd.inputs import attention_inputs
    from oracle import oracle as orc
    x32 = attention_inputs(256, 4, 2, 64, 1, device="cpu", dtype=torch.float32)
    d = {n: t.to(torch.bfloat16).to(DEV) for n, t in x32.items()}
    o, lse = gpu_fwd(d, 2)
    dq, dk, dv = gpu_bwd(d, o, lse, 2)
    ro, rl = orc.attn_fwd(x32["q"], x32["k"], x32["v"], True)
    rg = orc.attn_bwd(x32["q"], x32["k"], x32["v"], x32["dout"], True)
    errs = {"o": maxabs(f64(o), ro), "lse": maxabs(f64(lse), rl), "dq": maxabs(f64(dq), rg["dq"]),
            "dk": maxabs(f64(dk), rg["dk"]), "dv": maxabs(f64(dv), rg["dv"])}
    print("fp32 variant, GPU(bf16(x)) vs oracle(x):",
          "  ".join(f"{n} {e:.3e}" for n, e in errs.items()), flush=True)
    assert all(np.isfinite(e) and e < 0.25 for e in errs.values()), errs


def test_ragged_tail_d128():
    _run_case(1000, 4, 2, 128, [4, 1, 2], seed=11)


def test_gqa_chunks_not_aligned_with_groups():
    # g = 4; hc = 3 makes groups span chunks (two fp32 carry slots), hc = 1 nests
    _run_case(700, 8, 2, 128, [8, 3, 1, 2], seed=12)


def test_wide_group_chunks_of_odd_size():
    # g = 8 (one kv head): hc = 3 and 5 leave ragged chunks whose group spans
    # two or three chunks, D = 64, ragged sequence end
    _run_case(601, 8, 1, 64, [8, 3, 5], seed=17)


def test_non_causal():
    _run_case(300, 4, 1, 128, [4, 1], seed=13, causal=False)


def test_non_causal_d64_ragged():
    _run_case(333, 2, 2, 64, [2, 1], seed=14, causal=False)


def test_peaked_softmax():
    # Q scaled by 8 (scores ~N(0, 64)): a stress case outside the N(0,1) workloads,
    # where |dK| reaches ~30; gradients are held to 2e-2 relative to their peak
    _run_case(512, 2, 1, 128, [2, 1], seed=15, q_scale=8.0, rel=True)


@pytest.mark.parametrize("S,D", [(319, 128), (320, 128), (321, 64), (384, 64)])
def test_tile_load_boundaries(S, D):
    # the last 64-row tile of keys (forward, dQ) and of queries (dK/dV) is
    # short by one row, exactly full, or holds a single row: full tiles take
    # the scalar-base loads, short ones the clamping path
    _run_case(S, 4, 2, D, [4, 1], seed=40 + S)


def test_single_token_and_tiny():
    for S in (1, 2, 33):
        _run_case(S, 2, 1, 128, [2, 1], seed=16 + S)


def _random_cases(n, seed):
    # seeded shapes: S across tile and workgroup boundaries, GQA ratios 1-8,
    # chunks that split groups, D 64/128, causal or not, key/value trunks
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * g
        S = int(rng.integers(1, 1600))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.75)
        hcs = sorted({Hq, int(rng.integers(1, Hq + 1))}, reverse=True)
        T = int(rng.choice([0, 0, 256, 512])) if S > 256 else 0
        cases.append((S, Hq, Hkv, D, causal, hcs, T))
    return cases


@pytest.mark.parametrize("case", _random_cases(10, 2024))
def test_random_shapes_match_oracle(case):
    S, Hq, Hkv, D, causal, hcs, T = case
    inp = inputs_cpu(S, Hq, Hkv, D, 50 + S % 97)
    d = to_dev(inp)
    outs = []
    for hc in hcs:
        print(f"random case S={S} Hq={Hq} Hkv={Hkv} D={D} causal={causal} hc={hc} T={T}",
              flush=True)
        o, lse = gpu_fwd(d, hc, trunk=T, causal=causal)
        outs.append((o, lse) + tuple(gpu_bwd(d, o, lse, hc, trunk=T, causal=causal)))
    for x, y in zip(outs[0], outs[-1]):
        assert torch.equal(x, y), "results differ bitwise across head_chunk"
    check_fwd(inp, outs[0][0], outs[0][1], causal)
    check_bwd(inp, outs[0][2:], causal)


def test_run_to_run_deterministic():
    inp = inputs_cpu(777, 4, 2, 128, 21)
    d = to_dev(inp)
    a = gpu_fwd(d, 2)
    b = gpu_fwd(d, 2)
    ga = gpu_bwd(d, a[0], a[1], 2)
    gb = gpu_bwd(d, b[0], b[1], 2)
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


@pytest.mark.parametrize("D", [128, 64])
def test_wide_launch_run_to_run_deterministic(D):
    # 64 row tiles x 16 heads = 1024 forward / dQ workgroups: the 8-wave shape,
    # whose waves 4-7 run a phase behind waves 0-3 through a 5-slot V ring
    # (a slot reloaded while another wave still reads it shows up as bits
    # that change from run to run)
    from head_chunked_context_amd.inputs import attention_inputs
    S, Hq, Hkv = 16384, 16, 4
    d = attention_inputs(S, Hq, Hkv, D, 31, device=DEV)
    runs = []
    for r in range(3):
        print(f"wide run-to-run S={S} Hq={Hq} D={D} run {r}", flush=True)
        o, lse = gpu_fwd(d, Hq)
        runs.append((o, lse) + tuple(gpu_bwd(d, o, lse, Hq)))
    for b in runs[1:]:
        for x, y, n in zip(runs[0], b, ("o", "lse", "dq", "dk", "dv")):
            assert torch.equal(x, y), f"{n} changes from run to run"


@pytest.mark.parametrize("D", [128, 64])
def test_wide_and_narrow_launches_agree_non_causal(D):
    # non-causal: every wave walks every tile, so the 8-wave shape's deferred
    # P V products run on every pair.  head_chunk 16 launches 64 x 16 = 1024
    # forward / dQ workgroups (8 waves), head_chunk 1 launches 64 (4 waves,
    # checked against the oracle at small sizes in test_non_causal*): the two
    # must give the same bits
    from head_chunked_context_amd.inputs import attention_inputs
    S, Hq, Hkv = 16384, 16, 4
    d = attention_inputs(S, Hq, Hkv, D, 37, device=DEV)
    out = {}
    for hc in (Hq, 1):
        print(f"non-causal wide/narrow S={S} Hq={Hq} D={D} hc={hc}", flush=True)
        o, lse = gpu_fwd(d, hc, causal=False)
        out[hc] = (o, lse) + tuple(gpu_bwd(d, o, lse, hc, causal=False))
    for x, y, n in zip(out[Hq], out[1], ("o", "lse", "dq", "dk", "dv")):
        assert torch.equal(x, y), f"{n} differs between the wide and narrow launches"


def test_q_zero_closed_form():
    # q = 0: P is uniform over the visible keys, LSE_i = ln(i+1), O_i = mean(v_0..v_i)
    S, Hq, Hkv, D = 4096, 2, 1, 128
    inp = inputs_cpu(S, Hq, Hkv, D, 22)
    inp["q"].zero_()
    d = to_dev(inp)
    o, lse = gpu_fwd(d, 1)
    i = np.arange(S)
    v = f64(inp["v"])[:, 0, :]
    prefix = np.cumsum(v, 0) / (i + 1.0)[:, None]
    for h in range(Hq):
        assert maxabs(f64(lse)[h], np.log(i + 1.0)) <= 1e-5
        assert maxabs(f64(o)[:, h, :], prefix) <= 1e-2
    # O_0 = v_0 exactly (one visible key, p = 1)
    assert torch.equal(o[0, 0].cpu(), inp["v"][0, 0])


@pytest.mark.parametrize("kv_host", [False, True])
def test_kv_trunks_match_oracle_and_untrunked_backward(kv_host):
    S, Hq, Hkv, D, hc, T = 1100, 4, 2, 128, 2, 256  # 5 trunks, ragged last one
    inp = inputs_cpu(S, Hq, Hkv, D, 31)
    d = to_dev(inp)
    dt = to_dev(inp, kv_host=kv_host)
    print(f"trunked S={S} T={T} kv_host={kv_host}", flush=True)
    ot, lt = gpu_fwd(dt, hc, trunk=T)
    check_fwd(inp, ot, lt)
    o, lse = gpu_fwd(d, hc)
    # the softmax state is carried from trunk to trunk exactly
    assert torch.equal(ot, o), "trunked forward O differs bitwise from untrunked"
    assert torch.equal(lt, lse), "trunked forward LSE differs bitwise from untrunked"
    g = gpu_bwd(d, o, lse, hc)
    gt = gpu_bwd(dt, o, lse, hc, trunk=T)
    for a, b, n in zip(g, gt, ("dq", "dk", "dv")):
        assert torch.equal(a.cpu(), b.cpu()), f"trunked {n} differs bitwise from untrunked"
    check_bwd(inp, g)


@pytest.mark.parametrize("causal,D", [(False, 128), (True, 64)])
def test_trunks_non_causal_and_d64(causal, D):
    # non-causal: every query trunk attends all key trunks; D = 64 tiles
    S, Hq, Hkv, hc, T = 900, 4, 1, 2, 256
    inp = inputs_cpu(S, Hq, Hkv, D, 37)
    d = to_dev(inp)
    dt = to_dev(inp, kv_host=True)
    print(f"trunked S={S} D={D} causal={causal} T={T}", flush=True)
    ot, lt = gpu_fwd(dt, hc, trunk=T, causal=causal)
    check_fwd(inp, ot, lt, causal)
    o, lse = gpu_fwd(d, hc, causal=causal)
    assert torch.equal(ot, o) and torch.equal(lt, lse)
    g = gpu_bwd(d, o, lse, hc, causal=causal)
    gt = gpu_bwd(dt, o, lse, hc, trunk=T, causal=causal)
    for a, b, n in zip(g, gt, ("dq", "dk", "dv")):
        assert torch.equal(a.cpu(), b.cpu()), f"trunked {n} differs bitwise from untrunked"
    check_bwd(inp, g, causal)


def test_picked_trunk_runs_bitwise_equal_to_untrunked():
    # the trunk chosen for a workspace budget that the untrunked run exceeds
    from head_chunked_context_amd import fwd_workspace_bytes, pick_kv_trunk
    S, Hq, Hkv, D, hc = 3000, 4, 2, 128, 2
    budget = fwd_workspace_bytes(S, Hq, Hkv, D, True, hc, 0) // 2
    T = pick_kv_trunk(S, Hq, Hkv, D, True, hc, kv_on_host=True, with_backward=False,
                      budget_bytes=budget)
    assert 0 < T < S and fwd_workspace_bytes(S, Hq, Hkv, D, True, hc, T) <= budget
    inp = inputs_cpu(S, Hq, Hkv, D, 38)
    d = to_dev(inp)
    dt = to_dev(inp, kv_host=True)
    print(f"picked trunk S={S} T={T}", flush=True)
    ot, lt = gpu_fwd(dt, hc, trunk=T)
    o, lse = gpu_fwd(d, hc)
    assert torch.equal(ot, o) and torch.equal(lt, lse)
    check_fwd(inp, ot, lt)


@pytest.mark.parametrize("kv_host", [False, True])
def test_trunk_merge_schedule_matches_oracle(kv_host):
    # per-trunk partial outputs merged by log-sum-exp: equal to rounding
    from head_chunked_context_amd import set_trunk_merge
    S, Hq, Hkv, D, hc, T = 1100, 4, 2, 128, 2, 256
    inp = inputs_cpu(S, Hq, Hkv, D, 35)
    d = to_dev(inp)
    dt = to_dev(inp, kv_host=kv_host)
    prev = set_trunk_merge(True)
    try:
        print(f"trunk merge S={S} T={T} kv_host={kv_host}", flush=True)
        ot, lt = gpu_fwd(dt, hc, trunk=T)
    finally:
        set_trunk_merge(prev)
    check_fwd(inp, ot, lt)
    o, lse = gpu_fwd(d, hc)
    assert maxabs(f64(ot), f64(o)) <= TOL
    assert maxabs(f64(lt), f64(lse)) <= TOL_LSE


@pytest.mark.parametrize("trunk,kv_host", [(0, False), (256, False), (256, True)])
def test_forward_without_lse(trunk, kv_host):
    # forward-only (prefill) use: no LSE is kept; O must match the oracle and
    # the output of the call that keeps the LSE, bit for bit
    from head_chunked_context_amd import attn_fwd
    S, Hq, Hkv, D = 777, 4, 2, 128
    inp = inputs_cpu(S, Hq, Hkv, D, 36)
    d = to_dev(inp, kv_host=kv_host)
    print(f"forward without LSE S={S} T={trunk} kv_host={kv_host}", flush=True)
    o2, none = attn_fwd(d["q"], d["k"], d["v"], head_chunk=2, kv_trunk=trunk, with_lse=False)
    torch.cuda.synchronize()
    assert none is None
    check_fwd(inp, o2, None)
    o, lse = attn_fwd(d["q"], d["k"], d["v"], head_chunk=2, kv_trunk=trunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def test_trunked_groups_spanning_chunks_on_host():
    # hc = 1 < g = 2: dK/dV carried in fp32 across chunks while K/V stream from host
    S, Hq, Hkv, D, T = 768, 4, 2, 128, 256
    inp = inputs_cpu(S, Hq, Hkv, D, 32)
    d = to_dev(inp)
    dt = to_dev(inp, kv_host=True)
    o, lse = gpu_fwd(d, 1)
    g = gpu_bwd(d, o, lse, 4)
    gt = gpu_bwd(dt, o, lse, 1, trunk=T)
    for a, b in zip(g, gt):
        assert torch.equal(a.cpu(), b.cpu())


def test_single_stream_equals_overlapped():
    from head_chunked_context_amd import set_single_stream
    S, Hq, Hkv, D, T = 1024, 2, 1, 128, 256
    inp = inputs_cpu(S, Hq, Hkv, D, 33)
    dt = to_dev(inp, kv_host=True)
    o1, l1 = gpu_fwd(dt, 1, trunk=T)
    g1 = gpu_bwd(dt, o1, l1, 1, trunk=T)
    prev = set_single_stream(True)
    try:
        o2, l2 = gpu_fwd(dt, 1, trunk=T)
        g2 = gpu_bwd(dt, o2, l2, 1, trunk=T)
    finally:
        set_single_stream(prev)
    for a, b in zip((o1, l1) + tuple(g1), (o2, l2) + tuple(g2)):
        assert torch.equal(a.cpu(), b.cpu())


def test_errors_are_reported_without_work():
    from head_chunked_context_amd import HcAttnError, attn_fwd
    from head_chunked_context_amd.hcattn import lib
    inp = inputs_cpu(64, 2, 1, 128, 34)
    d = to_dev(inp)
    ws = torch.empty(1 << 24, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        attn_fwd(inp["q"], d["k"], d["v"], workspace=ws)  # q in host memory: the binding refuses
    # the library's own pointer check, called through the C ABI directly: q in
    # pageable host memory is refused before any work
    o = torch.empty_like(d["q"])
    rc = lib().attn_fwd(inp["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), o.data_ptr(),
                        None, 64, 2, 1, 128, 1, 0, 0, ws.data_ptr(), ws.numel(),
                        torch.cuda.current_stream().cuda_stream)
    assert rc == -4
    with pytest.raises((HcAttnError, ValueError)):
        attn_fwd(d["q"], d["k"], d["v"], workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    with pytest.raises(HcAttnError) as e:
        attn_fwd(d["q"], d["k"], d["v"], head_chunk=5)  # more than Hq
    assert e.value.code == -1


@pytest.mark.parametrize("trunk,kv_host", [(0, False), (256, True)])
def test_hip_graph_capture_replays_bitwise(trunk, kv_host):
    # attn_fwd + attn_bwd captured into one graph (the library's copy stream
    # forks from and joins the captured stream); every replay, with eager work
    # in between, gives the eager result bit for bit
    from head_chunked_context_amd import (attn_bwd, attn_fwd, bwd_workspace_bytes,
                                          fwd_workspace_bytes)
    S, Hq, Hkv, D, hc = 640, 4, 2, 128, 2
    inp = inputs_cpu(S, Hq, Hkv, D, 38)
    d = to_dev(inp, kv_host=kv_host)
    q, k, v, do = d["q"], d["k"], d["v"], d["dout"]
    o_e, l_e = attn_fwd(q, k, v, head_chunk=hc, kv_trunk=trunk)
    g_e = attn_bwd(q, k, v, o_e, do, l_e, head_chunk=hc, kv_trunk=trunk)
    torch.cuda.synchronize()
    o, lse = torch.empty_like(o_e), torch.empty_like(l_e)
    dq = torch.empty_like(g_e[0])
    dk = torch.empty(k.shape, dtype=k.dtype, device=k.device, pin_memory=kv_host)
    dv = torch.empty(v.shape, dtype=v.dtype, device=v.device, pin_memory=kv_host)
    fws = torch.empty(fwd_workspace_bytes(S, Hq, Hkv, D, True, hc, trunk), dtype=torch.uint8,
                      device=DEV)
    bws = torch.empty(bwd_workspace_bytes(S, Hq, Hkv, D, True, hc, trunk), dtype=torch.uint8,
                      device=DEV)

    def step():
        attn_fwd(q, k, v, head_chunk=hc, kv_trunk=trunk, out=o, lse=lse, workspace=fws)
        attn_bwd(q, k, v, o, do, lse, head_chunk=hc, kv_trunk=trunk, dq=dq, dk=dk, dv=dv,
                 workspace=bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="thread_local"):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y, n in zip((o, lse, dq, dk, dv), (o_e, l_e) + tuple(g_e), ("o", "lse", "dq", "dk", "dv")):
            assert torch.equal(x.cpu(), y.cpu()), f"replay {rep}: {n} differs from the eager result"


def _guarded(n, dtype, device, fill, guard_bytes=4096, pin=False):
    """n elements inside a buffer whose every byte (and guard_bytes more on
    each side) starts as `fill`; returns (buffer, view of the n elements)."""
    el = torch.empty((), dtype=dtype).element_size()
    g = guard_bytes // el
    buf = torch.empty(n + 2 * g, dtype=dtype, device=device, pin_memory=pin)
    buf.view(torch.uint8).fill_(fill)
    return buf, buf[g:g + n]


def _guards_intact(buf, view, fill):
    b = buf.view(torch.uint8)
    lo = view.data_ptr() - buf.data_ptr()
    hi = lo + view.numel() * view.element_size()
    return bool((b[:lo] == fill).all()) and bool((b[hi:] == fill).all())


@pytest.mark.parametrize("trunk,kv_host,hc", [(0, False, 4), (0, False, 1), (256, False, 3),
                                              (256, True, 1)])
def test_poisoned_workspace_and_guard_bytes(trunk, kv_host, hc):
    # every workspace byte starts as 0xFF (NaN in bf16 and fp32): results must
    # equal those of a zeroed workspace bit for bit, so no kernel reads
    # workspace it has not written; the outputs and the workspace sit between
    # guard bytes that must come back untouched
    from head_chunked_context_amd import attn_bwd, attn_fwd
    from head_chunked_context_amd import hcattn as H
    S, Hq, Hkv, D = 900, 8, 2, 128  # g = 4: hc = 1 and 3 carry dK/dV across chunks
    inp = inputs_cpu(S, Hq, Hkv, D, 61)
    d = to_dev(inp, kv_host=kv_host)
    print(f"poison S={S} hc={hc} T={trunk} kv_host={kv_host}", flush=True)
    nf = H.fwd_workspace_bytes(S, Hq, Hkv, D, True, hc, trunk)
    nb = H.bwd_workspace_bytes(S, Hq, Hkv, D, True, hc, trunk)
    zf = torch.zeros(nf, dtype=torch.uint8, device=DEV)
    zb = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    o_ref, l_ref = attn_fwd(d["q"], d["k"], d["v"], head_chunk=hc, kv_trunk=trunk, workspace=zf)
    g_ref = attn_bwd(d["q"], d["k"], d["v"], o_ref, d["dout"], l_ref, head_chunk=hc,
                     kv_trunk=trunk, workspace=zb)
    torch.cuda.synchronize()

    C = 0x5A
    wfb, wf = _guarded(nf, torch.uint8, DEV, 0xFF)
    wbb, wb = _guarded(nb, torch.uint8, DEV, 0xFF)
    ob, o = _guarded(S * Hq * D, torch.bfloat16, DEV, C)
    lb, lse = _guarded(Hq * S, torch.float32, DEV, C)
    dqb, dq = _guarded(S * Hq * D, torch.bfloat16, DEV, C)
    kdev = "cpu" if kv_host else DEV
    dkb, dk = _guarded(S * Hkv * D, torch.bfloat16, kdev, C, pin=kv_host)
    dvb, dv = _guarded(S * Hkv * D, torch.bfloat16, kdev, C, pin=kv_host)
    o, lse = o.view(S, Hq, D), lse.view(Hq, S)
    dq, dk, dv = dq.view(S, Hq, D), dk.view(S, Hkv, D), dv.view(S, Hkv, D)
    attn_fwd(d["q"], d["k"], d["v"], head_chunk=hc, kv_trunk=trunk, out=o, lse=lse, workspace=wf)
    attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, head_chunk=hc, kv_trunk=trunk,
             dq=dq, dk=dk, dv=dv, workspace=wb)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "forward depends on workspace contents"
    for a, b, n in zip((dq, dk, dv), g_ref, ("dq", "dk", "dv")):
        assert torch.equal(a, b), f"{n} depends on workspace contents"
    for buf, view, fill, n in ((ob, o, C, "o"), (lb, lse, C, "lse"), (dqb, dq, C, "dq"),
                               (dkb, dk, C, "dk"), (dvb, dv, C, "dv"),
                               (wfb, wf, 0xFF, "forward workspace"),
                               (wbb, wb, 0xFF, "backward workspace")):
        assert _guards_intact(buf, view, fill), f"bytes next to {n} were written"
