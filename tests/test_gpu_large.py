"""GPU parity at the full workload sizes, on entries the oracle can compute one
by one, plus properties that hold at any size.

* Workload 2 (S=32768, 32/8/128; head_chunk 4 and 32, the configuration the
  benchmark used to time) and a ragged S=16484 case whose head_chunk 4 and 1
  runs take the 256-row and the 128-row workgroup shapes of the forward and
  dQ kernels.
* Workloads 3, 4 and 5 (S=262144 / 524288 / 5242880): about 3.5 minutes of
  GPU and host time together, most of it the 5.24M-token run.

Checks: O, LSE and dQ on sampled query rows (each row's oracle costs O(S*D)
per head); dK and dV on the last keys (they need only the last rows' LSE and
Delta), and at workload 2 also on the first 16 keys and a 16-key block at
S/2 of one GQA group (keys that run the whole query loop of the dK/dV
kernel: their oracle needs every later row's LSE and Delta, ~20 s of host
time for the group's 4 heads); bitwise equality across head_chunk, trunked vs
untrunked, and the O(S*D) identities sum_j dK_j = 0 and
sum_j dV_j = sum_{h in group} sum_i dO_i.
"""
import numpy as np
import pytest
import torch

from head_chunked_context_amd import attn_bwd, attn_fwd
from head_chunked_context_amd.inputs import WORKLOADS, attention_inputs
from oracle import oracle as orc
from tests.gpu_util import TOL, TOL_LSE, gated_error, maxabs

pytestmark = pytest.mark.gpu
# full-size workload 3/4/5 runs: tens of seconds to a few minutes each
slow = pytest.mark.slow

DEV = "cuda"


def f64(t):
    return t.detach().to("cpu", torch.float32).double().numpy()


def sample_rows(S, T=None, n_random=6, seed=0):
    rows = {0, 1, 63, 64, 127, 128, S // 2, S - 2, S - 1}
    if T:
        for b in range(T, S, T):
            rows |= {b - 1, b}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, S, n_random))
    return np.array(sorted(r for r in rows if 0 <= r < S), dtype=np.int64)


def check_rows(d, o, lse, dq, rows, causal=True):
    """O, LSE, dQ of the sampled rows against the oracle (fp64)."""
    q_rows = d["q"][rows].cpu()
    do_rows = d["dout"][rows].cpu()
    k, v = d["k"].cpu(), d["v"].cpu()
    ro, rl = orc.attn_fwd_rows(q_rows, rows, k, v, causal)
    eo = gated_error(f64(o[rows]), ro)
    el = maxabs(f64(lse[:, rows]), rl)
    rdq, _ = orc.attn_dq_rows(q_rows, do_rows, rows, k, v, causal)
    edq = gated_error(f64(dq[rows]), rdq)
    print(f"  rows {len(rows)}: O {eo:.3e}  LSE {el:.3e}  dQ {edq:.3e}", flush=True)
    assert eo <= TOL and el <= TOL_LSE and edq <= TOL


def check_last_keys(d, dk, dv, n=16, causal=True):
    """dK, dV of the last n keys against the oracle (rows i >= S - n only)."""
    S = d["q"].shape[0]
    i0 = S - n
    cols = np.arange(i0, S)
    rdk, rdv = orc.attn_dkdv_cols(d["q"][i0:].cpu(), d["dout"][i0:].cpu(), i0, d["k"].cpu(),
                                  d["v"].cpu(), cols, causal)
    edk = gated_error(f64(dk[i0:]), rdk)
    edv = gated_error(f64(dv[i0:]), rdv)
    print(f"  last {n} keys: dK {edk:.3e}  dV {edv:.3e}", flush=True)
    assert edk <= TOL and edv <= TOL


def check_group_keys(d, dk, dv, kv, cols):
    """dK, dV of the keys `cols` of kv head `kv` against the oracle, from the
    query heads of that kv head's group only (the other heads do not touch
    them): rows i >= min(cols) of those heads."""
    S, Hq, D = d["q"].shape
    g = Hq // d["k"].shape[1]
    i0 = int(min(cols))
    hs = slice(kv * g, (kv + 1) * g)
    rdk, rdv = orc.attn_dkdv_cols(d["q"][i0:, hs].cpu(), d["dout"][i0:, hs].cpu(), i0,
                                  d["k"][:, kv:kv + 1].cpu(), d["v"][:, kv:kv + 1].cpu(),
                                  np.asarray(cols), True)
    edk = gated_error(f64(dk[cols, kv:kv + 1]), rdk)
    edv = gated_error(f64(dv[cols, kv:kv + 1]), rdv)
    print(f"  kv head {kv}, keys {cols[0]}..{cols[-1]} ({len(cols)}): dK {edk:.3e}  dV {edv:.3e}",
          flush=True)
    assert edk <= TOL and edv <= TOL


def check_sum_identities(d, dk, dv, g):
    """sum_j dK_j = 0 and sum_j dV_j = sum over the group's heads and rows of dO."""
    dkf = dk.to(DEV, torch.float64)
    dvf = dv.to(DEV, torch.float64)
    do = d["dout"].to(DEV, torch.float64)
    S, Hkv, D = dkf.shape
    for kv in range(Hkv):
        sk = dkf[:, kv].sum(0)
        l1 = dkf[:, kv].abs().sum(0)
        assert float((sk.abs() / l1).max()) <= 1e-3, "sum_j dK_j is not ~0"
        want = do[:, kv * g:(kv + 1) * g].sum((0, 1))
        sv = dvf[:, kv].sum(0)
        l1v = dvf[:, kv].abs().sum(0)
        assert float(((sv - want).abs() / l1v).max()) <= 1e-3, "sum_j dV_j != sum dO"


def run(d, hc, trunk=0, kv_host=False):
    k, v = d["k"], d["v"]
    if kv_host:
        k, v = d["k_host"], d["v_host"]
    o, lse = attn_fwd(d["q"], k, v, head_chunk=hc, kv_trunk=trunk)
    torch.cuda.synchronize()
    print("  forward done", flush=True)
    dq, dk, dv = attn_bwd(d["q"], k, v, o, d["dout"], lse, head_chunk=hc, kv_trunk=trunk)
    torch.cuda.synchronize()
    print("  backward done", flush=True)
    return o, lse, dq, dk, dv


@pytest.mark.timeout(600)
def test_workload2_full_size_head_chunks_and_samples():
    w = WORKLOADS[2]
    d = attention_inputs(w.S, w.Hq, w.Hkv, w.D, w.wid, device=DEV)
    print(f"workload 2 S={w.S} hc=4", flush=True)
    a = run(d, 4)
    print("workload 2 hc=32", flush=True)
    b = run(d, 32)
    for x, y, n in zip(a, b, ("o", "lse", "dq", "dk", "dv")):
        assert torch.equal(x, y), f"{n} differs between head_chunk 4 and 32"
    o, lse, dq, dk, dv = a
    check_rows(d, o, lse, dq, sample_rows(w.S))
    check_last_keys(d, dk, dv, n=32)
    # keys that run the dK/dV kernel's whole query loop (512 64-row steps for
    # key 0, 256 for the block at S/2), in the last GQA group
    kv = w.Hkv - 1
    check_group_keys(d, dk, dv, kv, np.arange(w.S // 2, w.S // 2 + 16))
    check_group_keys(d, dk, dv, kv, np.arange(0, 16))
    check_sum_identities(d, dk, dv, w.Hq // w.Hkv)


@pytest.mark.parametrize("D", [128, 64])
def test_wide_and_narrow_workgroups_give_the_same_bits(D):
    # head_chunk 4 launches 65 x 4 = 260 forward / dQ workgroups of 256 rows
    # (8 waves, deep K/V ring); head_chunk 1 launches fewer than 256 and takes
    # the 128-row shape: every row must come out bit for bit the same
    S, Hq, Hkv = 16484, 4, 1
    d = attention_inputs(S, Hq, Hkv, D, 7, device=DEV)
    print(f"wide/narrow S={S} D={D} hc=4", flush=True)
    a = run(d, 4)
    print(f"wide/narrow S={S} D={D} hc=1", flush=True)
    b = run(d, 1)
    for x, y, n in zip(a, b, ("o", "lse", "dq", "dk", "dv")):
        assert torch.equal(x, y), f"{n} differs between the wide and narrow launches"
    o, lse, dq, dk, dv = a
    check_rows(d, o, lse, dq, sample_rows(S, n_random=4))
    check_last_keys(d, dk, dv, n=16)


@pytest.mark.parametrize("D", [128, 64])
def test_die_aware_dkdv_order_gives_the_same_bits(D):
    # dK/dV launches whose head count is not a multiple of 4 take runs of 32
    # work items per die in a snake order over windows of 256 workgroups;
    # S = 66000 has 516 key tiles of 128, so head_chunk 1 (516 workgroups: two
    # full windows and a partial one) and 2 (1032) take that order while 4
    # keeps the plain one: every result must come out bit for bit the same
    S, Hq, Hkv = 66000, 4, 1
    d = attention_inputs(S, Hq, Hkv, D, 9, device=DEV)
    outs = []
    for hc in (4, 2, 1):
        print(f"die-aware order S={S} D={D} hc={hc}", flush=True)
        outs.append(run(d, hc))
    for b in outs[1:]:
        for x, y, n in zip(outs[0], b, ("o", "lse", "dq", "dk", "dv")):
            assert torch.equal(x, y), f"{n} differs between the plain and die-aware orders"
    o, lse, dq, dk, dv = outs[0]
    check_rows(d, o, lse, dq, sample_rows(S, n_random=4))
    check_last_keys(d, dk, dv, n=16)
    check_sum_identities(d, dk, dv, Hq // Hkv)


@slow
@pytest.mark.timeout(600)
def test_workload3_head_chunk_sweep_bitwise_and_samples():
    w = WORKLOADS[3]
    d = attention_inputs(w.S, w.Hq, w.Hkv, w.D, w.wid, device=DEV)
    ref = None
    for hc in (4, 1, 2, 8, 32):
        print(f"workload 3 S={w.S} hc={hc}", flush=True)
        out = run(d, hc)
        if ref is None:
            ref = out
        else:
            for x, y, n in zip(ref, out, ("o", "lse", "dq", "dk", "dv")):
                assert torch.equal(x, y), f"{n} differs between head_chunk 4 and {hc}"
            del out
    o, lse, dq, dk, dv = ref
    check_rows(d, o, lse, dq, sample_rows(w.S, n_random=4))
    check_last_keys(d, dk, dv, n=8)
    check_sum_identities(d, dk, dv, w.Hq // w.Hkv)


@slow
def test_workload3_q_zero_closed_form():
    w = WORKLOADS[3]
    d = attention_inputs(w.S, 2, 1, w.D, w.wid, device=DEV, with_dout=False)
    d["q"].zero_()
    o, lse = attn_fwd(d["q"], d["k"], d["v"], head_chunk=1)
    torch.cuda.synchronize()
    i = torch.arange(w.S, device=DEV, dtype=torch.float64)
    assert float((lse.double() - torch.log1p(i)).abs().max()) <= TOL_LSE
    prefix = torch.cumsum(d["v"][:, 0].double(), 0) / (i + 1)[:, None]
    err = (o.double() - prefix[:, None, :]).abs().max()
    assert float(err) <= TOL


@slow
@pytest.mark.timeout(600)
def test_workload4_pinned_host_trunks():
    w = WORKLOADS[4]
    d = attention_inputs(w.S, w.Hq, w.Hkv, w.D, w.wid, device=DEV)
    d["k_host"] = d["k"].cpu().pin_memory()
    d["v_host"] = d["v"].cpu().pin_memory()
    hc, T = w.head_chunks[0], w.kv_trunk
    print(f"workload 4 S={w.S} hc={hc} T={T} K/V in pinned host memory", flush=True)
    ot, lt, dqt, dkt, dvt = run(d, hc, trunk=T, kv_host=True)
    check_rows(d, ot, lt, dqt, sample_rows(w.S, T=T, n_random=2))
    check_last_keys(d, dkt.to(DEV), dvt.to(DEV), n=8)
    check_sum_identities(d, dkt, dvt, w.Hq // w.Hkv)
    # the untrunked forward and backward give the same bits
    print("workload 4 untrunked", flush=True)
    o, lse = attn_fwd(d["q"], d["k"], d["v"], head_chunk=hc)
    assert torch.equal(o, ot) and torch.equal(lse, lt)
    del o, lse
    g = attn_bwd(d["q"], d["k"], d["v"], ot, d["dout"], lt, head_chunk=hc)
    torch.cuda.synchronize()
    assert torch.equal(g[0], dqt)
    assert torch.equal(g[1].cpu(), dkt) and torch.equal(g[2].cpu(), dvt)


@slow
@pytest.mark.timeout(900)
def test_workload5_five_million_tokens_completes_and_matches_samples():
    w = WORKLOADS[5]
    d = attention_inputs(w.S, w.Hq, w.Hkv, w.D, w.wid, device=DEV)
    hc, T = w.head_chunks[0], w.kv_trunk
    print(f"workload 5 S={w.S} hc={hc} T={T}", flush=True)
    o, lse, dq, dk, dv = run(d, hc, trunk=T)
    assert torch.isfinite(lse).all()
    check_rows(d, o, lse, dq, sample_rows(w.S, T=T, n_random=2))
    check_last_keys(d, dk, dv, n=4)
    check_sum_identities(d, dk, dv, w.Hq // w.Hkv)
