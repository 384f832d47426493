"""GPU parity of the attention layer (attn_layer_fwd / attn_layer_bwd: the
chunk's Q/K/V projections recomputed per head chunk, attention, the chunk's
share of the output projection accumulated, and the gradients) against the
fp64 oracle on the same seeded bf16 inputs, and bitwise equality across
head_chunk.

Bar: the layer's intermediates (q, k, v, the attention output, dO, dQ, dK,
dV) are rounded to bf16 where the attention kernels take or give them, so
each result carries errors of order 2^-8 of its own scale (the weight
gradients sum S terms and grow like sqrt(S)).  The attention's 2e-2 max-abs
bar is applied relative to each output's peak magnitude when that exceeds 1:
max|gpu - oracle| <= 2e-2 * max(1, max|oracle|).
"""
import numpy as np
import pytest
import torch

from head_chunked_context_amd import attn_layer_bwd, attn_layer_fwd
from head_chunked_context_amd.inputs import layer_inputs
from oracle import oracle as orc

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def f64(t):
    return t.detach().float().cpu().double().numpy()


def check(name, gpu, ref):
    ref = np.asarray(ref)
    err = float(np.max(np.abs(f64(gpu) - ref)))
    scale = max(1.0, float(np.max(np.abs(ref))))
    print(f"  {name}: max-abs {err:.3e}, peak |ref| {np.max(np.abs(ref)):.3e}, "
          f"ratio {err / scale:.3e}", flush=True)
    assert err <= TOL * scale, (name, err, scale)


@pytest.mark.parametrize("S,dm,Hq,Hkv,D,causal,hcs", [
    (300, 128, 8, 2, 64, True, [8, 3, 1, 4]),     # groups split across chunks, ragged S
    (1000, 256, 4, 2, 128, True, [4, 2, 1]),
    (513, 192, 4, 1, 128, False, [4, 3]),         # non-causal, ragged chunk
    (4096, 1024, 8, 2, 128, True, [4, 8]),        # many 128 x 128 product tiles, 8 splits
])
@pytest.mark.timeout(600)
def test_layer_matches_oracle_and_is_bitwise_across_head_chunk(S, dm, Hq, Hkv, D, causal, hcs):
    inp = layer_inputs(S, dm, Hq, Hkv, D, 80 + S % 17)
    d = {n: t.to(DEV) for n, t in inp.items()}
    outs = []
    for hc in hcs:
        print(f"layer S={S} dm={dm} Hq={Hq} Hkv={Hkv} D={D} causal={causal} hc={hc}", flush=True)
        y, lse = attn_layer_fwd(d["x"], d["wq"], d["wk"], d["wv"], d["wo"], Hq=Hq, Hkv=Hkv, D=D,
                                head_chunk=hc, causal=causal, with_lse=True)
        g = attn_layer_bwd(d["x"], d["wq"], d["wk"], d["wv"], d["wo"], d["dy"], Hq=Hq, Hkv=Hkv,
                           D=D, head_chunk=hc, causal=causal)
        torch.cuda.synchronize()
        outs.append((y, lse) + tuple(g))
    names = ("y", "lse", "dx", "dwq", "dwk", "dwv", "dwo")
    for o in outs[1:]:
        for a, b, n in zip(outs[0], o, names):
            assert torch.equal(a, b), f"{n} differs bitwise across head_chunk"
    ry, rl = orc.layer_fwd(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], Hq, Hkv, D, causal)
    rg = orc.layer_bwd(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["dy"], Hq, Hkv, D,
                       causal)
    y, lse, dx, dwq, dwk, dwv, dwo = outs[0]
    check("y", y, ry)
    lerr = float(np.max(np.abs(f64(lse) - rl)))
    print(f"  lse: max-abs {lerr:.3e}", flush=True)
    assert lerr <= 1e-2  # scores from bf16-rounded projections
    for n, t in (("dx", dx), ("dwq", dwq), ("dwk", dwk), ("dwv", dwv), ("dwo", dwo)):
        check(n, t, rg[n])


def test_layer_projection_of_identity_weights_is_the_attention():
    # identity projections (d_model = Hq * D, Hq = Hkv): the layer is the
    # attention itself, so y must equal attn_fwd's output on x (bf16-exact
    # projections, the same flash kernel) up to the output projection's
    # bf16 -> fp32 identity product, i.e. exactly the bf16 output
    from head_chunked_context_amd import attn_fwd
    S, Hq, D = 640, 2, 128
    dm = Hq * D
    g = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn((S, dm), generator=g).to(torch.bfloat16).to(DEV)
    eye = torch.eye(dm, dtype=torch.bfloat16, device=DEV)
    y, lse = attn_layer_fwd(x, eye, eye, eye, eye, Hq=Hq, Hkv=Hq, D=D, head_chunk=1, with_lse=True)
    xs = x.view(S, Hq, D).contiguous()
    o, l = attn_fwd(xs, xs, xs, head_chunk=1)
    torch.cuda.synchronize()
    assert torch.equal(y, o.float().view(S, dm))
    assert torch.equal(lse, l)


@pytest.mark.timeout(900)
def test_llama3_8b_layer_full_size_sampled_rows_and_head_chunks():
    # the Llama3-8B attention layer at S = 32768 (d_model 4096, 32/8 heads,
    # D 128): head_chunk 4 (one GQA group) and 32 give the same bits for y and
    # every gradient; y and LSE on sampled rows against the oracle (its cost
    # is the key/value projections of the whole sequence, ~1e12 fp64 FLOP)
    S, Hq, Hkv, D = 32768, 32, 8, 128
    dm = Hq * D
    inp = layer_inputs(S, dm, Hq, Hkv, D, 2, device=DEV)
    outs = []
    for hc in (4, 32):
        print(f"layer S={S} dm={dm} hc={hc}", flush=True)
        y, lse = attn_layer_fwd(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], Hq=Hq,
                                Hkv=Hkv, D=D, head_chunk=hc, with_lse=True)
        g = attn_layer_bwd(inp["x"], inp["wq"], inp["wk"], inp["wv"], inp["wo"], inp["dy"], Hq=Hq,
                           Hkv=Hkv, D=D, head_chunk=hc)
        torch.cuda.synchronize()
        outs.append((y, lse) + tuple(g))
    for a, b, n in zip(outs[0], outs[1], ("y", "lse", "dx", "dwq", "dwk", "dwv", "dwo")):
        assert torch.equal(a, b), f"{n} differs bitwise between head_chunk 4 and 32"
        assert torch.isfinite(a).all(), f"{n} has non-finite values"
    rows = np.array([0, 1, 127, 128, 4095, S // 2, S - 2, S - 1])
    cpu = {n: t.cpu() for n, t in inp.items()}
    ry, rl = orc.layer_fwd_rows(cpu["x"], cpu["wq"], cpu["wk"], cpu["wv"], cpu["wo"], rows, Hq, Hkv,
                                D, True)
    y, lse = outs[0][0], outs[0][1]
    check("y rows", y[rows], ry)
    lerr = float(np.max(np.abs(f64(lse[:, rows]) - rl)))
    print(f"  lse rows: max-abs {lerr:.3e}", flush=True)
    assert lerr <= 1e-2


@pytest.mark.parametrize("S,dm,Hq,Hkv,D,causal,hc_f,hc_b", [
    (300, 128, 8, 2, 64, True, 8, 3),      # groups split across chunks, ragged S
    (1000, 256, 4, 2, 128, True, 4, 1),
    (513, 192, 4, 1, 128, False, 3, 4),    # non-causal, ragged chunk
])
def test_layer_backward_from_kept_output_is_bitwise_the_recomputing_one(S, dm, Hq, Hkv, D, causal,
                                                                        hc_f, hc_b):
    # the forward keeps the attention output and LSE (keep_o); a backward that
    # reads them instead of recomputing gives the same bits, whatever the two
    # calls' head_chunk, and the forward's y is unchanged by keeping
    inp = layer_inputs(S, dm, Hq, Hkv, D, 90 + S % 13)
    d = {n: t.to(DEV) for n, t in inp.items()}
    w = (d["x"], d["wq"], d["wk"], d["wv"], d["wo"])
    print(f"layer keep-O S={S} dm={dm} Hq={Hq} Hkv={Hkv} D={D} causal={causal} "
          f"hc {hc_f} / {hc_b}", flush=True)
    y0, l0 = attn_layer_fwd(*w, Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc_f, causal=causal, with_lse=True)
    y1, l1, o1 = attn_layer_fwd(*w, Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc_f, causal=causal,
                                keep_o=True)
    g0 = attn_layer_bwd(*w, d["dy"], Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc_b, causal=causal)
    g1 = attn_layer_bwd(*w, d["dy"], Hq=Hq, Hkv=Hkv, D=D, head_chunk=hc_b, causal=causal,
                        o_kept=o1, lse_kept=l1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(l0, l1)
    for a, b, n in zip(g0, g1, ("dx", "dwq", "dwk", "dwv", "dwo")):
        assert torch.equal(a, b), f"{n} differs between kept and recomputed attention output"


def test_kept_output_is_the_attention_output_head_major():
    # identity projections: the kept output is attn_fwd's output, head-major
    from head_chunked_context_amd import attn_fwd
    S, Hq, D = 640, 2, 128
    dm = Hq * D
    g = torch.Generator(device="cpu").manual_seed(6)
    x = torch.randn((S, dm), generator=g).to(torch.bfloat16).to(DEV)
    eye = torch.eye(dm, dtype=torch.bfloat16, device=DEV)
    y, lse, o = attn_layer_fwd(x, eye, eye, eye, eye, Hq=Hq, Hkv=Hq, D=D, head_chunk=1,
                               keep_o=True)
    xs = x.view(S, Hq, D).contiguous()
    ref, l = attn_fwd(xs, xs, xs, head_chunk=2)
    torch.cuda.synchronize()
    assert torch.equal(o, ref.permute(1, 0, 2).contiguous())
    assert torch.equal(lse, l)
