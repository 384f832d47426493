"""Pins for the oracle's attention layer (projections around the attention),
independent of the oracle itself: brute-force central finite differences of
L = sum(y * dy) for every input and weight; torch (matmuls, scaled dot-product
attention and autograd in fp64 on the CPU) as a library cross-check; a closed
form (Wq = 0: every query sees its visible keys uniformly, so y_i is the
prefix mean of x projected through Wv and Wo); the reduction to the attention
oracle (identity projections); and the chunked walk the U-Pipe paragraph
describes equal to the unchunked layer."""
import numpy as np
import pytest
import torch

from oracle import oracle as orc

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def layer_inputs(S, dm, Hq, Hkv, D, seed=0):
    return dict(x=rnd((S, dm), seed), wq=rnd((Hq * D, dm), seed + 1, dm ** -0.5),
                wk=rnd((Hkv * D, dm), seed + 2, dm ** -0.5),
                wv=rnd((Hkv * D, dm), seed + 3, dm ** -0.5),
                wo=rnd((dm, Hq * D), seed + 4, (Hq * D) ** -0.5), dy=rnd((S, dm), seed + 5))


NAMES = ("x", "wq", "wk", "wv", "wo")


@pytest.mark.parametrize("S", [1, 3, 6])
@pytest.mark.parametrize("causal", [True, False])
def test_layer_gradients_match_central_differences(S, causal):
    Hq, Hkv, D, dm = 4, 2, 3, 5
    a = layer_inputs(S, dm, Hq, Hkv, D, seed=7 * S + int(causal))
    g = orc.layer_bwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["dy"], Hq, Hkv, D, causal)

    def loss(**over):
        b = dict(a, **over)
        y, _ = orc.layer_fwd(b["x"], b["wq"], b["wk"], b["wv"], b["wo"], Hq, Hkv, D, causal)
        return float(np.sum(y * a["dy"]))

    for name in NAMES:
        t = a[name]
        fd = np.empty_like(t)
        it = np.nditer(t, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            h = 1e-5 * max(1.0, abs(t[idx]))
            tp, tm = t.copy(), t.copy()
            tp[idx] += h
            tm[idx] -= h
            fd[idx] = (loss(**{name: tp}) - loss(**{name: tm})) / (2 * h)
        an = g["d" + name]
        err = np.max(np.abs(fd - an))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(an))), (name, err)


def torch_layer(a, Hq, Hkv, D, causal):
    """The layer in torch fp64 on the CPU (matmuls + SDPA + autograd)."""
    t = {n: torch.tensor(a[n]).requires_grad_(n != "dy") for n in a}
    S = a["x"].shape[0]
    g = Hq // Hkv
    q = (t["x"] @ t["wq"].T).view(S, Hq, D).permute(1, 0, 2)
    k = (t["x"] @ t["wk"].T).view(S, Hkv, D).repeat_interleave(g, dim=1).permute(1, 0, 2)
    v = (t["x"] @ t["wv"].T).view(S, Hkv, D).repeat_interleave(g, dim=1).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    y = o.permute(1, 0, 2).reshape(S, Hq * D) @ t["wo"].T
    y.backward(t["dy"])
    return y.detach().numpy(), {"d" + n: t[n].grad.numpy() for n in NAMES}


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,dm,Hq,Hkv,D", [(37, 24, 4, 2, 8), (20, 16, 6, 3, 4), (9, 32, 2, 2, 16)])
def test_layer_matches_torch_fp64(S, dm, Hq, Hkv, D, causal):
    a = layer_inputs(S, dm, Hq, Hkv, D, seed=S + dm)
    y, _ = orc.layer_fwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], Hq, Hkv, D, causal)
    g = orc.layer_bwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["dy"], Hq, Hkv, D, causal)
    ty, tg = torch_layer(a, Hq, Hkv, D, causal)
    assert np.max(np.abs(y - ty)) <= 1e-12
    for n in tg:
        assert np.max(np.abs(g[n] - tg[n])) <= 1e-11 * max(1.0, np.max(np.abs(tg[n]))), n


def test_layer_q_projection_zero_closed_form():
    # Wq = 0: all scores are 0, so query i weighs its visible keys 0..i
    # equally: o_i = Wv-projection of the prefix mean of x, y_i = o_i Wo^T
    S, dm, Hq, Hkv, D = 12, 10, 4, 2, 3
    a = layer_inputs(S, dm, Hq, Hkv, D, seed=3)
    a["wq"][:] = 0.0
    y, lse = orc.layer_fwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], Hq, Hkv, D, True)
    prefix = np.cumsum(a["x"], 0) / np.arange(1, S + 1)[:, None]
    v = (prefix @ a["wv"].T).reshape(S, Hkv, D)
    o = np.repeat(v, Hq // Hkv, axis=1).reshape(S, Hq * D)
    assert np.max(np.abs(y - o @ a["wo"].T)) <= 1e-12
    assert np.max(np.abs(lse - np.log(np.arange(1, S + 1))[None, :])) <= 1e-12


def test_identity_projections_reduce_to_the_attention_oracle():
    S, Hq, D = 25, 3, 4
    dm = Hq * D
    a = layer_inputs(S, dm, Hq, Hq, D, seed=5)
    eye = np.eye(dm)
    y, lse = orc.layer_fwd(a["x"], eye, eye, eye, eye, Hq, Hq, D, True)
    xs = a["x"].reshape(S, Hq, D)
    o, l = orc.attn_fwd(xs, xs, xs, True)
    assert np.array_equal(y, o.reshape(S, dm)) and np.array_equal(lse, l)
    g = orc.layer_bwd(a["x"], eye, eye, eye, eye, a["dy"], Hq, Hq, D, True)
    ga = orc.attn_bwd(xs, xs, xs, a["dy"].reshape(S, Hq, D), True)
    dsum = (ga["dq"] + ga["dk"] + ga["dv"]).reshape(S, dm)
    assert np.max(np.abs(g["dx"] - dsum)) <= 1e-12
    assert np.max(np.abs(g["dwo"] - a["dy"].T @ o.reshape(S, dm))) <= 1e-12
    assert np.max(np.abs(g["dwq"] - ga["dq"].reshape(S, dm).T @ a["x"])) <= 1e-12


@pytest.mark.parametrize("hc", [1, 2, 3, 5, 6])
def test_layer_head_chunks_give_the_unchunked_result(hc):
    # g = 2 heads per kv head: hc = 1, 3 and 5 split groups across chunks
    S, dm, Hq, Hkv, D = 30, 16, 6, 3, 4
    a = layer_inputs(S, dm, Hq, Hkv, D, seed=11)
    y, _ = orc.layer_fwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], Hq, Hkv, D, True)
    yc = orc.layer_fwd_chunked(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], Hq, Hkv, D, hc, True)
    assert np.max(np.abs(y - yc)) <= 1e-12 * max(1.0, np.max(np.abs(y)))


def test_layer_is_linear_in_the_output_projection_and_dy():
    S, dm, Hq, Hkv, D = 16, 12, 4, 1, 3
    a = layer_inputs(S, dm, Hq, Hkv, D, seed=13)
    y1, _ = orc.layer_fwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], Hq, Hkv, D, True)
    y2, _ = orc.layer_fwd(a["x"], a["wq"], a["wk"], a["wv"], 2.5 * a["wo"], Hq, Hkv, D, True)
    assert np.max(np.abs(2.5 * y1 - y2)) <= 1e-12
    g1 = orc.layer_bwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], a["dy"], Hq, Hkv, D, True)
    g2 = orc.layer_bwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], -2 * a["dy"], Hq, Hkv, D, True)
    for n in g1:
        assert np.max(np.abs(-2 * g1[n] - g2[n])) <= 1e-11 * max(1.0, np.max(np.abs(g1[n])))


def test_layer_rows_match_the_full_layer():
    S, dm, Hq, Hkv, D = 40, 16, 4, 2, 4
    a = layer_inputs(S, dm, Hq, Hkv, D, seed=17)
    rows = np.array([0, 1, 7, 20, 39])
    for causal in (True, False):
        y, lse = orc.layer_fwd(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], Hq, Hkv, D, causal)
        yr, lr = orc.layer_fwd_rows(a["x"], a["wq"], a["wk"], a["wv"], a["wo"], rows, Hq, Hkv, D,
                                    causal)
        assert np.max(np.abs(yr - y[rows])) <= 1e-13
        assert np.max(np.abs(lr - lse[:, rows])) <= 1e-13
