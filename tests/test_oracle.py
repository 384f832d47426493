"""Pins for the fp64 oracle, independent of the oracle itself.

The pages print no worked numbers for attention, so the oracle is pinned by:
brute-force central finite differences of L = sum(O * dO), closed forms
(Q = 0, equal keys, row 0, S = 1, a 3-token worked example whose forward and
backward values, derived by hand, are stored in tests/golden/), the library
routine torch scaled_dot_product_attention (+ autograd) in fp64 on the CPU,
the structural identities of the gradients, and the invariances the pages
rely on (head chunks reuse buffers without changing results; key trunks merge
by softmax statistics into the untrunked result).
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle as orc

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def small(S, Hq, Hkv, D, seed=0, qs=1.0):
    return (rnd((S, Hq, D), seed, qs), rnd((S, Hkv, D), seed + 1), rnd((S, Hkv, D), seed + 2),
            rnd((S, Hq, D), seed + 3))


# --------------------------------------------------------------- finite diffs

@pytest.mark.parametrize("S", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("D", [4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_gradients_match_central_differences(S, D, causal):
    Hq, Hkv = 4, 2
    q, k, v, do = small(S, Hq, Hkv, D, seed=10 * S + D)
    g = orc.attn_bwd(q, k, v, do, causal)

    def loss(q_, k_, v_):
        o, _ = orc.attn_fwd(q_, k_, v_, causal)
        return float(np.sum(o * do))

    for name, x, an in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        fd = np.empty_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            h = 1e-5 * max(1.0, abs(x[idx]))
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(fd - an))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(an))), (name, err)


# ---------------------------------------------------- library cross-checks

def torch_ref(q, k, v, do, causal):
    """torch SDPA in fp64 on the CPU, K/V repeated to every query head."""
    g = q.shape[1] // k.shape[1]
    qt = torch.tensor(q).permute(1, 0, 2).contiguous().requires_grad_(True)
    kt = torch.tensor(k).requires_grad_(True)
    vt = torch.tensor(v).requires_grad_(True)
    kr = kt.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
    vr = vt.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kr, vr, is_causal=causal)
    o.backward(torch.tensor(do).permute(1, 0, 2))
    return (o.detach().permute(1, 0, 2).numpy(), qt.grad.permute(1, 0, 2).numpy(),
            kt.grad.numpy(), vt.grad.numpy())


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,Hq,Hkv,D", [(50, 4, 2, 16), (33, 6, 3, 8), (17, 4, 4, 32)])
def test_matches_torch_sdpa_fp64(S, Hq, Hkv, D, causal):
    q, k, v, do = small(S, Hq, Hkv, D, seed=S)
    o, _ = orc.attn_fwd(q, k, v, causal)
    g = orc.attn_bwd(q, k, v, do, causal)
    ro, rdq, rdk, rdv = torch_ref(q, k, v, do, causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dq"], rdq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dk"], rdk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dv"], rdv, rtol=0, atol=1e-11)


def test_matches_torch_sdpa_peaked_softmax():
    # Q scaled by 8: peaked rows exercise the max subtraction
    q, k, v, do = small(64, 2, 1, 16, seed=7, qs=8.0)
    o, _ = orc.attn_fwd(q, k, v, True)
    ro, rdq, rdk, rdv = torch_ref(q, k, v, do, True)
    g = orc.attn_bwd(q, k, v, do, True)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-11)
    np.testing.assert_allclose(g["dq"], rdq, rtol=0, atol=1e-10)
    np.testing.assert_allclose(g["dk"], rdk, rtol=0, atol=1e-10)


# ------------------------------------------------------------- closed forms

def test_worked_example_three_tokens():
    # D = 1 so the scale is 1; s_ij = q_i * k_j.
    q = np.array([1.0, 2.0, 0.0]).reshape(3, 1, 1)
    k = np.array([0.0, 1.0, 1.0]).reshape(3, 1, 1)
    v = np.array([3.0, -1.0, 5.0]).reshape(3, 1, 1)
    o, lse = orc.attn_fwd(q, k, v, True)
    e2 = math.exp(2.0)
    # row 0 sees key 0 only: O = v0, LSE = q0 k0 = 0
    assert o[0, 0, 0] == pytest.approx(3.0, abs=1e-15) and lse[0, 0] == pytest.approx(0.0, abs=1e-15)
    # row 1: scores (0, 2)
    assert lse[0, 1] == pytest.approx(math.log(1.0 + e2), abs=1e-14)
    assert o[1, 0, 0] == pytest.approx((3.0 - e2) / (1.0 + e2), abs=1e-14)
    # row 2: q = 0, uniform over three keys
    assert lse[0, 2] == pytest.approx(math.log(3.0), abs=1e-14)
    assert o[2, 0, 0] == pytest.approx(7.0 / 3.0, abs=1e-14)
    # non-causal row 0 sees all keys: scores (0, 1, 1)
    o2, lse2 = orc.attn_fwd(q, k, v, False)
    e1 = math.exp(1.0)
    assert lse2[0, 0] == pytest.approx(math.log(1 + 2 * e1), abs=1e-14)
    assert o2[0, 0, 0] == pytest.approx((3.0 + e1 * (-1.0 + 5.0)) / (1 + 2 * e1), abs=1e-14)


def _closed_form(expr: str, names: dict) -> float:
    """Evaluate a hand-written closed form: numbers, + - * /, unary minus,
    exp, log and previously defined names only."""
    import ast
    import operator as op
    bins = {ast.Add: op.add, ast.Sub: op.sub, ast.Mult: op.mul, ast.Div: op.truediv}
    funcs = {"exp": math.exp, "log": math.log}

    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.BinOp) and type(n.op) in bins:
            return bins[type(n.op)](ev(n.left), ev(n.right))
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, ast.USub):
            return -ev(n.operand)
        if isinstance(n, ast.Name) and n.id in names:
            return names[n.id]
        if isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id in funcs \
                and len(n.args) == 1:
            return funcs[n.func.id](ev(n.args[0]))
        raise ValueError(f"unsupported closed form: {expr}")
    return ev(ast.parse(expr, mode="eval"))


def _golden_files():
    import glob
    import os
    return sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "*.json")))


def _check_golden(path):
    import json
    with open(path) as f:
        g = json.load(f)
    names = {}
    for n, e in g["names"].items():
        names[n] = _closed_form(e, names)
    x = g["inputs"]
    S, Hq, Hkv, D = x["S"], x["Hq"], x["Hkv"], x["D"]
    shape = {"q": (S, Hq, D), "k": (S, Hkv, D), "v": (S, Hkv, D), "dout": (S, Hq, D)}
    q, k, v, do = (np.array(x[n], dtype=np.float64).reshape(shape[n])
                   for n in ("q", "k", "v", "dout"))
    o, lse = orc.attn_fwd(q, k, v, x["causal"])
    grads = orc.attn_bwd(q, k, v, do, x["causal"])
    got = {"o": o, "lse": lse, "dq": grads["dq"], "dk": grads["dk"], "dv": grads["dv"]}
    # the same forward through the oracle's schedules of the pages: key trunks
    # of one token merged by log-sum-exp, and one query head per chunk
    got["o (trunked)"], got["lse (trunked)"] = orc.attn_fwd_trunked(q, k, v, 1, x["causal"])
    got["o (chunked)"], got["lse (chunked)"] = orc.attn_fwd_chunked(q, k, v, 1, x["causal"])
    ev = np.vectorize(lambda e: _closed_form(e, names), otypes=[np.float64])
    for n in got:
        want = ev(np.array(g["expected"][n.split(" ")[0]], dtype=object)).reshape(got[n].shape)
        np.testing.assert_allclose(got[n], want, rtol=0, atol=g["tolerance"], err_msg=n)


@pytest.mark.parametrize("name", [os.path.basename(p) for p in _golden_files()])
def test_golden_worked_examples(name):
    """tests/golden/*.json: small examples whose outputs and gradients were
    derived by hand from the definition (a 3-token single head with D = 1;
    two query heads sharing one key/value head with D = 4)."""
    _check_golden(os.path.join(os.path.dirname(__file__), "golden", name))


def test_q_zero_closed_form():
    S, Hq, Hkv, D = 40, 4, 2, 8
    _, k, v, do = small(S, Hq, Hkv, D, seed=3)
    q = np.zeros((S, Hq, D))
    o, lse = orc.attn_fwd(q, k, v, True)
    i = np.arange(S)
    for h in range(Hq):
        np.testing.assert_allclose(lse[h], np.log(i + 1.0), rtol=0, atol=1e-13)
        prefix = np.cumsum(v[:, h // 2, :], axis=0) / (i + 1.0)[:, None]
        np.testing.assert_allclose(o[:, h, :], prefix, rtol=0, atol=1e-13)
    g = orc.attn_bwd(q, k, v, do, True)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-13)
    for kv in range(Hkv):
        acc = np.zeros((S, D))
        for h in range(kv * 2, kv * 2 + 2):
            w = do[:, h, :] / (i + 1.0)[:, None]
            acc += np.cumsum(w[::-1], axis=0)[::-1]  # suffix sums over i >= j
        np.testing.assert_allclose(g["dv"][:, kv, :], acc, rtol=0, atol=1e-12)


def test_equal_keys_closed_form():
    S, Hq, Hkv, D = 30, 2, 1, 8
    q, _, v, do = small(S, Hq, Hkv, D, seed=4)
    krow = rnd((D,), 99)
    k = np.broadcast_to(krow, (S, Hkv, D)).copy()
    o, lse = orc.attn_fwd(q, k, v, True)
    c = 1 / math.sqrt(D)
    i = np.arange(S)
    for h in range(Hq):
        np.testing.assert_allclose(lse[h], c * q[:, h, :] @ krow + np.log(i + 1.0), atol=1e-12)
        np.testing.assert_allclose(o[:, h, :], np.cumsum(v[:, 0, :], 0) / (i + 1.0)[:, None],
                                   atol=1e-12)
    g = orc.attn_bwd(q, k, v, do, True)
    np.testing.assert_allclose(g["dq"], 0.0, atol=1e-12)


def test_row_zero_and_single_token():
    S, Hq, Hkv, D = 9, 4, 2, 16
    q, k, v, _ = small(S, Hq, Hkv, D, seed=5)
    o, lse = orc.attn_fwd(q, k, v, True)
    c = 1 / math.sqrt(D)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], v[0, h // 2], atol=1e-15)
        assert lse[h, 0] == pytest.approx(c * q[0, h] @ k[0, h // 2], abs=1e-14)
    o1, lse1 = orc.attn_fwd(q[:1], k[:1], v[:1], False)
    for h in range(Hq):
        np.testing.assert_allclose(o1[0, h], v[0, h // 2], atol=1e-15)


def test_one_hot_values_expose_a_stochastic_causal_p():
    # v_j = e_j (D = S) makes O_i the probability row P_i.
    S = D = 8
    q, k, _, _ = small(S, 2, 1, D, seed=6)
    v = np.eye(S).reshape(S, 1, D)
    for causal in (True, False):
        o, _ = orc.attn_fwd(q, k, v, causal)
        for h in range(2):
            P = o[:, h, :]
            np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)
            assert np.all(P >= 0)
            if causal:
                assert np.all(np.triu(P, 1) == 0.0)
                assert np.all(np.diag(P) > 0)
            else:
                assert np.all(P > 0)


def test_delta_equals_rowsum_of_dout_times_out():
    S, Hq, Hkv, D = 24, 4, 1, 8
    q, k, v, do = small(S, Hq, Hkv, D, seed=8)
    o, _ = orc.attn_fwd(q, k, v, True)
    g = orc.attn_bwd(q, k, v, do, True)
    np.testing.assert_allclose(g["delta"], np.einsum("shd,shd->hs", do, o), atol=1e-12)


# ------------------------------------------------------------- identities

@pytest.mark.parametrize("causal", [True, False])
def test_gradient_identities(causal):
    S, Hq, Hkv, D = 37, 6, 2, 8
    q, k, v, do = small(S, Hq, Hkv, D, seed=9)
    g = orc.attn_bwd(q, k, v, do, causal)
    grp = Hq // Hkv
    # sum_j dS_ij = 0  =>  sum_j dK_j = 0
    np.testing.assert_allclose(g["dk"].sum(0), 0.0, atol=1e-11)
    # rows of P sum to 1  =>  sum_j dV_j = sum over the group's heads and rows of dO
    for kv in range(Hkv):
        np.testing.assert_allclose(g["dv"][:, kv].sum(0),
                                   do[:, kv * grp:(kv + 1) * grp].sum((0, 1)), atol=1e-11)
    # scale homogeneity: s depends on q and k only through q.k
    lhs = np.sum(q * g["dq"])
    rhs = np.sum(k * g["dk"])
    assert lhs == pytest.approx(rhs, abs=1e-10)


def test_shift_invariances():
    S, Hq, Hkv, D = 20, 2, 1, 8
    q, k, v, do = small(S, Hq, Hkv, D, seed=11)
    cv = rnd((D,), 12)
    o, lse = orc.attn_fwd(q, k, v, True)
    g = orc.attn_bwd(q, k, v, do, True)
    # V + c: O + c, gradients unchanged
    o2, lse2 = orc.attn_fwd(q, k, v + cv, True)
    g2 = orc.attn_bwd(q, k, v + cv, do, True)
    np.testing.assert_allclose(o2, o + cv, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g2[n], g[n], atol=1e-11)
    # K + c: each row's scores shift by one constant, so O and all gradients stay
    o3, _ = orc.attn_fwd(q, k + cv, v, True)
    g3 = orc.attn_bwd(q, k + cv, v, do, True)
    np.testing.assert_allclose(o3, o, atol=1e-12)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(g3[n], g[n], atol=1e-11)


# ------------------------------------------------------ GQA, chunks, trunks

@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_repeated_kv(causal):
    S, Hq, Hkv, D = 29, 8, 2, 8
    q, k, v, do = small(S, Hq, Hkv, D, seed=13)
    grp = Hq // Hkv
    kr, vr = np.repeat(k, grp, axis=1), np.repeat(v, grp, axis=1)
    o, lse = orc.attn_fwd(q, k, v, causal)
    orr, lser = orc.attn_fwd(q, kr, vr, causal)
    np.testing.assert_array_equal(o, orr)
    np.testing.assert_array_equal(lse, lser)
    g = orc.attn_bwd(q, k, v, do, causal)
    gr = orc.attn_bwd(q, kr, vr, do, causal)
    np.testing.assert_array_equal(g["dq"], gr["dq"])
    np.testing.assert_allclose(g["dk"], gr["dk"].reshape(S, Hkv, grp, D).sum(2), atol=1e-12)
    np.testing.assert_allclose(g["dv"], gr["dv"].reshape(S, Hkv, grp, D).sum(2), atol=1e-12)


@pytest.mark.parametrize("hc", [1, 2, 3, 4, 5, 8])
def test_head_chunks_reuse_buffers_without_changing_results(hc):
    S, Hq, Hkv, D = 23, 8, 2, 8
    q, k, v, _ = small(S, Hq, Hkv, D, seed=14)
    o, lse = orc.attn_fwd(q, k, v, True)
    oc, lsec = orc.attn_fwd_chunked(q, k, v, hc, True)
    np.testing.assert_array_equal(oc, o)
    np.testing.assert_array_equal(lsec, lse)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S,T", [(37, 8), (64, 16), (50, 50), (50, 64), (40, 1)])
def test_key_trunks_merge_to_untrunked(S, T, causal):
    q, k, v, _ = small(S, 4, 2, 8, seed=15, qs=3.0)
    o, lse = orc.attn_fwd(q, k, v, causal)
    ot, lset = orc.attn_fwd_trunked(q, k, v, T, causal)
    np.testing.assert_allclose(ot, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lset, lse, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------- sampled entries

def test_sampled_rows_and_columns_match_full():
    S, Hq, Hkv, D = 45, 4, 2, 8
    q, k, v, do = small(S, Hq, Hkv, D, seed=16)
    for causal in (True, False):
        o, lse = orc.attn_fwd(q, k, v, causal)
        g = orc.attn_bwd(q, k, v, do, causal)
        rows = np.array([0, 7, 31, 44])
        orow, lrow = orc.attn_fwd_rows(q[rows], rows, k, v, causal)
        np.testing.assert_array_equal(orow, o[rows])
        np.testing.assert_array_equal(lrow, lse[:, rows])
        dqr, dr = orc.attn_dq_rows(q[rows], do[rows], rows, k, v, causal)
        np.testing.assert_allclose(dqr, g["dq"][rows], atol=1e-14)
        np.testing.assert_allclose(dr, g["delta"][:, rows], atol=1e-14)
        cols = np.array([40, 41, 44]) if causal else np.array([0, 5, 44])
        i0 = 38 if causal else 0
        dkc, dvc = orc.attn_dkdv_cols(q[i0:], do[i0:], i0, k, v, cols, causal)
        np.testing.assert_allclose(dkc, g["dk"][cols], atol=1e-14)
        np.testing.assert_allclose(dvc, g["dv"][cols], atol=1e-14)


def test_rejects_bad_shapes():
    q, k, v, do = small(4, 3, 2, 4)
    with pytest.raises(ValueError):
        orc.attn_fwd(q, k, v, True)
    q, k, v, do = small(4, 4, 2, 4)
    with pytest.raises(ValueError):
        orc.attn_fwd_rows(q[:1], [4], k, v, True)
    with pytest.raises(ValueError):
        orc.attn_dkdv_cols(q[2:], do[2:], 2, k, v, [1], True)
