"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Each mutation is a textual edit of a copy of ``oracle/orc.c`` (a dropped term,
a wrong sign, a wrong index, a transposed operand, a missing scale), compiled
to a temporary library and swapped into the oracle binding.  The pins in
test_oracle.py then run against the broken oracle; at least one must fail.
Nothing here touches the GPU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from oracle import oracle as orc
from tests import test_oracle as T

SRC = os.path.join(os.path.dirname(orc.__file__), "orc.c")

# (name, old text, new text, count: -1 = every occurrence)
MUTATIONS = [
    ("causal set drops the diagonal",
     "return causal ? i : S - 1;", "return causal ? (i > 0 ? i - 1 : 0) : S - 1;", 1),
    ("scale 1/D instead of 1/sqrt(D)",
     "const double c = 1.0 / sqrt((double)D);", "const double c = 1.0 / (double)D;", -1),
    ("GQA maps head h to kv h % Hkv", "h / g", "h % Hkv", -1),
    ("LSE forgets the max shift", "return m + log(l);", "return log(l);", 1),
    ("output sums keys instead of values",
     "const double* vj = krow(v, j, kv, Hkv, D);\n        for (int d = 0; d < D; ++d) out[d] += p * vj[d];",
     "const double* vj = krow(k, j, kv, Hkv, D);\n        for (int d = 0; d < D; ++d) out[d] += p * vj[d];", 1),
    ("Delta drops P", "delta += p * dot(doi, krow(v, j, kv, Hkv, D), D);",
     "delta += dot(doi, krow(v, j, kv, Hkv, D), D);", 1),
    ("dS sign flipped in dQ", "double ds = p * (dot(doi, krow(v, j, kv, Hkv, D), D) - delta);",
     "double ds = p * (dot(doi, krow(v, j, kv, Hkv, D), D) + delta);", 1),
    ("dQ missing the scale", "        for (int d = 0; d < D; ++d) out[d] += ds * kj[d];\n    }\n    for (int d = 0; d < D; ++d) out[d] *= c;",
     "        for (int d = 0; d < D; ++d) out[d] += ds * kj[d];\n    }", 1),
    ("dK missing the scale", "    for (int d = 0; d < D; ++d) dkj[d] *= c;\n}", "}", 1),
    ("dV weighted by dS instead of P", "dvj[d] += p * doi[d];", "dvj[d] += ds * doi[d];", 1),
    ("dK accumulates dO instead of Q", "dkj[d] += ds * qi[d];", "dkj[d] += ds * doi[d];", 1),
    ("dK/dV miss the group's other heads", "for (int h = kv * g; h < kv * g + g; ++h)",
     "for (int h = kv * g; h < kv * g + 1; ++h)", 1),
    ("trunk merge weights swapped", "orow[d] = wr * orow[d] + wt * ot[d];",
     "orow[d] = wt * orow[d] + wr * ot[d];", 1),
    ("chunk buffers read the wrong kv head", "int kvl = (h0 + hh) / g - kv0;", "int kvl = hh / g;", 1),
]


def pins():
    return [
        ("fd", lambda: T.test_gradients_match_central_differences(3, 4, True)),
        ("fd-noncausal", lambda: T.test_gradients_match_central_differences(8, 4, False)),
        ("sdpa", lambda: T.test_matches_torch_sdpa_fp64(33, 6, 3, 8, True)),
        ("sdpa-noncausal", lambda: T.test_matches_torch_sdpa_fp64(33, 6, 3, 8, False)),
        ("worked example", T.test_worked_example_three_tokens),
        ("q=0", T.test_q_zero_closed_form),
        ("equal keys", T.test_equal_keys_closed_form),
        ("row 0 / S=1", T.test_row_zero_and_single_token),
        ("one-hot V", T.test_one_hot_values_expose_a_stochastic_causal_p),
        ("delta", T.test_delta_equals_rowsum_of_dout_times_out),
        ("identities", lambda: T.test_gradient_identities(True)),
        ("shifts", T.test_shift_invariances),
        ("gqa", lambda: T.test_gqa_equals_repeated_kv(True)),
        ("chunks", lambda: T.test_head_chunks_reuse_buffers_without_changing_results(3)),
        ("trunks", lambda: T.test_key_trunks_merge_to_untrunked(37, 8, True)),
        ("sampled", T.test_sampled_rows_and_columns_match_full),
        ("golden", lambda: [T._check_golden(p) for p in T._golden_files()]),
    ]


# mistakes the hand-derived golden examples alone must catch (they have one
# key/value head, so GQA-index and chunk-buffer mistakes are left to the
# other pins)
GOLDEN_CATCHES = [m[0] for m in MUTATIONS if m[0] not in (
    "GQA maps head h to kv h % Hkv", "chunk buffers read the wrong kv head")]


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="orc_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new,count", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(workdir, name, old, new, count):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new) if count < 0 else src.replace(old, new, count)
    cpath = os.path.join(workdir, "m.c")
    lpath = os.path.join(workdir, f"m_{abs(hash(name))}.so")
    open(cpath, "w").write(mutated)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", lpath, cpath, "-lm"],
                   check=True)
    prev = orc.use_library(lpath)
    caught = []
    try:
        for pin, fn in pins():
            try:
                fn()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                caught.append(pin)
    finally:
        orc.restore_library(prev)
    assert caught, f"no pin caught the planted mistake: {name}"


@pytest.mark.parametrize("name", GOLDEN_CATCHES)
def test_golden_examples_catch_planted_mistake(workdir, name):
    old, new, count = {m[0]: m[1:] for m in MUTATIONS}[name]
    src = open(SRC).read()
    mutated = src.replace(old, new) if count < 0 else src.replace(old, new, count)
    cpath = os.path.join(workdir, "g.c")
    lpath = os.path.join(workdir, f"g_{abs(hash(name))}.so")
    open(cpath, "w").write(mutated)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", lpath, cpath, "-lm"],
                   check=True)
    prev = orc.use_library(lpath)
    try:
        with pytest.raises(AssertionError):
            for p in T._golden_files():
                T._check_golden(p)
    finally:
        orc.restore_library(prev)


# ------------------------------------------------------------ attention layer

LAYER_MUTATIONS = [
    ("value projection uses Wk", "matmul_nt(x, wv, S, dm, nk, v);",
     "matmul_nt(x, wk, S, dm, nk, v);", -1),
    ("dx drops the key-projection term", "        matmul_nn(dk, wk, S, nk, dm, dx, 1);\n", "", 1),
    ("dWq taken against dy instead of x", "matmul_tn(dq, x, S, nq, dm, dwq);",
     "matmul_tn(dq, dy, S, nq, dm, dwq);", 1),
    ("dO not projected back through Wo", "matmul_nn(dy, wo, S, dm, nq, dov, 0);",
     "matmul_nt(dy, wo, S, dm, nq, dov);", 1),
    ("chunked walk keeps only the last chunk's output",
     "y[(size_t)s * dm + m] += dot(", "y[(size_t)s * dm + m] = dot(", 1),
    ("chunk projects the wrong kv heads", "matmul_nt(x, wk + (size_t)kv0 * D * dm, S, dm, nkv * D, kc);",
     "matmul_nt(x, wk, S, dm, nkv * D, kc);", 1),
]


def layer_pins():
    from tests import test_oracle_layer as L
    return [
        ("fd", lambda: L.test_layer_gradients_match_central_differences(3, True)),
        ("torch", lambda: L.test_layer_matches_torch_fp64(20, 16, 6, 3, 4, True)),
        ("wq=0", L.test_layer_q_projection_zero_closed_form),
        ("identity", L.test_identity_projections_reduce_to_the_attention_oracle),
        ("chunks", lambda: L.test_layer_head_chunks_give_the_unchunked_result(3)),
        ("linear", L.test_layer_is_linear_in_the_output_projection_and_dy),
    ]


@pytest.mark.parametrize("name,old,new,count", LAYER_MUTATIONS, ids=[m[0] for m in LAYER_MUTATIONS])
def test_layer_pins_catch_planted_mistake(workdir, name, old, new, count):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {name}"
    mutated = src.replace(old, new) if count < 0 else src.replace(old, new, count)
    cpath = os.path.join(workdir, "l.c")
    lpath = os.path.join(workdir, f"l_{abs(hash(name))}.so")
    open(cpath, "w").write(mutated)
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-o", lpath, cpath, "-lm"],
                   check=True)
    prev = orc.use_library(lpath)
    caught = []
    try:
        for pin, fn in layer_pins():
            try:
                fn()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                caught.append(pin)
    finally:
        orc.restore_library(prev)
    assert caught, f"no layer pin caught the planted mistake: {name}"
