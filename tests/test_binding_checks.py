"""The Python binding checks every tensor it hands to the C ABI (which sees
only pointers): shapes, dtypes, contiguity and placement, before any call.
These run on the CPU: a mismatched tensor must raise ValueError, never reach
the library as a pointer to a buffer of the wrong size."""
import pytest
import torch

import head_chunked_context_amd as hc

S, HQ, HKV, D = 16, 4, 2, 64
BF = torch.bfloat16


def t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def fwd_args(**over):
    a = dict(q=t(S, HQ, D), k=t(S, HKV, D), v=t(S, HKV, D))
    a.update(over)
    return a


def bwd_args(**over):
    a = dict(q=t(S, HQ, D), k=t(S, HKV, D), v=t(S, HKV, D), o=t(S, HQ, D),
             dout=t(S, HQ, D), lse=t(HQ, S, dtype=torch.float32))
    a.update(over)
    return a


@pytest.mark.parametrize("over,msg", [
    (dict(v=t(S - 1, HKV, D)), "v has shape"),
    (dict(v=t(S, HKV, D, dtype=torch.float16)), "v has dtype"),
    (dict(k=t(S, HKV, D + 1)), "k shape"),
    (dict(q=t(S, HQ, D, dtype=torch.float32)), "q must be a contiguous bfloat16"),
    (dict(v=t(S, D, HKV).transpose(1, 2)), "v must be contiguous"),
])
def test_forward_rejects_mismatched_inputs(over, msg):
    with pytest.raises(ValueError, match=msg):
        hc.attn_fwd(**fwd_args(**over))


@pytest.mark.parametrize("kw,msg", [
    (dict(out=t(S, HQ, D - 1)), "out has shape"),
    (dict(lse=t(S, HQ, dtype=torch.float32)), "lse has shape"),
    (dict(lse=t(HQ, S)), "lse has dtype"),
])
def test_forward_rejects_mismatched_outputs(kw, msg):
    with pytest.raises(ValueError, match=msg):
        hc.attn_fwd(**fwd_args(), **kw)


@pytest.mark.parametrize("over,msg", [
    (dict(o=t(S, HQ - 1, D)), "o has shape"),
    (dict(dout=t(S + 1, HQ, D)), "dout has shape"),
    (dict(lse=t(HQ, S)), "lse has dtype"),
    (dict(lse=t(S, HQ, dtype=torch.float32)), "lse has shape"),
    (dict(v=t(S, HKV, D, dtype=torch.float32)), "v has dtype"),
])
def test_backward_rejects_mismatched_inputs(over, msg):
    with pytest.raises(ValueError, match=msg):
        hc.attn_bwd(**bwd_args(**over))


@pytest.mark.parametrize("kw,msg", [
    (dict(dq=t(S, HQ, D, dtype=torch.float32)), "dq has dtype"),
    (dict(dk=t(S, HQ, D)), "dk has shape"),
    (dict(dv=t(S, HKV, D)[:, :1]), "dv has shape"),
])
def test_backward_rejects_mismatched_outputs(kw, msg):
    a = bwd_args()
    with pytest.raises(ValueError, match=msg):
        hc.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], **kw)


def test_tensors_off_the_gpu_are_rejected_before_the_library():
    # all shapes right, but q lives in host memory: the binding refuses it
    with pytest.raises(ValueError, match="q must be on a GPU"):
        hc.attn_fwd(**fwd_args())
    with pytest.raises(ValueError, match="q must be on a GPU"):
        hc.attn_bwd(**bwd_args())


DM = HQ * D


def layer_args():
    return dict(x=t(S, DM), wq=t(HQ * D, DM), wk=t(HKV * D, DM), wv=t(HKV * D, DM),
                wo=t(DM, HQ * D))


def test_layer_forward_checks_the_kept_output():
    a = layer_args()
    with pytest.raises(ValueError, match="o_keep has shape"):
        hc.attn_layer_fwd(*a.values(), Hq=HQ, Hkv=HKV, D=D, keep_o=True, o_keep=t(S, HQ, D))
    with pytest.raises(ValueError, match="o_keep has dtype"):
        hc.attn_layer_fwd(*a.values(), Hq=HQ, Hkv=HKV, D=D, keep_o=True,
                          o_keep=t(HQ, S, D, dtype=torch.float32))


def test_layer_backward_checks_the_kept_output_and_lse():
    a = list(layer_args().values()) + [t(S, DM)]
    with pytest.raises(ValueError, match="come together"):
        hc.attn_layer_bwd(*a, Hq=HQ, Hkv=HKV, D=D, o_kept=t(HQ, S, D))
    with pytest.raises(ValueError, match="come together"):
        hc.attn_layer_bwd(*a, Hq=HQ, Hkv=HKV, D=D, lse_kept=t(HQ, S, dtype=torch.float32))
    with pytest.raises(ValueError, match="o_kept has shape"):
        hc.attn_layer_bwd(*a, Hq=HQ, Hkv=HKV, D=D, o_kept=t(S, HQ, D),
                          lse_kept=t(HQ, S, dtype=torch.float32))
    with pytest.raises(ValueError, match="lse_kept has dtype"):
        hc.attn_layer_bwd(*a, Hq=HQ, Hkv=HKV, D=D, o_kept=t(HQ, S, D), lse_kept=t(HQ, S))
