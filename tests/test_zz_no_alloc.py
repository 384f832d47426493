"""attn_fwd_noalloc (the forward on the library's built-in workspace, for
callers that cannot allocate device memory) against attn_fwd with a caller
workspace, through the C ABI: bit for bit, and against the oracle, on two
calls in a row, the second with a smaller input (the built-in workspace
keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from head_chunked_context_amd import attn_fwd, attn_fwd_noalloc
from head_chunked_context_amd.hcattn import HcAttnError, lib
from tests.gpu_util import DEV, check_fwd, inputs_cpu, to_dev

pytestmark = pytest.mark.gpu

NOALLOC_BYTES = 64 << 20


@pytest.mark.parametrize("cases", [[(1100, 8, 2, 128, 4, 0, False), (300, 4, 2, 64, 2, 0, False)],
                                   [(1600, 4, 1, 128, 2, 512, True), (777, 2, 1, 128, 1, 256, False)]])
def test_noalloc_forward_equals_workspace_forward(cases):
    for S, Hq, Hkv, D, hc, T, kv_host in cases:
        print(f"noalloc S={S} Hq={Hq} Hkv={Hkv} D={D} hc={hc} T={T} kv_host={kv_host}", flush=True)
        inp = inputs_cpu(S, Hq, Hkv, D, 70 + S % 13)
        d = to_dev(inp, kv_host=kv_host)
        o_ref, l_ref = attn_fwd(d["q"], d["k"], d["v"], head_chunk=hc, kv_trunk=T)
        o = torch.empty_like(o_ref)
        lse = torch.empty_like(l_ref)
        o2, l2 = attn_fwd_noalloc(d["q"], d["k"], d["v"], head_chunk=hc, kv_trunk=T, out=o, lse=lse)
        torch.cuda.synchronize()
        assert o2.data_ptr() == o.data_ptr() and l2.data_ptr() == lse.data_ptr()
        assert torch.equal(o, o_ref), "O differs from attn_fwd with a workspace"
        assert torch.equal(lse, l_ref), "LSE differs from attn_fwd with a workspace"
        check_fwd(inp, o, lse)


def test_noalloc_refuses_shapes_beyond_its_workspace():
    from head_chunked_context_amd import fwd_workspace_bytes
    S, Hq, Hkv, D = 262144, 32, 8, 128
    assert fwd_workspace_bytes(S, Hq, Hkv, D, True, 4, 0) > NOALLOC_BYTES
    # nothing is touched: null tensors would be an error only after the size check
    rc = lib().attn_fwd_noalloc(None, None, None, None, None, S, Hq, Hkv, D, 1, 4, 0, None)
    assert rc == -3
    assert "built-in" in lib().attn_last_error().decode()
    # a trunk brings the same shape under the limit
    assert fwd_workspace_bytes(S, Hq, Hkv, D, True, 4, 8192) <= NOALLOC_BYTES
    q = torch.zeros((8, 4, 128), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((8, 1, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(HcAttnError):
        attn_fwd_noalloc(q, k, k, head_chunk=5)
