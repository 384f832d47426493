"""head_chunked_context_amd: head-chunked, KV-trunked causal GQA attention for MI355X.

``attn_fwd`` / ``attn_bwd`` call the C ABI of ``libhcattn.so`` (built in-tree by
``python -m head_chunked_context_amd.build``); the library is loaded on first
use, so importing this package does not need a GPU.
"""
from .hcattn import (HcAttnError, attn_bwd, attn_fwd, attn_fwd_noalloc,  # noqa: F401
                     attn_layer_bwd, attn_layer_fwd, bwd_workspace_bytes,
                     layer_bwd_workspace_bytes, layer_fwd_workspace_bytes,
                     fwd_workspace_bytes, last_error, pick_kv_trunk, set_group_loop_min_s, set_single_stream,
                     set_trunk_merge, timing_bytes, timing_enable, timing_read, timing_reset,
                     version)
