"""head_chunked_context_amd: head-chunked, KV-trunked causal GQA attention for MI355X."""
