"""Thin ctypes binding of libhcattn.so (include/hcattn.h).

Argument marshalling only: every step of attention runs in the library's HIP
kernels.  PyTorch provides device/pinned memory and the current HIP stream.
The library is loaded on first use; if it is missing the call raises (there
is no fallback path).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhcattn.so")

ATTN_OK = 0
STATUS = {0: "ATTN_OK", -1: "ATTN_EINVAL", -2: "ATTN_EUNSUPPORTED", -3: "ATTN_EWORKSPACE",
          -4: "ATTN_EPOINTER", -5: "ATTN_EHIP"}

_lib = None


class HcAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def lib():
    """Load libhcattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m head_chunked_context_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    shape = [i64, i32, i32, i32, i32, i32, i64]
    L.attn_fwd_workspace_bytes.argtypes = shape
    L.attn_fwd_workspace_bytes.restype = sz
    L.attn_bwd_workspace_bytes.argtypes = shape
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_fwd.argtypes = [vp] * 5 + shape + [vp, sz, vp]
    L.attn_fwd.restype = ctypes.c_int
    L.attn_bwd.argtypes = [vp] * 9 + shape + [vp, sz, vp]
    L.attn_bwd.restype = ctypes.c_int
    L.attn_pick_kv_trunk.argtypes = shape[:6] + [ctypes.c_int32, ctypes.c_int32, sz,
                                                  ctypes.c_double, ctypes.c_double,
                                                  ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
    L.attn_pick_kv_trunk.restype = ctypes.c_int
    L.attn_fwd_noalloc.argtypes = [vp] * 5 + shape + [vp]
    L.attn_fwd_noalloc.restype = ctypes.c_int
    lshape = [i64, i32, i32, i32, i32, i32, i32]  # S, d_model, Hq, Hkv, D, causal, head_chunk
    L.attn_layer_fwd_workspace_bytes.argtypes = lshape
    L.attn_layer_fwd_workspace_bytes.restype = sz
    L.attn_layer_bwd_workspace_bytes.argtypes = lshape
    L.attn_layer_bwd_workspace_bytes.restype = sz
    L.attn_layer_fwd.argtypes = [vp] * 8 + lshape + [vp, sz, vp]
    L.attn_layer_fwd.restype = ctypes.c_int
    L.attn_layer_bwd.argtypes = [vp] * 13 + lshape + [vp, sz, vp]
    L.attn_layer_bwd.restype = ctypes.c_int
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_set_single_stream.argtypes = [ctypes.c_int]
    L.attn_set_single_stream.restype = ctypes.c_int
    L.attn_set_trunk_merge.argtypes = [ctypes.c_int]
    L.attn_set_trunk_merge.restype = ctypes.c_int
    L.attn_set_group_loop_min_s.argtypes = [i64]
    L.attn_set_group_loop_min_s.restype = i64
    L.attn_version.argtypes = []
    L.attn_version.restype = ctypes.c_char_p
    L.attn_timing_enable.argtypes = [ctypes.c_int]
    L.attn_timing_enable.restype = ctypes.c_int
    L.attn_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                   ctypes.POINTER(ctypes.c_double)]
    L.attn_timing_read.restype = ctypes.c_int
    L.attn_timing_reset.argtypes = []
    L.attn_timing_reset.restype = None
    L.attn_timing_bytes.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double)]
    L.attn_timing_bytes.restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().attn_last_error().decode()


def _check(rc: int):
    if rc != ATTN_OK:
        raise HcAttnError(rc, last_error())


def _dims(q, k):
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [S, Hq, D] and k [S, Hkv, D]")
    S, Hq, D = q.shape
    if k.shape[0] != S or k.shape[2] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return S, Hq, k.shape[1], D


def _bf16(name, t):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor")


def _validate(specs, kv_names):
    """Check every tensor the call hands to the C ABI, which sees only
    pointers: specs are (name, tensor or None, shape, dtype); None (an output
    the binding allocates itself) is skipped.  Shapes, dtypes and contiguity
    come first; then placement: the first tensor (q) and every tensor not in
    kv_names on one GPU, and those in kv_names (k, v, dk, dv) all on that GPU
    or all in host memory (pinned; the trunked path streams them).  Returns
    (q's device, the k/v device)."""
    specs = [x for x in specs if x[1] is not None]
    for name, t, shape, dtype in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    dev = specs[0][1].device
    if dev.type != "cuda":
        raise ValueError(f"{specs[0][0]} must be on a GPU (is on {dev})")
    kvdev = None
    for name, t, _, _ in specs:
        if name in kv_names:
            if kvdev is None:
                kvdev = t.device
            if t.device != kvdev:
                raise ValueError(f"{name} is on {t.device}, k on {kvdev}")
            if t.device != dev and t.device.type != "cpu":
                raise ValueError(f"{name} is on {t.device}, q on {dev}")
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")
    return dev, kvdev


def fwd_workspace_bytes(S, Hq, Hkv, D, causal=True, head_chunk=0, kv_trunk=0) -> int:
    n = lib().attn_fwd_workspace_bytes(S, Hq, Hkv, D, int(causal), head_chunk, kv_trunk)
    if n == 0:
        raise HcAttnError(-1, last_error())
    return n


def bwd_workspace_bytes(S, Hq, Hkv, D, causal=True, head_chunk=0, kv_trunk=0) -> int:
    n = lib().attn_bwd_workspace_bytes(S, Hq, Hkv, D, int(causal), head_chunk, kv_trunk)
    if n == 0:
        raise HcAttnError(-1, last_error())
    return n


def pick_kv_trunk(S, Hq, Hkv, D, causal=True, head_chunk=0, *, kv_on_host=False,
                  with_backward=True, budget_bytes=0, link_bytes_per_s=0.0, flops_per_s=0.0,
                  num_cus=0) -> int:
    """kv_trunk for a device-memory budget (0 = untrunked); see attn_pick_kv_trunk."""
    t = ctypes.c_int64(-1)
    _check(lib().attn_pick_kv_trunk(S, Hq, Hkv, D, int(causal), head_chunk, int(kv_on_host),
                                    int(with_backward), budget_bytes, float(link_bytes_per_s),
                                    float(flops_per_s), num_cus, ctypes.byref(t)))
    return int(t.value)


def _stream(device) -> int:
    if device.type != "cuda":  # the library rejects such tensors before using the stream
        return torch.cuda.current_stream().cuda_stream
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes, device, workspace):
    if workspace is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or \
            not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, "
                         f"needs {nbytes}")
    return workspace


def attn_fwd(q, k, v, *, head_chunk: int = 0, kv_trunk: int = 0, causal: bool = True,
             out=None, lse=None, workspace=None, with_lse: bool = True):
    """Causal GQA attention forward.  q [S,Hq,D] bf16 on the GPU; k, v [S,Hkv,D]
    bf16 on the GPU or, with kv_trunk, in pinned host memory.  Returns
    (o [S,Hq,D] bf16, lse [Hq,S] fp32); with_lse=False (forward-only use)
    keeps no LSE and returns (o, None)."""
    for n, t in (("q", q), ("k", k)):
        _bf16(n, t)
    S, Hq, Hkv, D = _dims(q, k)
    bf = torch.bfloat16
    dev, _ = _validate([("q", q, q.shape, bf), ("k", k, k.shape, bf), ("v", v, k.shape, bf),
                        ("out", out, q.shape, bf),
                        ("lse", lse if with_lse else None, (Hq, S), torch.float32)],
                       ("k", "v"))
    o = torch.empty_like(q) if out is None else out
    l = None
    if with_lse:
        l = torch.empty((Hq, S), dtype=torch.float32, device=dev) if lse is None else lse
    nb = fwd_workspace_bytes(S, Hq, Hkv, D, causal, head_chunk, kv_trunk)
    ws = _workspace(nb, dev, workspace)
    rc = lib().attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                        l.data_ptr() if l is not None else None,
                        S, Hq, Hkv, D, int(causal), head_chunk, kv_trunk, ws.data_ptr(), nb,
                        _stream(dev))
    _check(rc)
    return o, l


def attn_fwd_noalloc(q, k, v, *, head_chunk: int = 0, kv_trunk: int = 0, causal: bool = True,
                     out=None, lse=None, with_lse: bool = True):
    """attn_fwd on the library's built-in workspace (attn_fwd_noalloc: no
    device allocation inside the call; ATTN_NOALLOC_WORKSPACE_BYTES per GPU).
    Pass out (and lse) to allocate nothing at all."""
    for n, t in (("q", q), ("k", k)):
        _bf16(n, t)
    S, Hq, Hkv, D = _dims(q, k)
    bf = torch.bfloat16
    dev, _ = _validate([("q", q, q.shape, bf), ("k", k, k.shape, bf), ("v", v, k.shape, bf),
                        ("out", out, q.shape, bf),
                        ("lse", lse if with_lse else None, (Hq, S), torch.float32)],
                       ("k", "v"))
    o = torch.empty_like(q) if out is None else out
    l = None
    if with_lse:
        l = torch.empty((Hq, S), dtype=torch.float32, device=dev) if lse is None else lse
    rc = lib().attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                l.data_ptr() if l is not None else None,
                                S, Hq, Hkv, D, int(causal), head_chunk, kv_trunk, _stream(dev))
    _check(rc)
    return o, l


def attn_bwd(q, k, v, o, dout, lse, *, head_chunk: int = 0, kv_trunk: int = 0,
             causal: bool = True, dq=None, dk=None, dv=None, workspace=None):
    """Backward of attn_fwd.  Returns (dq, dk, dv) in bf16; dk/dv are placed
    where k lives (device, or pinned host memory)."""
    for n, t in (("q", q), ("k", k)):
        _bf16(n, t)
    S, Hq, Hkv, D = _dims(q, k)
    bf = torch.bfloat16
    dev, kvdev = _validate([("q", q, q.shape, bf), ("k", k, k.shape, bf), ("v", v, k.shape, bf),
                            ("o", o, q.shape, bf), ("dout", dout, q.shape, bf),
                            ("lse", lse, (Hq, S), torch.float32), ("dq", dq, q.shape, bf),
                            ("dk", dk, k.shape, bf), ("dv", dv, k.shape, bf)],
                           ("k", "v", "dk", "dv"))
    dq = torch.empty_like(q) if dq is None else dq
    pin = kvdev.type == "cpu"
    if dk is None:
        dk = torch.empty(k.shape, dtype=k.dtype, device=kvdev, pin_memory=pin)
    if dv is None:
        dv = torch.empty(k.shape, dtype=k.dtype, device=kvdev, pin_memory=pin)
    nb = bwd_workspace_bytes(S, Hq, Hkv, D, causal, head_chunk, kv_trunk)
    ws = _workspace(nb, dev, workspace)
    rc = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), S, Hq, Hkv, D,
                        int(causal), head_chunk, kv_trunk, ws.data_ptr(), nb, _stream(dev))
    _check(rc)
    return dq, dk, dv


def _layer_specs(x, wq, wk, wv, wo, Hq, Hkv, D):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a [S, d_model] tensor")
    S, dm = x.shape
    bf = torch.bfloat16
    return S, dm, [("x", x, (S, dm), bf), ("wq", wq, (Hq * D, dm), bf),
                   ("wk", wk, (Hkv * D, dm), bf), ("wv", wv, (Hkv * D, dm), bf),
                   ("wo", wo, (dm, Hq * D), bf)]


def layer_fwd_workspace_bytes(S, d_model, Hq, Hkv, D, causal=True, head_chunk=0) -> int:
    n = lib().attn_layer_fwd_workspace_bytes(S, d_model, Hq, Hkv, D, int(causal), head_chunk)
    if n == 0:
        raise HcAttnError(-1, last_error())
    return n


def layer_bwd_workspace_bytes(S, d_model, Hq, Hkv, D, causal=True, head_chunk=0) -> int:
    n = lib().attn_layer_bwd_workspace_bytes(S, d_model, Hq, Hkv, D, int(causal), head_chunk)
    if n == 0:
        raise HcAttnError(-1, last_error())
    return n


def attn_layer_fwd(x, wq, wk, wv, wo, *, Hq: int, Hkv: int, D: int, head_chunk: int = 0,
                   causal: bool = True, out=None, lse=None, with_lse: bool = False,
                   keep_o: bool = False, o_keep=None, workspace=None):
    """y = attention(x wq^T, x wk^T, x wv^T) wo^T walked head chunk by head chunk
    (attn_layer_fwd).  x [S, d_model] bf16; weights [out, in] bf16.  Returns
    (y [S, d_model] fp32, lse [Hq, S] fp32 or None), plus the attention output
    o [Hq, S, D] bf16 as a third element when keep_o (it implies with_lse):
    attn_layer_bwd(..., o_kept=o, lse_kept=lse) then skips recomputing it."""
    S, dm, specs = _layer_specs(x, wq, wk, wv, wo, Hq, Hkv, D)
    with_lse = with_lse or keep_o
    specs += [("out", out, (S, dm), torch.float32),
              ("lse", lse if with_lse else None, (Hq, S), torch.float32),
              ("o_keep", o_keep if keep_o else None, (Hq, S, D), torch.bfloat16)]
    dev, _ = _validate(specs, ())
    y = torch.empty((S, dm), dtype=torch.float32, device=dev) if out is None else out
    l = None
    if with_lse:
        l = torch.empty((Hq, S), dtype=torch.float32, device=dev) if lse is None else lse
    ok = None
    if keep_o:
        ok = torch.empty((Hq, S, D), dtype=torch.bfloat16, device=dev) if o_keep is None else o_keep
    nb = layer_fwd_workspace_bytes(S, dm, Hq, Hkv, D, causal, head_chunk)
    ws = _workspace(nb, dev, workspace)
    _check(lib().attn_layer_fwd(x.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(),
                                wo.data_ptr(), y.data_ptr(), l.data_ptr() if l is not None else None,
                                ok.data_ptr() if ok is not None else None,
                                S, dm, Hq, Hkv, D, int(causal), head_chunk, ws.data_ptr(), nb,
                                _stream(dev)))
    return (y, l, ok) if keep_o else (y, l)


def attn_layer_bwd(x, wq, wk, wv, wo, dy, *, Hq: int, Hkv: int, D: int, head_chunk: int = 0,
                   causal: bool = True, o_kept=None, lse_kept=None, grads=None, workspace=None):
    """Gradients of sum(y * dy) through attn_layer_fwd (attn_layer_bwd): returns
    fp32 (dx, dwq, dwk, dwv, dwo).  dy [S, d_model] bf16.  o_kept / lse_kept: the
    attention output and LSE a forward kept (keep_o=True), or both None to
    recompute them; the results are bitwise the same."""
    S, dm, specs = _layer_specs(x, wq, wk, wv, wo, Hq, Hkv, D)
    if (o_kept is None) != (lse_kept is None):
        raise ValueError("o_kept and lse_kept come together (both None: recompute)")
    f32 = torch.float32
    shapes = [(S, dm), (Hq * D, dm), (Hkv * D, dm), (Hkv * D, dm), (dm, Hq * D)]
    names = ("dx", "dwq", "dwk", "dwv", "dwo")
    grads = list(grads) if grads is not None else [None] * 5
    specs += [("dy", dy, (S, dm), torch.bfloat16)]
    if o_kept is not None:
        specs += [("o_kept", o_kept, (Hq, S, D), torch.bfloat16),
                  ("lse_kept", lse_kept, (Hq, S), f32)]
    specs += [(n, g, sh, f32) for n, g, sh in zip(names, grads, shapes)]
    dev, _ = _validate(specs, ())
    grads = [torch.empty(sh, dtype=f32, device=dev) if g is None else g
             for g, sh in zip(grads, shapes)]
    nb = layer_bwd_workspace_bytes(S, dm, Hq, Hkv, D, causal, head_chunk)
    ws = _workspace(nb, dev, workspace)
    _check(lib().attn_layer_bwd(x.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(),
                                wo.data_ptr(), dy.data_ptr(),
                                o_kept.data_ptr() if o_kept is not None else None,
                                lse_kept.data_ptr() if lse_kept is not None else None,
                                *[g.data_ptr() for g in grads],
                                S, dm, Hq, Hkv, D, int(causal), head_chunk, ws.data_ptr(), nb,
                                _stream(dev)))
    return tuple(grads)


def set_single_stream(on: bool) -> bool:
    """Run trunk copies on the caller's stream (race check); returns the old value."""
    return bool(lib().attn_set_single_stream(int(on)))


def set_trunk_merge(on: bool) -> bool:
    """Trunked forward by log-sum-exp merge of per-trunk partials (True) instead
    of the in-kernel carried state (False, default); returns the old value."""
    return bool(lib().attn_set_trunk_merge(int(on)))


def set_group_loop_min_s(min_s: int) -> int:
    """Sequence length from which the backward's dK/dV pass takes the group-loop
    schedule (0 restores the default, 65536); returns the previous value."""
    return int(lib().attn_set_group_loop_min_s(int(min_s)))


def version() -> str:
    return lib().attn_version().decode()


KERNEL_FAMILIES = ("fwd", "merge", "pack", "prep", "dkdv", "reduce", "dq", "gemm")


def timing_enable(on: bool) -> bool:
    """Bracket every library kernel launch with HIP events (measurement only)."""
    return bool(lib().attn_timing_enable(int(on)))


def timing_reset() -> None:
    lib().attn_timing_reset()


def timing_bytes() -> dict:
    """{family: bytes} moved by the timed streaming-pass launches since the
    last reset (read + write, fixed by their parameters; 0 for MFMA kernels)."""
    out = {}
    for name in KERNEL_FAMILIES:
        b = ctypes.c_double(0.0)
        _check(lib().attn_timing_bytes(name.encode(), ctypes.byref(b)))
        out[name] = float(b.value)
    return out


def timing_read() -> dict:
    """{family: (launches, total_ms)} for the launches since the last reset."""
    out = {}
    for name in KERNEL_FAMILIES:
        n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
        _check(lib().attn_timing_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)))
        out[name] = (int(n.value), float(ms.value))
    return out
