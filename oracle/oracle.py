"""ctypes binding for the fp64 attention oracle in ``orc.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU library never does.

Inputs are numpy arrays or torch tensors of any float dtype; they are widened
to float64, which holds every bf16, fp16 and fp32 value exactly.  Layouts:
q, o, dout ``[S, Hq, D]``; k, v ``[S, Hkv, D]``; lse ``[Hq, S]``.  Outputs are
float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "orc.c")
_LIB = os.path.join(_HERE, "liborc.so")
_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_dp = ctypes.POINTER(ctypes.c_double)
_lp = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile ``orc.c`` into ``liborc.so`` (gcc, OpenMP, generic x86-64-v3)."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-shared", "-fPIC",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def use_library(path: str):
    """Point this binding at another build of ``orc.c`` (the mutation tests
    load deliberately broken copies); returns the previous library handle."""
    global _lib
    prev = _lib
    _lib = _bind(ctypes.CDLL(path))
    return prev


def restore_library(prev) -> None:
    global _lib
    _lib = prev


def _bind(lib):
    shape = [_i64, _int, _int, _int, _int]
    lib.orc_attn_fwd.argtypes = [_dp, _dp, _dp] + shape + [_dp, _dp]
    lib.orc_attn_fwd_rows.argtypes = [_dp, _lp, _i64, _dp, _dp] + shape + [_dp, _dp]
    lib.orc_attn_fwd_trunked.argtypes = [_dp, _dp, _dp] + shape + [_i64, _dp, _dp]
    lib.orc_attn_fwd_chunked.argtypes = [_dp, _dp, _dp] + shape + [_int, _dp, _dp]
    lib.orc_attn_bwd.argtypes = [_dp, _dp, _dp, _dp] + shape + [_dp, _dp, _dp, _dp, _dp]
    lib.orc_attn_dq_rows.argtypes = [_dp, _dp, _lp, _i64, _dp, _dp] + shape + [_dp, _dp]
    lib.orc_attn_dkdv_cols.argtypes = [_dp, _dp, _i64, _dp, _dp] + shape + [_lp, _i64, _dp, _dp]
    lshape = [_i64, _int, _int, _int, _int, _int]  # S, dm, Hq, Hkv, D, causal
    lib.orc_layer_fwd.argtypes = [_dp] * 5 + lshape + [_dp, _dp]
    lib.orc_layer_fwd_chunked.argtypes = [_dp] * 5 + lshape + [_int, _dp]
    lib.orc_layer_bwd.argtypes = [_dp] * 6 + lshape + [_dp] * 5
    lib.orc_layer_fwd_rows.argtypes = [_dp] * 5 + lshape + [_lp, _i64, _dp, _dp]
    for f in (lib.orc_attn_fwd, lib.orc_attn_fwd_rows, lib.orc_attn_fwd_trunked,
              lib.orc_attn_fwd_chunked, lib.orc_attn_bwd, lib.orc_attn_dq_rows,
              lib.orc_attn_dkdv_cols, lib.orc_layer_fwd, lib.orc_layer_fwd_chunked,
              lib.orc_layer_bwd, lib.orc_layer_fwd_rows):
        f.restype = _int
    return lib


def _f64(x) -> np.ndarray:
    """Widen to a contiguous float64 array (exact for bf16, fp16 and fp32)."""
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().cpu()
        if not x.dtype.is_floating_point or x.element_size() < 8:
            x = x.float()
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _rows(r) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(r, dtype=np.int64))


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments (rc={rc})")


def _dims(q, k):
    if q.ndim != 3 or k.ndim != 3 or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [S,Hq,D] and k [S,Hkv,D]")
    return q.shape[1], k.shape[1], q.shape[2]


def attn_fwd(q, k, v, causal: bool = True):
    """Exact forward: returns (o [S,Hq,D], lse [Hq,S]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, Hkv, D = _dims(q, k)
    S = q.shape[0]
    o = np.empty((S, Hq, D))
    lse = np.empty((Hq, S))
    _check(_load().orc_attn_fwd(_p(q), _p(k), _p(v), S, Hq, Hkv, D, int(causal), _p(o), _p(lse)),
           "orc_attn_fwd")
    return o, lse


def attn_fwd_rows(q_rows, rows, k, v, causal: bool = True):
    """Forward for chosen rows.  ``q_rows`` [n,Hq,D] are the query rows at
    positions ``rows``; k, v hold the whole sequence.  Returns (o [n,Hq,D],
    lse [Hq,n])."""
    q_rows, k, v, rows = _f64(q_rows), _f64(k), _f64(v), _rows(rows)
    Hq, Hkv, D = _dims(q_rows, k)
    S, n = k.shape[0], rows.shape[0]
    o = np.empty((n, Hq, D))
    lse = np.empty((Hq, n))
    _check(_load().orc_attn_fwd_rows(_p(q_rows), rows.ctypes.data_as(_lp), n, _p(k), _p(v),
                                     S, Hq, Hkv, D, int(causal), _p(o), _p(lse)),
           "orc_attn_fwd_rows")
    return o, lse


def attn_fwd_trunked(q, k, v, trunk: int, causal: bool = True):
    """Forward over key trunks of ``trunk`` tokens merged by log-sum-exp."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, Hkv, D = _dims(q, k)
    S = q.shape[0]
    o = np.empty((S, Hq, D))
    lse = np.empty((Hq, S))
    _check(_load().orc_attn_fwd_trunked(_p(q), _p(k), _p(v), S, Hq, Hkv, D, int(causal),
                                        int(trunk), _p(o), _p(lse)), "orc_attn_fwd_trunked")
    return o, lse


def attn_fwd_chunked(q, k, v, head_chunk: int, causal: bool = True):
    """Forward that walks query-head chunks through one reused buffer set."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, Hkv, D = _dims(q, k)
    S = q.shape[0]
    o = np.empty((S, Hq, D))
    lse = np.empty((Hq, S))
    _check(_load().orc_attn_fwd_chunked(_p(q), _p(k), _p(v), S, Hq, Hkv, D, int(causal),
                                        int(head_chunk), _p(o), _p(lse)), "orc_attn_fwd_chunked")
    return o, lse


def attn_bwd(q, k, v, dout, causal: bool = True):
    """Exact backward of L = sum(O * dout): dict with dq, dk, dv, lse, delta."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    Hq, Hkv, D = _dims(q, k)
    S = q.shape[0]
    out = {"dq": np.empty((S, Hq, D)), "dk": np.empty((S, Hkv, D)), "dv": np.empty((S, Hkv, D)),
           "lse": np.empty((Hq, S)), "delta": np.empty((Hq, S))}
    _check(_load().orc_attn_bwd(_p(q), _p(k), _p(v), _p(dout), S, Hq, Hkv, D, int(causal),
                                _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["lse"]),
                                _p(out["delta"])), "orc_attn_bwd")
    return out


def attn_dq_rows(q_rows, dout_rows, rows, k, v, causal: bool = True):
    """dQ for chosen rows: (dq [n,Hq,D], delta [Hq,n])."""
    q_rows, dout_rows, k, v, rows = _f64(q_rows), _f64(dout_rows), _f64(k), _f64(v), _rows(rows)
    Hq, Hkv, D = _dims(q_rows, k)
    S, n = k.shape[0], rows.shape[0]
    dq = np.empty((n, Hq, D))
    delta = np.empty((Hq, n))
    _check(_load().orc_attn_dq_rows(_p(q_rows), _p(dout_rows), rows.ctypes.data_as(_lp), n,
                                    _p(k), _p(v), S, Hq, Hkv, D, int(causal), _p(dq), _p(delta)),
           "orc_attn_dq_rows")
    return dq, delta


def attn_dkdv_cols(q_tail, dout_tail, i0: int, k, v, cols, causal: bool = True):
    """dK, dV for chosen keys.  ``q_tail``/``dout_tail`` hold query rows
    [i0, S) (all rows that see the keys).  Returns (dk [n,Hkv,D], dv [n,Hkv,D])."""
    q_tail, dout_tail, k, v, cols = _f64(q_tail), _f64(dout_tail), _f64(k), _f64(v), _rows(cols)
    Hq, Hkv, D = _dims(q_tail, k)
    S, n = k.shape[0], cols.shape[0]
    dk = np.empty((n, Hkv, D))
    dv = np.empty((n, Hkv, D))
    _check(_load().orc_attn_dkdv_cols(_p(q_tail), _p(dout_tail), int(i0), _p(k), _p(v), S, Hq,
                                      Hkv, D, int(causal), cols.ctypes.data_as(_lp), n, _p(dk),
                                      _p(dv)), "orc_attn_dkdv_cols")
    return dk, dv


# ------------------------------------------------------------ attention layer
#
# x [S, dm]; wq [Hq*D, dm]; wk, wv [Hkv*D, dm]; wo [dm, Hq*D] (weights in the
# [out][in] convention, y = x W^T); no bias, no rotary embedding, batch 1.


def _layer_dims(x, wq, wk, wo, Hq, Hkv, D):
    if x.ndim != 2 or wq.shape != (Hq * D, x.shape[1]) or wk.shape != (Hkv * D, x.shape[1]) \
            or wo.shape != (x.shape[1], Hq * D):
        raise ValueError("layer shapes: x [S,dm], wq [Hq*D,dm], wk/wv [Hkv*D,dm], wo [dm,Hq*D]")
    return x.shape[0], x.shape[1]


def layer_fwd(x, wq, wk, wv, wo, Hq: int, Hkv: int, D: int, causal: bool = True):
    """y = attention(x Wq^T, x Wk^T, x Wv^T) Wo^T: returns (y [S,dm], lse [Hq,S])."""
    x, wq, wk, wv, wo = (_f64(t) for t in (x, wq, wk, wv, wo))
    S, dm = _layer_dims(x, wq, wk, wo, Hq, Hkv, D)
    y = np.empty((S, dm))
    lse = np.empty((Hq, S))
    _check(_load().orc_layer_fwd(_p(x), _p(wq), _p(wk), _p(wv), _p(wo), S, dm, Hq, Hkv, D,
                                 int(causal), _p(y), _p(lse)), "orc_layer_fwd")
    return y, lse


def layer_fwd_chunked(x, wq, wk, wv, wo, Hq: int, Hkv: int, D: int, head_chunk: int,
                      causal: bool = True):
    """The layer walked head chunk by head chunk (projections of the chunk's
    heads, attention, the chunk's share of the output projection)."""
    x, wq, wk, wv, wo = (_f64(t) for t in (x, wq, wk, wv, wo))
    S, dm = _layer_dims(x, wq, wk, wo, Hq, Hkv, D)
    y = np.empty((S, dm))
    _check(_load().orc_layer_fwd_chunked(_p(x), _p(wq), _p(wk), _p(wv), _p(wo), S, dm, Hq, Hkv,
                                         D, int(causal), int(head_chunk), _p(y)),
           "orc_layer_fwd_chunked")
    return y


def layer_bwd(x, wq, wk, wv, wo, dy, Hq: int, Hkv: int, D: int, causal: bool = True):
    """Gradients of sum(y * dy): dict with dx, dwq, dwk, dwv, dwo."""
    x, wq, wk, wv, wo, dy = (_f64(t) for t in (x, wq, wk, wv, wo, dy))
    S, dm = _layer_dims(x, wq, wk, wo, Hq, Hkv, D)
    out = {"dx": np.empty((S, dm)), "dwq": np.empty(wq.shape), "dwk": np.empty(wk.shape),
           "dwv": np.empty(wv.shape), "dwo": np.empty(wo.shape)}
    _check(_load().orc_layer_bwd(_p(x), _p(wq), _p(wk), _p(wv), _p(wo), _p(dy), S, dm, Hq, Hkv,
                                 D, int(causal), _p(out["dx"]), _p(out["dwq"]), _p(out["dwk"]),
                                 _p(out["dwv"]), _p(out["dwo"])), "orc_layer_bwd")
    return out


def layer_fwd_rows(x, wq, wk, wv, wo, rows, Hq: int, Hkv: int, D: int, causal: bool = True):
    """The layer's output at chosen rows: (y [n, dm], lse [Hq, n]); x, the
    weights and the whole sequence as for layer_fwd."""
    x, wq, wk, wv, wo = (_f64(t) for t in (x, wq, wk, wv, wo))
    rows = _rows(rows)
    S, dm = _layer_dims(x, wq, wk, wo, Hq, Hkv, D)
    n = rows.shape[0]
    y = np.empty((n, dm))
    lse = np.empty((Hq, n))
    _check(_load().orc_layer_fwd_rows(_p(x), _p(wq), _p(wk), _p(wv), _p(wo), S, dm, Hq, Hkv, D,
                                      int(causal), rows.ctypes.data_as(_lp), n, _p(y), _p(lse)),
           "orc_layer_fwd_rows")
    return y, lse
