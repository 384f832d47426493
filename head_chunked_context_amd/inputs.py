"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module only draws random numbers; it holds none of the attention
arithmetic.  Every tensor is i.i.d. N(0, 1), drawn in fp32 from a seeded
``torch.Generator`` and then rounded to the requested dtype (bf16 by default,
round-to-nearest-even).  The seed of tensor ``t`` in workload ``w`` is
``1000 * w + t`` with t = 0 for Q, 1 for K, 2 for V, 3 for dO.

The pages' workloads are long-context Llama3-8B / 32B / 7B training runs on
unnamed data; no dataset or trained weight is involved here.  Gaussian tensors
at the same attention shapes stand in for them: scores are then ~N(0, 1), a
high-entropy softmax with no data-dependent sparsity.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dout": 3}


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes plus the head-chunk / trunk settings."""
    wid: int
    name: str
    S: int
    Hq: int
    Hkv: int
    D: int
    head_chunks: tuple
    kv_trunk: int = 0
    kv_on_host: bool = False


# The five attention shapes measured and tested here.
WORKLOADS = {
    1: Workload(1, "tiny exactness case S=256 Hq=4 Hkv=2 D=64", 256, 4, 2, 64, (1, 2, 4)),
    2: Workload(2, "Llama3-8B attention layer S=32768 Hq=32 Hkv=8 D=128", 32768, 32, 8, 128,
                (4, 32)),
    3: Workload(3, "Llama3-8B heads at S=262144 Hq=32 Hkv=8 D=128", 262144, 32, 8, 128,
                (1, 2, 4, 8, 32)),
    4: Workload(4, "32B-class S=524288 Hq=40 Hkv=8 D=128, 65536-token K/V trunks in pinned host",
                524288, 40, 8, 128, (5,), kv_trunk=65536, kv_on_host=True),
    5: Workload(5, "one GPU's 1/8 head share of Llama3-8B at S=5242880 Hq=4 Hkv=1 D=128",
                5242880, 4, 1, 128, (1,), kv_trunk=262144),
}


def gaussian(shape, seed: int, device="cpu", dtype=torch.bfloat16, scale: float = 1.0):
    """N(0, scale^2) tensor drawn in fp32 from a generator seeded with ``seed``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def attention_inputs(S: int, Hq: int, Hkv: int, D: int, seed_base: int, device="cpu",
                     dtype=torch.bfloat16, q_scale: float = 1.0, with_dout: bool = True):
    """Q [S,Hq,D], K/V [S,Hkv,D] (and dO [S,Hq,D]) with seeds seed_base*1000 + id."""
    out = {
        "q": gaussian((S, Hq, D), 1000 * seed_base + TENSOR_IDS["q"], device, dtype, q_scale),
        "k": gaussian((S, Hkv, D), 1000 * seed_base + TENSOR_IDS["k"], device, dtype),
        "v": gaussian((S, Hkv, D), 1000 * seed_base + TENSOR_IDS["v"], device, dtype),
    }
    if with_dout:
        out["dout"] = gaussian((S, Hq, D), 1000 * seed_base + TENSOR_IDS["dout"], device, dtype)
    return out


LAYER_TENSOR_IDS = {"x": 4, "wq": 5, "wk": 6, "wv": 7, "wo": 8, "dy": 9}


def layer_inputs(S: int, d_model: int, Hq: int, Hkv: int, D: int, seed_base: int, device="cpu",
                 dtype=torch.bfloat16, with_dy: bool = True):
    """Synthetic inputs of the attention layer around the attention (no trained
    weights exist here): x [S, d_model] ~ N(0, 1); weights in the [out][in]
    convention, wq [Hq*D, d_model], wk / wv [Hkv*D, d_model] ~ N(0, 1/d_model)
    and wo [d_model, Hq*D] ~ N(0, 1/(Hq*D)) (fan-in scaling, so the
    projected q, k, v are ~N(0, 1) like the attention workloads); dy ~ N(0, 1).
    Seeds 1000 * seed_base + {x: 4, wq: 5, wk: 6, wv: 7, wo: 8, dy: 9}."""
    sd = lambda n: 1000 * seed_base + LAYER_TENSOR_IDS[n]
    out = {
        "x": gaussian((S, d_model), sd("x"), device, dtype),
        "wq": gaussian((Hq * D, d_model), sd("wq"), device, dtype, d_model ** -0.5),
        "wk": gaussian((Hkv * D, d_model), sd("wk"), device, dtype, d_model ** -0.5),
        "wv": gaussian((Hkv * D, d_model), sd("wv"), device, dtype, d_model ** -0.5),
        "wo": gaussian((d_model, Hq * D), sd("wo"), device, dtype, (Hq * D) ** -0.5),
    }
    if with_dy:
        out["dy"] = gaussian((S, d_model), sd("dy"), device, dtype)
    return out
