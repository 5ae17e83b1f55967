"""Seeded synthetic inputs for the SharQ hot path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no norm, no mask, no quantization).  Both the CPU
oracle and the HIP path are fed from here, so the same bytes reach both.

SharQ is evaluated on Llama-3.1-8B, Qwen2.5-7B and Qwen3-30B-A3B (SharQ:
Bridging Activation Sparsity and FP4 Quantization for LLM Inference,
Abstract).  No weights or activations of those models are available, so
seeded tensors with their layer shapes stand in: Gaussian (or Student-t)
activations with a few outlier channels -- the case the abstract describes,
where a handful of large values set the FP4 block scales -- and N(0, 0.02)
weights.

Every array is returned as raw 16-bit patterns (numpy uint16) plus a dtype
tag ("bf16" or "f16"), because numpy has no bfloat16.  Values are drawn in
float32 and rounded to the 16-bit type with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

NORM_NONE, NORM_RMS, NORM_LAYER = 0, 1, 2
FMT_MXFP4, FMT_NVFP4 = 0, 1


@dataclasses.dataclass(frozen=True)
class Linear:
    """One linear layer of a workload: Y[T][nout] = prep(X[T][k]) . W[nout][k]^T.

    swiglu_of names the linear whose float32 output [gate | up] feeds this
    one's preparation as SiLU(gate) * up (the down projection of a SwiGLU
    MLP); its input is then not drawn at random in a layer step."""
    name: str
    k: int
    nout: int
    norm: int
    lin_id: int
    swiglu_of: Optional[str] = None


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    dtype: str            # activation / weight storage type: "bf16" or "f16"
    tokens: int
    linears: tuple
    fmt: int
    n: int
    m: int
    eps: float
    act_dist: str         # "normal" or "student_t3_half"
    outlier_frac: float   # fraction of channels that are outliers
    outlier_count: Optional[int]  # fixed count (overrides the fraction)
    outlier_mult: float
    experts: int = 1
    topk: int = 0
    description: str = ""


# A decoder layer's four linears in execution order: qkv (after the input
# RMSNorm), o_proj (attention output, no norm), gate_up (after the
# post-attention RMSNorm) and down (SiLU(gate) * up of gate_up's output, no
# norm).  lin_id fixes each tensor's random stream.
LLAMA_LINEARS = (
    Linear("qkv", 4096, 6144, NORM_RMS, 0),
    Linear("o_proj", 4096, 4096, NORM_NONE, 3),
    Linear("gate_up", 4096, 28672, NORM_RMS, 1),
    Linear("down", 14336, 4096, NORM_NONE, 2, swiglu_of="gate_up"),
)

WORKLOADS: Dict[int, Workload] = {
    0: Workload(0, "single_linear_fp16_256", "f16", 16,
                (Linear("lin", 256, 256, NORM_RMS, 0),),
                FMT_MXFP4, 2, 4, 1e-5, "normal", 0.0, 4, 30.0,
                description="X fp16 [16,256], 4 outlier channels x30, RMSNorm, "
                            "W fp16 [256,256], MXFP4 2:4"),
    1: Workload(1, "llama3.1-8b_prefill_T2048_mxfp4", "bf16", 2048, LLAMA_LINEARS,
                FMT_MXFP4, 2, 4, 1e-5, "normal", 0.005, None, 50.0,
                description="Llama-3.1-8B-shaped prefill layer, 2048 tokens, "
                            "qkv/o_proj/gate_up/down (down prepared from SiLU(gate)*up), MXFP4 2:4"),
    2: Workload(2, "llama3.1-8b_decode_mxfp4", "bf16", 1, LLAMA_LINEARS,
                FMT_MXFP4, 2, 4, 1e-5, "normal", 0.005, None, 50.0,
                description="Llama-3.1-8B-shaped decode layer at 1, 8 and 64 tokens"),
    3: Workload(3, "qwen2.5-7b_prefill_T4096_nvfp4", "bf16", 4096,
                (Linear("qkv", 3584, 4608, NORM_RMS, 0),
                 Linear("o_proj", 3584, 3584, NORM_NONE, 3),
                 Linear("gate_up", 3584, 37888, NORM_RMS, 1),
                 Linear("down", 18944, 3584, NORM_NONE, 2, swiglu_of="gate_up")),
                FMT_NVFP4, 2, 4, 1e-6, "student_t3_half", 0.01, None, 40.0,
                description="Qwen2.5-7B-shaped prefill layer, 4096 tokens, NVFP4 2:4"),
    4: Workload(4, "qwen3-30b-a3b_moe_T4096_mxfp4", "bf16", 4096,
                (Linear("expert_gate_up", 2048, 1536, NORM_RMS, 0),
                 Linear("expert_down", 768, 2048, NORM_NONE, 1, swiglu_of="expert_gate_up")),
                FMT_MXFP4, 2, 4, 1e-6, "normal", 0.005, None, 50.0,
                experts=128, topk=8,
                description="Qwen3-30B-A3B-shaped MoE expert FFN, 4096 tokens, "
                            "128 experts, top-8, MXFP4 2:4"),
}

DECODE_TOKENS = (1, 8, 64)


def _rng(seed: int, cid: int, tensor_id: int, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tensor_id, extra])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    raise ValueError(dtype)


def bits_to_f32(b: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of 16-bit patterns to float32 (both types embed exactly)."""
    if dtype == "bf16":
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    raise ValueError(dtype)


def outlier_channels(w: Workload, k: int, lin_id: int, seed: int = 0) -> np.ndarray:
    n = w.outlier_count if w.outlier_count is not None else int(round(w.outlier_frac * k))
    rng = _rng(seed, w.cid, 10 * lin_id + 3, k)
    return np.sort(rng.choice(k, size=n, replace=False))


def activation_f32(w: Workload, lin: Linear, tokens: int, seed: int = 0) -> np.ndarray:
    """Float32 activation [tokens][k] before rounding to the storage type."""
    rng = _rng(seed, w.cid, 10 * lin.lin_id + 0, tokens)
    if w.act_dist == "normal":
        x = rng.standard_normal((tokens, lin.k), dtype=np.float32)
    elif w.act_dist == "student_t3_half":
        x = (0.5 * rng.standard_t(3.0, size=(tokens, lin.k))).astype(np.float32)
    else:
        raise ValueError(w.act_dist)
    ch = outlier_channels(w, lin.k, lin.lin_id, seed)
    x[:, ch] *= np.float32(w.outlier_mult)
    return x


def activation(w: Workload, lin: Linear, tokens: Optional[int] = None, seed: int = 0) -> np.ndarray:
    t = w.tokens if tokens is None else tokens
    return to_bits(activation_f32(w, lin, t, seed), w.dtype)


def gamma(w: Workload, lin: Linear, seed: int = 0) -> np.ndarray:
    rng = _rng(seed, w.cid, 10 * lin.lin_id + 1)
    g = (1.0 + 0.1 * rng.standard_normal(lin.k, dtype=np.float32)).astype(np.float32)
    return to_bits(g, w.dtype)


def weight_f32(w: Workload, lin: Linear, seed: int = 0) -> np.ndarray:
    """Float32 weight [experts][nout][k] (experts == 1 for dense layers)."""
    rng = _rng(seed, w.cid, 10 * lin.lin_id + 2)
    return (0.02 * rng.standard_normal((w.experts, lin.nout, lin.k), dtype=np.float32)).astype(np.float32)


def weight(w: Workload, lin: Linear, seed: int = 0) -> np.ndarray:
    return to_bits(weight_f32(w, lin, seed), w.dtype)


@dataclasses.dataclass
class Routing:
    """Top-k routing of tokens to experts, sorted by (expert, token)."""
    offsets: np.ndarray     # int32 [experts + 1]
    row_index: np.ndarray   # int32 [tokens * topk]: token of each sorted row
    expert_of_row: np.ndarray


def moe_routing(w: Workload, seed: int = 0) -> Routing:
    """Seeded softmax routing over N(0,1) logits; top-k with ties to the lower expert id.

    Softmax is monotone, so the top-k of the logits equals the top-k of the
    routing probabilities; the probabilities themselves only weight the
    combine step, which lies outside the linear layer and is not produced.
    """
    rng = _rng(seed, w.cid, 100)
    logits = rng.standard_normal((w.tokens, w.experts), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, : w.topk]
    tok = np.repeat(np.arange(w.tokens, dtype=np.int64), w.topk)
    exp = order.reshape(-1).astype(np.int64)
    key = exp * w.tokens + tok
    perm = np.argsort(key, kind="stable")
    exp_sorted = exp[perm]
    tok_sorted = tok[perm]
    counts = np.bincount(exp_sorted, minlength=w.experts)
    offsets = np.zeros(w.experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return Routing(offsets, tok_sorted.astype(np.int32), exp_sorted.astype(np.int32))


def small_case(k: int, tokens: int, dtype: str = "bf16", seed: int = 0, outliers: int = 4,
               mult: float = 30.0, dist: str = "normal", tag: int = 0) -> np.ndarray:
    """A small seeded activation for parity sweeps (ragged shapes, edge cases)."""
    rng = _rng(seed, 1000 + tag, k, tokens)
    if dist == "normal":
        x = rng.standard_normal((tokens, k), dtype=np.float32)
    else:
        x = (0.5 * rng.standard_t(3.0, size=(tokens, k))).astype(np.float32)
    if outliers:
        ch = rng.choice(k, size=min(outliers, k), replace=False)
        x[:, ch] *= np.float32(mult)
    return to_bits(x, dtype)


def small_gamma(k: int, dtype: str = "bf16", seed: int = 0, tag: int = 0) -> np.ndarray:
    rng = _rng(seed, 2000 + tag, k)
    return to_bits(1.0 + 0.1 * rng.standard_normal(k, dtype=np.float32), dtype)


def small_weight(nout: int, k: int, experts: int = 1, dtype: str = "bf16", seed: int = 0,
                 tag: int = 0) -> np.ndarray:
    rng = _rng(seed, 3000 + tag, nout, k)
    return to_bits(0.02 * rng.standard_normal((experts, nout, k), dtype=np.float32), dtype)


def uniform_bits_f32(n: int, seed: int = 0) -> np.ndarray:
    """Random float32 bit patterns (finite only), for conversion sweeps."""
    rng = _rng(seed, 4000, n)
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    exp = (u >> np.uint32(23)) & np.uint32(0xFF)
    u = np.where(exp == 0xFF, u & np.uint32(0x807FFFFF), u)
    return u.view(np.float32)


def small_gate_up(k: int, tokens: int, ld: Optional[int] = None, seed: int = 0, outliers: int = 4,
                  mult: float = 20.0, tag: int = 0) -> np.ndarray:
    """Float32 rows [gate (k) | up (k) | padding] shaped like a gate/up
    product's output: N(0, 3^2) gates, N(0, 1) ups, a few up channels scaled
    up as outliers."""
    ld = 2 * k if ld is None else ld
    rng = _rng(seed, 5000 + tag, k, tokens)
    gu = rng.standard_normal((tokens, ld), dtype=np.float32)
    gu[:, :k] *= np.float32(3.0)
    if outliers:
        ch = rng.choice(k, size=min(outliers, k), replace=False)
        gu[:, k + ch] *= np.float32(mult)
    return gu
