"""Algorithmic work of the decode step and roofline arithmetic.

Measurement only (host arithmetic, no part of the decode path).  The
formulas follow the pages' cost models:

* page "gpu-waiting-not-working" (nanoserve notes), section "The number that
  didn't fit": the step's memory floor is the weight bytes divided by the
  copy bandwidth; throughput is batch / step time (section "The tell:
  batching was almost free");
* page "The roofline flips: why optimising small models is a different
  performance game": arithmetic intensity = FLOPs / bytes, attainable rate =
  min(peak, bandwidth x intensity), ridge = peak / bandwidth; decode weight
  GEMMs do about 2B FLOP per weight byte at batch B;
* page "NanoFlow: LLM Serving Is Compute Bound, and Your GPU Is Half Idle",
  introduction: the compute-bound ceiling peak_flops / (2 n_params) tokens/s;
* page "The chef who calls out every order: SMs, CUDA streams and CUDA
  graphs", launch maths: launches x per-launch cost vs bytes / bandwidth.

Algorithmic bytes count each weight once per launch and each cached K/V byte
once (nano-op weight reloads are overhead, not algorithmic work).
"""
from __future__ import annotations

from typing import Iterable

# MI355X published peaks (dense; no structured sparsity).
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_VECTOR_PEAK_TFLOPS = 157.3


def elem_bytes(shape) -> int:
    return 2 if shape.dtype == "bf16" else 4


def layer_params(shape) -> int:
    H, F = shape.hidden, shape.ffn
    return shape.qkv_dim * H + H * shape.n_q_heads * shape.head_dim + 3 * H * F + 2 * H


def params(shape, qkv_bias: bool = False) -> int:
    """Parameter count; the LM head counts once when tied to the embedding."""
    p = shape.n_layers * layer_params(shape)
    if qkv_bias:
        p += shape.n_layers * shape.qkv_dim
    if shape.vocab:
        p += shape.hidden + shape.vocab * shape.hidden * (1 if shape.tied else 2)
    return p


def weight_bytes(shape, qkv_bias: bool = False) -> int:
    return params(shape, qkv_bias) * elem_bytes(shape)


def streamed_weight_bytes(shape) -> int:
    """Weight bytes a decode step reads: every layer, the final norm and the
    LM head (the embedding is gathered row by row, not streamed)."""
    b = shape.n_layers * layer_params(shape)
    if shape.vocab:
        b += shape.hidden + shape.vocab * shape.hidden
    return b * elem_bytes(shape)


def kv_bytes_per_position(shape) -> int:
    """K and V of one cached position in one layer."""
    return 2 * shape.n_kv_heads * shape.head_dim * elem_bytes(shape)


def attention_bytes(shape, ctx: Iterable[int]) -> int:
    """Cache bytes one attention launch reads for rows with these context
    lengths (each K/V byte once), plus q in and o out."""
    ctx = list(ctx)
    per_row_qo = 2 * shape.n_q_heads * shape.head_dim * elem_bytes(shape)
    return sum(ctx) * kv_bytes_per_position(shape) + len(ctx) * per_row_qo


def attention_flops(shape, ctx: Iterable[int]) -> int:
    return 4 * sum(ctx) * shape.n_q_heads * shape.head_dim


def step_bytes(shape, ctx: Iterable[int]) -> int:
    """Algorithmic HBM bytes of one decode step: streamed weights once plus
    every layer's cache read."""
    return streamed_weight_bytes(shape) + shape.n_layers * sum(ctx) * kv_bytes_per_position(shape)


def gemm_flops(M: int, N: int, K: int, swiglu: bool = False) -> int:
    return 2 * M * (2 * N if swiglu else N) * K


def gemm_bytes(M: int, N: int, K: int, elem: int, epilogue: str) -> int:
    """A [M, K] and B [N, K] (B [2N, K] for SwiGLU) read once; the output
    written once (fp32, or dtype for SwiGLU); a residual add also reads C."""
    nb = 2 * N if epilogue == "silu" else N
    b = (M * K + nb * K) * elem
    if epilogue == "silu":
        b += M * N * elem
    elif epilogue == "resid":
        b += 2 * M * N * 4
    else:
        b += M * N * 4
    return b


def floor_seconds(nbytes: float, gbs: float = HBM_PEAK_GBS) -> float:
    return nbytes / (gbs * 1e9)


def tokens_per_second(batch: int, step_seconds: float) -> float:
    return batch / step_seconds


def ridge(peak_tflops: float, gbs: float) -> float:
    """FLOP per byte where the roofline's slope meets its flat top."""
    return peak_tflops * 1e12 / (gbs * 1e9)


def attainable_tflops(ai: float, peak_tflops: float, gbs: float) -> float:
    return min(peak_tflops, gbs * 1e9 * ai / 1e12)


def compute_bound_tokens(peak_flops: float, n_params: float) -> float:
    """peak FLOP/s / (2 FLOP per parameter per token)."""
    return peak_flops / (2.0 * n_params)


def launch_seconds(n_launches: int, per_launch_s: float) -> float:
    return n_launches * per_launch_s
