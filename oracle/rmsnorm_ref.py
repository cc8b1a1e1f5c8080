"""CPU oracle: RMS normalization with an MXFP8 output (test infrastructure, never product code).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the GPU library and imports nothing from it.

What it computes (vLLM PR #57977 "[Perf][DSv4.1] Keep activations MXFP8 between
DeepGEMM kernels", the before/after diagrams and Pieces): the normalizing
producer at the top of the attention sublayer hands the fused wqa/wkv GEMM its
input as MXFP8 (codes + packed UE8M0 scales) together with its BF16 output,
instead of a standalone quantize launch in between.

The pages name the producer's normalization (RMSNorm) but give neither its
formula nor its precision.  Readings taken here:
  * y = x / sqrt(mean(x^2) + eps) * gamma per row, mean over the row's K values,
    eps > 0 added to the mean square (the usual RMS normalization);
  * the producer's BF16 output is y rounded once to BF16 (nearest even), and its
    MXFP8 output is the quantization of that BF16 y -- the same reading as the
    einsum epilogue (PR #60118: the fused bytes equal what the consumer's own
    quantizer makes of the BF16 tensor);
  * here every step is float64; the GPU computes in fp32, so its BF16 y is
    compared within one BF16 step, and its MXFP8 output bit for bit against the
    quantization of its own BF16 y.
"""
from __future__ import annotations

import numpy as np

from . import mxfp8_ref as mx


def rmsnorm(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    """float64 y [M, K] = x / sqrt(mean(x^2) + eps) * gamma for BF16 bits x [M, K] and gamma [K]."""
    x = mx.bf16_decode(np.asarray(x_bits, dtype=np.uint16))
    g = mx.bf16_decode(np.asarray(gamma_bits, dtype=np.uint16))
    if x.ndim != 2 or g.shape != (x.shape[1],):
        raise ValueError("rmsnorm: x must be [M, K] and gamma [K]")
    if not eps >= 0.0:
        raise ValueError("rmsnorm: eps must be non-negative")
    ms = np.mean(x * x, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = 1.0 / np.sqrt(ms + eps)
    return x * r * g


def rmsnorm_quantize(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float):
    """(y_bits BF16 [M, K], codes uint8 [M, K], packed scales int32 [M, K/128]): the BF16 y, then its MXFP8."""
    y_bits = mx.bf16_round(rmsnorm(x_bits, gamma_bits, eps))
    q, sf = mx.quantize(y_bits)
    return y_bits, q, sf
