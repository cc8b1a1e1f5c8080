"""Seeded synthetic inputs for the MXFP8 o_proj chain and the standalone quantize sweep.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds none of the quantization or GEMM arithmetic: it draws
float32 Gaussians from numpy's PCG64, applies the outlier pattern, and rounds
to BF16 with torch's CPU cast (round-to-nearest-even).  Everything it returns is
a raw BF16 bit pattern in a ``uint16`` numpy array, so the GPU path and the
oracle consume identical bytes.

Shapes follow the DeepSeek-V4.1-Flash TP1 o_proj that vLLM PR #60118
("[Perf][DSv4.1] MegaAttn: wo_a writes wo_b's MXFP8 input", section
Validation) measures: 8 groups x 4096 -> 1024 for wo_a, then 8192 -> 5120 for
wo_b.  The quantize sweep uses a hidden size of 7168, the input of the fused
wqa/wkv projection in vLLM PR #57977 ("[Perf][DSv4.1] Keep activations MXFP8
between DeepGEMM kernels", section Purpose).

Recipe (all draws float32, then one RNE rounding to BF16):
  * ``SeedSequence(seed).spawn(4)`` gives independent streams for x, the
    outlier positions, wo_a and wo_b.
  * Matrices are drawn in blocks of ``ROW_BLOCK`` rows; block i uses the i-th
    child of its stream, so rows are a prefix-stable function of the seed and
    blocks can be drawn in parallel threads.
  * x ~ N(0, 1).  With ``outlier_rate`` r > 0, exactly round(r * numel)
    positions, drawn without replacement, are multiplied by 100 before the
    BF16 rounding.
  * wo_a, wo_b ~ N(0, 0.02) in BF16; they become MXFP8 by the quantizer under
    test (GPU) or the oracle's quantizer (CPU), never here.
  * Quantize sweep rows ~ N(0, 1); for M >= 7, n = max(1, round(0.01 M)) rows
    are scaled by 1e3 and n other rows are all zero (rows drawn without
    replacement).  The same rows feed the RMS-normalizing producer, whose
    weight gamma ~ N(1, 0.1) in BF16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROW_BLOCK = 1024
SEED_BASE = 20260000


@dataclass(frozen=True)
class ChainShape:
    """o_proj chain sizes: x [M, G*K], wo_a [G, N, K], z [M, G*N], wo_b [P, G*N], out [M, P]."""

    M: int
    G: int
    K: int
    N: int
    P: int

    @property
    def flop(self) -> int:
        return 2 * self.M * (self.G * self.K * self.N + self.G * self.N * self.P)


@dataclass(frozen=True)
class ChainConfig:
    name: str
    shape: ChainShape
    seed: int
    outlier_rate: float


CHAIN_CONFIGS = {
    "tiny": ChainConfig("tiny", ChainShape(4, 2, 256, 128, 256), SEED_BASE + 1, 0.0),
    "decode": ChainConfig("decode", ChainShape(64, 8, 4096, 1024, 5120), SEED_BASE + 2, 0.001),
    "prefill": ChainConfig("prefill", ChainShape(4096, 8, 4096, 1024, 5120), SEED_BASE + 3, 0.001),
    "long": ChainConfig("long", ChainShape(32768, 8, 4096, 1024, 5120), SEED_BASE + 4, 0.001),
}

QUANT_SWEEP_K = 7168
QUANT_SWEEP_M = (1, 7, 64, 300, 8192)
QUANT_SWEEP_SEED = SEED_BASE + 5


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (torch CPU cast, RNE) and return the bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal_rows(seq: np.random.SeedSequence, rows: int, cols: int, std: float) -> np.ndarray:
    """float32 [rows, cols] of N(0, std^2), drawn per ROW_BLOCK-row block from child streams."""
    nblk = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    children = seq.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(i: int) -> None:
        r0 = i * ROW_BLOCK
        r1 = min(rows, r0 + ROW_BLOCK)
        g = np.random.Generator(np.random.PCG64(children[i]))
        blk = g.standard_normal((r1 - r0) * cols, dtype=np.float32).reshape(r1 - r0, cols)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r1] = blk

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def chain_inputs(shape: ChainShape, seed: int, outlier_rate: float = 0.0,
                 with_weights: bool = True) -> dict:
    """BF16 bit patterns for x [M, G*K], wo_a [G, N, K] and wo_b [P, G*N]."""
    M, G, K, N, P = shape.M, shape.G, shape.K, shape.N, shape.P
    sx, so, sa, sb = np.random.SeedSequence(seed).spawn(4)
    x = _normal_rows(sx, M, G * K, 1.0)
    if outlier_rate > 0.0 and M > 0:
        numel = x.size
        n_out = int(round(outlier_rate * numel))
        if n_out > 0:
            pos = np.random.Generator(np.random.PCG64(so)).choice(numel, size=n_out, replace=False)
            flat = x.reshape(-1)
            flat[pos] *= np.float32(100.0)
    res = {"x": bf16_bits(x)}
    del x
    if with_weights:
        res["wo_a"] = bf16_bits(_normal_rows(sa, G * N, K, 0.02)).reshape(G, N, K)
        res["wo_b"] = bf16_bits(_normal_rows(sb, P, G * N, 0.02))
    return res


def config_inputs(name: str, with_weights: bool = True) -> dict:
    cfg = CHAIN_CONFIGS[name]
    return chain_inputs(cfg.shape, cfg.seed, cfg.outlier_rate, with_weights)


RMSNORM_GAMMA_SEED = SEED_BASE + 6


def rmsnorm_gamma(K: int = QUANT_SWEEP_K, seed: int = RMSNORM_GAMMA_SEED) -> np.ndarray:
    """BF16 bits [K] of an RMS-normalization weight: N(1, 0.1) (the weight is not on the pages; a weight
    near one with a spread of ten percent stands in for a trained one)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed))).standard_normal(K, dtype=np.float32)
    return bf16_bits((np.float32(1.0) + np.float32(0.1) * g).reshape(1, K))[0]


def quant_sweep_input(M: int, K: int = QUANT_SWEEP_K, seed: int = QUANT_SWEEP_SEED) -> np.ndarray:
    """BF16 bits [M, K]: N(0,1) rows, plus (M >= 7) n rows x1e3 and n all-zero rows."""
    sx, sr = np.random.SeedSequence([seed, M]).spawn(2)
    x = _normal_rows(sx, M, K, 1.0)
    if M >= 7:
        n = max(1, int(round(0.01 * M)))
        rows = np.random.Generator(np.random.PCG64(sr)).choice(M, size=2 * n, replace=False)
        x[rows[:n]] *= np.float32(1e3)
        x[rows[n:]] = 0.0
    return bf16_bits(x)
