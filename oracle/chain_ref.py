"""CPU oracle: the MXFP8 o_proj chain in float64 (test infrastructure, never product code).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the GPU library.

The chain (vLLM PR #60118 "[Perf][DSv4.1] MegaAttn: wo_a writes wo_b's MXFP8
input", sections Conversation, Overview and Claims; vLLM PR #57977
"[Perf][DSv4.1] Keep activations MXFP8 between DeepGEMM kernels", the
before/after diagrams and Pieces):

  x (BF16 [M, G*K]) --MXFP8 quantize--> (x_q, x_sf)
    --grouped FP8 einsum with wo_a [G, N, K]--> z (written as MXFP8 (z_q, z_sf))
    --FP8 GEMM "NT" with wo_b [P, G*N], 1x32 scale blocks on both operands--> out (BF16 [M, P])

Readings of the pages (plain text, where they are silent or garbled):
  * einsum index map for "8 groups x 4096 -> 1024":
        z[m, g*N + n] = sum_k x[m, g*K + k] * wo_a[g, n, k]
  * the fused producer must hand the consumer the same bytes the consumer's own
    quantizer makes from the BF16 z (PR #60118, Claims and Tests), so z is
    rounded to BF16 (round-to-nearest-even) first and the BF16 z is quantized;
  * both GEMMs are defined exactly: dequantize every operand (code times its
    power-of-two block scale) and sum in float64 (a library matmul serves as the
    summation step).  The GPU accumulates in fp32, so the final output is
    compared against the float64 value within a tolerance, not bit for bit.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import mxfp8_ref as mx


def grouped_einsum(x_q, x_sf, w_q, w_sf, G: int, K: int, N: int) -> np.ndarray:
    """float64 z [M, G*N] with z[m, g*N+n] = sum_k dq(x)[m, g*K+k] * dq(wo_a)[g, n, k].

    x_q [M, G*K] uint8 + x_sf [M, G*K/128] int32; w_q [G, N, K] uint8 + w_sf [G, N, K/128] int32.
    """
    x = mx.dequantize(x_q, x_sf)                                   # [M, G*K]
    M = x.shape[0]
    w = mx.dequantize(np.asarray(w_q).reshape(G * N, K),
                      np.asarray(w_sf).reshape(G * N, K // mx.WORD_SPAN)).reshape(G, N, K)
    z = np.empty((M, G * N), dtype=np.float64)
    for g in range(G):
        z[:, g * N:(g + 1) * N] = x[:, g * K:(g + 1) * K] @ w[g].T
    return z


def gemm_nt(a_q, a_sf, b_q, b_sf) -> np.ndarray:
    """float64 out [M, P] = dq(A) [M, Kt] @ dq(B)^T, B [P, Kt]; both K-contiguous with 1x32 scale blocks."""
    a = mx.dequantize(a_q, a_sf)
    b = mx.dequantize(b_q, b_sf)
    return a @ b.T


@dataclass
class ChainResult:
    x_q: np.ndarray
    x_sf: np.ndarray
    z64: np.ndarray        # float64 einsum output
    z_bf16: np.ndarray     # BF16 bits of z (RNE)
    z_q: np.ndarray        # MXFP8 codes of z_bf16
    z_sf: np.ndarray       # packed scales of z_bf16
    out64: np.ndarray      # float64 wo_b output
    out_bf16: np.ndarray   # BF16 bits of out64 (RNE)


def quantize_weights(wo_a_bits: np.ndarray, wo_b_bits: np.ndarray):
    """BF16 weights -> MXFP8 along K: wo_a [G, N, K] -> ([G, N, K], [G, N, K/128]); wo_b [P, Kt] likewise."""
    G, N, K = wo_a_bits.shape
    wa_q, wa_sf = mx.quantize(wo_a_bits.reshape(G * N, K))
    wb_q, wb_sf = mx.quantize(wo_b_bits)
    return (wa_q.reshape(G, N, K), wa_sf.reshape(G, N, K // mx.WORD_SPAN), wb_q, wb_sf)


def o_proj_chain(x_bits, wa_q, wa_sf, wb_q, wb_sf) -> ChainResult:
    """The whole chain on BF16 x and MXFP8 weights; every intermediate is returned."""
    G, N, K = wa_q.shape
    x_q, x_sf = mx.quantize(x_bits)
    z64 = grouped_einsum(x_q, x_sf, wa_q, wa_sf, G, K, N)
    z_bf16 = mx.bf16_round(z64)
    z_q, z_sf = mx.quantize(z_bf16)
    out64 = gemm_nt(z_q, z_sf, wb_q, wb_sf)
    return ChainResult(x_q, x_sf, z64, z_bf16, z_q, z_sf, out64, mx.bf16_round(out64))


def o_proj_chain_rows(x_bits, wa_q, wa_sf, wb_q, wb_sf, rows) -> ChainResult:
    """The chain for a subset of rows (rows are independent; used at sizes too large for the whole batch)."""
    return o_proj_chain(np.asarray(x_bits)[np.asarray(rows)], wa_q, wa_sf, wb_q, wb_sf)
