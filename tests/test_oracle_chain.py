"""Pins of the oracle's o_proj chain: index maps by one-hot operands, an exact
rational brute force of the whole chain on a tiny case, and the BF16-before-
quantize order of the fused epilogue.

The index map z[m, g*N+n] = sum_k x[m, g*K+k] * wo_a[g, n, k] is the plain
reading of "8 groups x 4096 -> 1024" in vLLM PR #60118 ("[Perf][DSv4.1]
MegaAttn: wo_a writes wo_b's MXFP8 input", section Validation); one-hot
operands make every entry of z a single, predictable element of x or wo_a, so a
transposed operand, a wrong group offset or a dropped scale fails here.
"""
from fractions import Fraction

import numpy as np
import torch

import synth_inputs as si
from oracle import chain_ref as cr
from oracle import mxfp8_ref as mx


def bf16(vals):
    t = torch.tensor(np.asarray(vals, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_einsum_one_hot_weights_gathers_x():
    M, G, K, N = 3, 3, 256, 128
    x = si.chain_inputs(si.ChainShape(M, G, K, N, 128), 17, 0.0, with_weights=False)["x"]
    sel = np.array([[(5 * n + 11 * g) % K for n in range(N)] for g in range(G)])
    w = np.zeros((G, N, K))
    for g in range(G):
        w[g, np.arange(N), sel[g]] = 1.0
    wq, wsf = mx.quantize(bf16(w).reshape(G * N, K))
    xq, xsf = mx.quantize(x)
    z = cr.grouped_einsum(xq, xsf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N)
    xd = mx.dequantize(xq, xsf)
    for g in range(G):
        assert np.array_equal(z[:, g * N:(g + 1) * N], xd[:, g * K + sel[g]])


def test_einsum_one_hot_x_gathers_weights():
    M, G, K, N = 4, 2, 256, 128
    w = si.chain_inputs(si.ChainShape(1, G, K, N, 128), 23, 0.0)["wo_a"]
    x = np.zeros((M, G * K))
    cols = [7, K + 200, 31, 2 * K - 1]                       # row m reads group cols[m] // K
    for m, c in enumerate(cols):
        x[m, c] = 1.0
    xq, xsf = mx.quantize(bf16(x))
    wq, wsf = mx.quantize(w.reshape(G * N, K))
    z = cr.grouped_einsum(xq, xsf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N)
    wd = mx.dequantize(wq, wsf).reshape(G, N, K)
    for m, c in enumerate(cols):
        g, k = divmod(c, K)
        assert np.array_equal(z[m, g * N:(g + 1) * N], wd[g, :, k])
        other = [h for h in range(G) if h != g]
        for h in other:
            assert np.all(z[m, h * N:(h + 1) * N] == 0)


def test_gemm_one_hot_b_gathers_a():
    M, Kt, P = 5, 384, 256
    a = si.chain_inputs(si.ChainShape(M, 1, Kt, 128, 128), 29, 0.0, with_weights=False)["x"]
    sel = (np.arange(P) * 37 + 3) % Kt
    b = np.zeros((P, Kt))
    b[np.arange(P), sel] = 1.0
    aq, asf = mx.quantize(a)
    bq, bsf = mx.quantize(bf16(b))
    out = cr.gemm_nt(aq, asf, bq, bsf)
    assert np.array_equal(out, mx.dequantize(aq, asf)[:, sel])


def test_gemm_scales_multiply_both_operands():
    # 128 equal elements 2**ea and 2**eb: out = 128 * 2**(ea + eb) whatever the scales
    for ea in (-20, 0, 7):
        for eb in (-3, 0, 11):
            a = bf16([2.0 ** ea] * 128)[None, :]
            b = bf16([2.0 ** eb] * 128)[None, :]
            aq, asf = mx.quantize(a)
            bq, bsf = mx.quantize(b)
            assert cr.gemm_nt(aq, asf, bq, bsf)[0, 0] == 128 * 2.0 ** (ea + eb)


def _exact_chain(x_bits, wa_bits, wb_bits):
    """The chain in exact rationals with pure-Python loops (tiny sizes only)."""
    G, N, K = wa_bits.shape
    M = x_bits.shape[0]
    P = wb_bits.shape[0]

    def q_rows(bits):
        out = []
        for row in bits:
            vals = []
            for b0 in range(0, len(row), 32):
                s, codes = mx.quantize_block_scalar(row[b0:b0 + 32])
                scale = Fraction(2) ** (s - 127)
                vals.extend(Fraction(mx.e4m3_decode_scalar(c)) * scale for c in codes)
            out.append(vals)
        return out

    xd = q_rows(x_bits)
    wad = q_rows(wa_bits.reshape(G * N, K))
    wbd = q_rows(wb_bits)
    z = [[sum(xd[m][g * K + k] * wad[g * N + n][k] for k in range(K)) for g in range(G) for n in range(N)]
         for m in range(M)]
    # BF16 of the exact z (the exact value rounds once; float64 is not involved)
    z_bits = np.array([[_bf16_exact(v) for v in row] for row in z], dtype=np.uint16)
    zd = q_rows(z_bits)
    out = [[sum(zd[m][j] * wbd[p][j] for j in range(G * N)) for p in range(P)] for m in range(M)]
    return z, z_bits, out


def _bf16_exact(v: Fraction) -> int:
    """RNE of an exact rational to BF16 by comparing with the two BF16 neighbours of float(v)."""
    b = int(mx.bf16_round(np.array([float(v)]))[0])
    best = None
    for d in (-1, 0, 1):
        c = b + d
        if 0 <= (c & 0x7FFF) <= 0x7F7F:
            dist = abs(Fraction(mx.bf16_decode_scalar(c)) - v)
            key = (dist, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
    return best[1]


def test_chain_matches_exact_rational_bruteforce():
    shape = si.ChainShape(2, 2, 128, 128, 128)
    inp = si.chain_inputs(shape, 31, 0.0)
    wa_q, wa_sf, wb_q, wb_sf = cr.quantize_weights(inp["wo_a"], inp["wo_b"])
    r = cr.o_proj_chain(inp["x"], wa_q, wa_sf, wb_q, wb_sf)
    z_ex, zb_ex, out_ex = _exact_chain(inp["x"], inp["wo_a"], inp["wo_b"])
    z_ex = np.array([[float(v) for v in row] for row in z_ex])
    out_ex = np.array([[float(v) for v in row] for row in out_ex])
    assert np.max(np.abs(r.z64 - z_ex)) <= 1e-12 * np.max(np.abs(z_ex))
    assert np.array_equal(r.z_bf16, zb_ex)
    assert np.max(np.abs(r.out64 - out_ex)) <= 1e-12 * np.max(np.abs(out_ex))


def test_fused_epilogue_quantizes_the_bf16_z():
    # z64 = 448 + 0.4375 lies below the midpoint to the next BF16 (450), so the BF16 z
    # is exactly 448 and its block scale is e = 0 (0x7F).  Quantizing the float64 value
    # instead would give e = 1 (0x80): the test separates the two orders.
    G, K, N = 1, 128, 128
    x = np.zeros((1, K))
    x[0, 0], x[0, 1] = 448.0, 0.4375
    w = np.zeros((G, N, K))
    w[0, 0, 0] = w[0, 0, 1] = 1.0
    wb = np.eye(128)
    wa_q, wa_sf, wb_q, wb_sf = cr.quantize_weights(bf16(w).reshape(G, N, K), bf16(wb))
    r = cr.o_proj_chain(bf16(x), wa_q, wa_sf, wb_q, wb_sf)
    assert r.z64[0, 0] == 448.4375
    assert r.z_bf16[0, 0] == bf16([448.0])[0]
    assert mx.unpack_scales(r.z_sf)[0, 0] == 0x7F and r.z_q[0, 0] == 0x7E
    assert r.out64[0, 0] == 448.0                              # identity wo_b passes dq(z) through


def test_chain_rows_are_independent():
    shape = si.ChainShape(6, 2, 256, 128, 256)
    inp = si.chain_inputs(shape, 37, 0.01)
    w = cr.quantize_weights(inp["wo_a"], inp["wo_b"])
    full = cr.o_proj_chain(inp["x"], *w)
    part = cr.o_proj_chain_rows(inp["x"], *w, rows=[4, 1])
    assert np.array_equal(part.out64, full.out64[[4, 1]])
    assert np.array_equal(part.z_q, full.z_q[[4, 1]])
