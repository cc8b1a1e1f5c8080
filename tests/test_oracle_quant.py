"""Pins of the oracle's MXFP8 quantizer: hand-derived blocks, packing, invariants,
and bit-identity of the vectorized quantizer with the exact scalar specification.

Hand-picked blocks are derived in the comments from the OCP E4M3FN / E8M0
definitions and the scale rule (smallest e with amax <= 448 * 2**e); the other
elements of each 32-element block are +0.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import mxfp8_ref as mx


def bf16(vals):
    """float values -> BF16 bit patterns (torch CPU cast; every value below is exact in BF16)."""
    t = torch.tensor(vals, dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def block(head):
    b = np.zeros(32, dtype=np.uint16)
    h = bf16(head) if not isinstance(head, np.ndarray) else head
    b[:len(h)] = h
    return b


HANDPICKED = [
    # zeros: amax 0 -> e = -127 (byte 0x00), codes +0
    ([0.0], 0x00, [0x00]),
    # 448 = 448 * 2**0 -> e = 0 (0x7F); 448 = 1.75 * 2**8 -> exponent field 15, mantissa 6 -> 0x7E
    ([448.0], 0x7F, [0x7E]),
    # 1.0: 256 <= 448 < 512 -> e = -8 (0x77); 1.0 * 2**8 = 256 -> field 15, mantissa 0 -> 0x78
    ([1.0], 0x77, [0x78]),
    # next BF16 above 448 is 450 -> e = 1 (0x80); 225 rounds to 224 on the 16-spaced grid -> 0x76
    ([450.0], 0x80, [0x76]),
    # 448 * 2**-127 -> e = -127 (0x00) and scaled value exactly 448 -> 0x7E
    ([448.0 * 2.0 ** -127], 0x00, [0x7E]),
    # smallest BF16 subnormal 2**-133: e clamps at -127, 2**-133 * 2**127 = 2**-6 -> 0x08
    ([2.0 ** -133], 0x00, [0x08]),
    # ties go to the even code: -2**-10 is halfway 0..2**-9 -> -0 (0x80); 3 * 2**-10 -> 2**-8 (0x02);
    # 232 = 14.5 * 16 -> 224 (0x76); 248 = 15.5 * 16 -> 256 (0x78); -0.0 keeps its sign
    ([448.0, -2.0 ** -10, 3 * 2.0 ** -10, 232.0, 248.0, -0.0, 2.0 ** -9, -448.0], 0x7F,
     [0x7E, 0x80, 0x02, 0x76, 0x78, 0x80, 0x01, 0xFE]),
    # amax 2**-20 -> e = -28 (byte 99 = 0x63): 2**8 -> 0x78, 2**7 -> 0x70, 2**-6 -> 0x08, 2**-7 -> 0x04
    ([2.0 ** -20, 2.0 ** -21, 2.0 ** -34, 2.0 ** -35], 0x63, [0x78, 0x70, 0x08, 0x04]),
]


@pytest.mark.parametrize("head,sf,codes", HANDPICKED)
def test_handpicked_blocks(head, sf, codes):
    b = block(head)
    s_scalar, q_scalar = mx.quantize_block_scalar(b)
    q_vec, s_vec = mx.quantize_bytes(b[None, :])
    assert s_scalar == sf and s_vec[0, 0] == sf
    want = codes + [0x00] * (32 - len(codes))
    assert q_scalar == want
    assert list(q_vec[0]) == want


def test_handpicked_negative_max_bf16():
    # -max BF16 = -(2 - 2**-7) * 2**127: e = 120 (0xF7); scaled 255 rounds to 256 -> 0xF8
    b = np.zeros(32, dtype=np.uint16)
    b[0] = 0xFF7F
    s, q = mx.quantize_block_scalar(b)
    assert s == 0xF7 and q[0] == 0xF8 and q[1:] == [0] * 31
    qv, sv = mx.quantize_bytes(b[None, :])
    assert sv[0, 0] == 0xF7 and qv[0, 0] == 0xF8


def test_blocks_are_independent_and_in_row_order():
    # block b of a row only sees elements [32b, 32b+32)
    row = np.zeros(128, dtype=np.uint16)
    row[0:32] = bf16([1.0] * 32)
    row[32] = bf16([448.0])[0]
    row[64 + 31] = bf16([2.0 ** -20])[0]
    q, sfw = mx.quantize(row[None, :])
    sb = mx.unpack_scales(sfw)[0]
    assert list(sb) == [0x77, 0x7F, 0x63, 0x00]
    assert q[0, 32] == 0x7E and q[0, 95] == 0x78 and np.all(q[0, 96:] == 0)


def test_pack_layout_little_endian():
    rng = np.random.default_rng(3)
    sb = rng.integers(0, 255, size=(5, 56), dtype=np.uint8)
    w = mx.pack_scales(sb)
    assert w.shape == (5, 14) and w.dtype == np.int32
    # a little-endian byte view of the words is the per-block byte array
    assert np.array_equal(w.astype("<i4").view(np.uint8).reshape(5, 56), sb)
    for r in range(5):
        for wi in range(14):
            for j in range(4):
                assert (int(w[r, wi]) >> (8 * j)) & 0xFF == sb[r, 4 * wi + j]
    assert np.array_equal(mx.unpack_scales(w), sb)


def test_dequantize_value_idempotent():
    x = si.chain_inputs(si.ChainShape(16, 1, 512, 128, 128), 99, 0.01, with_weights=False)["x"]
    q, s = mx.quantize(x)
    d = mx.dequantize(q, s)
    q2, s2 = mx.quantize(mx.bf16_round(d))                 # dq values are exact in BF16
    assert np.array_equal(mx.dequantize(q2, s2), d)


def test_dequantize_error_bound():
    # |x - dq(q(x))| <= half an E4M3 ulp at the scaled value (2**-4 relative for normals,
    # 2**-10 * 2**e absolute in the subnormal range)
    x = si.chain_inputs(si.ChainShape(32, 1, 1024, 128, 128), 5, 0.001, with_weights=False)["x"]
    q, s = mx.quantize(x)
    d = mx.dequantize(q, s)
    v = mx.bf16_decode(x)
    e = np.repeat(mx.unpack_scales(s).astype(np.int64) - 127, 32, axis=1)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, np.ldexp(1.0, e - 10))
    assert np.all(np.abs(v - d) <= bound)


def test_non_finite_rejected():
    b = np.zeros((1, 128), dtype=np.uint16)
    b[0, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        mx.quantize(b)
    with pytest.raises(ValueError):
        mx.quantize_block_scalar(b[0, :32])


def test_vector_equals_scalar_tiny_config():
    inp = si.config_inputs("tiny")
    for name in ("x", "wo_a", "wo_b"):
        a = inp[name].reshape(-1, inp[name].shape[-1])
        if name != "x":
            a = a[::7]                                      # every 7th weight row keeps this quick
        qs, ss = mx.quantize_scalar(a)
        qv, sv = mx.quantize(a)
        assert np.array_equal(qs, qv), name
        assert np.array_equal(mx.pack_scales(ss), sv), name


def test_vector_equals_scalar_sweep_rows():
    # quantize sweep M = 7: one row x1e3 and one all-zero row among 7
    x = si.quant_sweep_input(7)
    qs, ss = mx.quantize_scalar(x)
    qv, sv = mx.quantize(x)
    assert np.array_equal(qs, qv) and np.array_equal(mx.pack_scales(ss), sv)
    zero_rows = np.flatnonzero(np.all(x == 0, axis=1))
    assert len(zero_rows) == 1 and np.all(sv[zero_rows] == 0)


def test_vector_equals_scalar_decode_outlier_rows():
    x = si.config_inputs("decode", with_weights=False)["x"]
    v = mx.bf16_decode(x)
    rows = np.unique(np.argwhere(np.abs(v) > 50)[:2, 0])   # rows holding x100 outliers
    sample = x[rows][:, :4096]
    qs, ss = mx.quantize_scalar(sample)
    qv, sv = mx.quantize(sample)
    assert np.array_equal(qs, qv) and np.array_equal(mx.pack_scales(ss), sv)
