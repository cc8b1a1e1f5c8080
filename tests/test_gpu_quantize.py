"""GPU parity of mxfp8_quantize against the CPU oracle: bit-exact codes and scales.

Cases: every finite BF16 value at every reachable block scale, the hand-derived
blocks, the standalone quantize sweep [M, 7168] for M in {1, 7, 64, 300, 8192}
(N(0,1) rows, 1% rows x1e3 and 1% all-zero rows; the hidden size of the
wqa/wkv input in vLLM PR #57977, Purpose), strided rows with guard bytes, and
the empty batch.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import mxfp8_ref as mx

pytestmark = pytest.mark.gpu

from tests.gpu_common import bf16_to_dev, dev, to_np  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    import mxfp8_activation_quantization_amd as m
    m.device_check()
    return m


def run(lib, bits):
    q, sf = lib.mxfp8_quantize(bf16_to_dev(bits))
    torch.cuda.synchronize()
    return to_np(q), to_np(sf)


def check_exact(lib, bits):
    gq, gs = run(lib, bits)
    oq, os_ = mx.quantize(bits)
    bad = np.flatnonzero((gq != oq).any(axis=1) | (gs != os_).any(axis=1))
    assert bad.size == 0, f"rows {bad[:8]} differ"


def all_bf16_at_every_scale():
    """Blocks [anchor, v1..v31] with anchor = 448 * 2**e (or the largest BF16): the block's scale is e and
    every finite BF16 v with |v| <= anchor appears once at that scale, for every e the rule can give."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = mx.bf16_decode(b)
    fin = np.isfinite(v)
    b, v = b[fin], v[fin]
    blocks = []
    for e in range(-127, 121):
        anchor = 448.0 * 2.0 ** e if e < 120 else float(mx.bf16_decode(np.array([0x7F7F], np.uint16))[0])
        a_bits = mx.bf16_round(np.array([anchor]))[0]
        vals = b[np.abs(v) <= anchor]
        pad = (-len(vals)) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        blk = np.concatenate([np.full((len(vals), 1), a_bits, np.uint16), vals], axis=1)
        blocks.append(blk)
    blocks = np.concatenate(blocks).reshape(-1)
    pad = (-len(blocks)) % 7168
    blocks = np.concatenate([blocks, np.zeros(pad, np.uint16)])
    return blocks.reshape(-1, 7168)


def test_every_bf16_value_at_every_scale(lib):
    x = all_bf16_at_every_scale()
    print(f"exhaustive: {x.size} elements in {x.shape[0]} rows", flush=True)
    check_exact(lib, x)


@pytest.mark.parametrize("M", si.QUANT_SWEEP_M)
def test_quant_sweep(lib, M):
    print(f"quantize sweep M={M} K={si.QUANT_SWEEP_K}", flush=True)
    check_exact(lib, si.quant_sweep_input(M))


def test_handpicked_blocks(lib):
    rows = np.zeros((4, 128), dtype=np.uint16)
    t = torch.tensor([448.0, -2.0 ** -10, 3 * 2.0 ** -10, 232.0, 248.0, -0.0, 2.0 ** -9, -448.0],
                     dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rows[0, :8] = t
    rows[1, 0] = 0xFF7F                       # -max BF16
    rows[1, 32] = 0x0001                      # smallest subnormal
    rows[2, 64] = mx.bf16_round(np.array([450.0]))[0]
    rows[3, 96:100] = mx.bf16_round(np.array([2.0 ** -20, 2.0 ** -21, 2.0 ** -34, 2.0 ** -35]))
    gq, gs = run(lib, rows)
    sb = mx.unpack_scales(gs)
    assert sb[0, 0] == 0x7F and list(gq[0, :8]) == [0x7E, 0x80, 0x02, 0x76, 0x78, 0x80, 0x01, 0xFE]
    assert sb[1, 0] == 0xF7 and gq[1, 0] == 0xF8
    assert sb[1, 1] == 0x00 and gq[1, 32] == 0x08
    assert sb[2, 2] == 0x80 and gq[2, 64] == 0x76
    assert sb[3, 3] == 0x63 and list(gq[3, 96:100]) == [0x78, 0x70, 0x08, 0x04]
    assert sb[0, 1] == 0 and np.all(gq[0, 8:] == 0)     # zero blocks


def test_strided_rows_leave_padding_untouched(lib):
    M, K = 37, 640
    x = si.chain_inputs(si.ChainShape(M, 1, K, 128, 128), 41, 0.01, with_weights=False)["x"]
    xs = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=dev())
    xs[:, :K] = bf16_to_dev(x)
    q = torch.full((M, K + 48), 0xA5, dtype=torch.uint8, device=dev())
    sf = torch.full((M, K // 128 + 3), 0x5A5A5A5A, dtype=torch.int32, device=dev())
    lib.mxfp8_quantize(xs[:, :K], q[:, :K], sf[:, :K // 128])
    torch.cuda.synchronize()
    oq, os_ = mx.quantize(x)
    assert np.array_equal(to_np(q)[:, :K], oq) and np.array_equal(to_np(sf)[:, :K // 128], os_)
    assert np.all(to_np(q)[:, K:] == 0xA5) and np.all(to_np(sf)[:, K // 128:] == 0x5A5A5A5A)


def test_rows_past_one_grid_trip(lib):
    """More 128-element spans than one trip of the capped grid covers (256 x 64 workgroups x 16 span
    groups x 4 spans = 2^20 spans = 4096 rows of 32768): the kernel loops, and rows of both trips --
    the first and last rows, rows at the trip boundary and random rows -- are bit-exact against the
    oracle.  Rows are independent random finite BF16 patterns, so a row written to the wrong place
    cannot match by accident."""
    M, K = 4608, 32768
    rng = np.random.default_rng(4608)
    bits = rng.integers(0, 1 << 16, size=(M, K), dtype=np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] &= 0xBFFF                     # no Inf / NaN patterns: clear an exponent bit
    print(f"quantize grid loop M={M} K={K}", flush=True)
    q, sf = lib.mxfp8_quantize(bf16_to_dev(bits))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(4), np.arange(4090, 4102), np.arange(M - 4, M),
                                     rng.choice(M, 96, replace=False)]))
    oq, os_ = mx.quantize(bits[rows])
    idx = torch.from_numpy(rows).to(dev())
    assert np.array_equal(to_np(q[idx]), oq) and np.array_equal(to_np(sf[idx]), os_)


def test_empty_batch_is_noop(lib):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev())
    q, sf = lib.mxfp8_quantize(x)
    assert q.shape == (0, 256) and sf.shape == (0, 2)


def test_bad_shape_raises_value_error(lib):
    x = torch.zeros((4, 96), dtype=torch.bfloat16, device=dev())
    with pytest.raises(ValueError):
        lib.mxfp8_quantize(x)
