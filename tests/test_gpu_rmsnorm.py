"""GPU parity of the RMS-normalizing MXFP8 producer (mxfp8_rmsnorm_quantize) against the CPU oracle.

The producer in front of the fused wqa/wkv projection (vLLM PR #57977 "[Perf][DSv4.1] Keep activations
MXFP8 between DeepGEMM kernels", before/after diagrams and Pieces) emits that GEMM's MXFP8 input and its
BF16 output in one launch.  The GPU normalizes in fp32 and the oracle in float64, so:
  * the BF16 y is within one BF16 step of the oracle's everywhere and equal on >= 99.9% of elements;
  * the MXFP8 output equals the oracle quantizer applied to the GPU's own BF16 y, bit for bit (the
    fused bytes are what a standalone quantize of the BF16 output makes);
  * against the oracle's own MXFP8 output the codes are within one E4M3 step on >= 99.9%.
Rows are the quantize-sweep rows at the fused wqa/wkv input width (7168): N(0, 1) with 1% of rows x1e3 and
1% all zero; gamma ~ N(1, 0.1).
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import chain_ref as cr
from oracle import mxfp8_ref as mx
from oracle import rmsnorm_ref as rn
from tests.gpu_common import bf16_to_dev, dev, mx_ulp_distance, to_np

pytestmark = pytest.mark.gpu
EPS = 1e-6


@pytest.fixture(scope="module")
def lib():
    import mxfp8_activation_quantization_amd as L
    L.device_check()
    return L


def bf16_ordinal(bits):
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_against_oracle(x_bits, g_bits, y_g, q_g, sf_g):
    y_o, q_o, sf_o = rn.rmsnorm_quantize(x_bits, g_bits, EPS)
    d = np.abs(bf16_ordinal(y_g) - bf16_ordinal(y_o))
    assert d.max() <= 1, f"BF16 y off by {d.max()} steps"
    assert (d == 0).mean() >= 0.999
    q2, sf2 = mx.quantize(y_g)
    assert np.array_equal(q_g, q2) and np.array_equal(sf_g, sf2), "MXFP8 output != quantize(own BF16 y)"
    ulps = mx_ulp_distance(q_g, sf_g, q_o, sf_o)
    assert (ulps <= 1).mean() >= 0.999


@pytest.mark.parametrize("M", [1, 7, 64, 300])
def test_sweep_rows_vs_oracle(lib, M):
    x = si.quant_sweep_input(M)
    g = si.rmsnorm_gamma(x.shape[1])
    y, q, sf = lib.mxfp8_rmsnorm_quantize(bf16_to_dev(x), bf16_to_dev(g), EPS, bf16_out=True)
    q1, sf1 = lib.mxfp8_rmsnorm_quantize(bf16_to_dev(x), bf16_to_dev(g), EPS)        # codes only
    assert torch.equal(q1, q) and torch.equal(sf1, sf)
    y1 = lib.mxfp8_rmsnorm_quantize(bf16_to_dev(x), bf16_to_dev(g), EPS, mxfp8_out=False)   # BF16 only
    assert torch.equal(y1, y)
    q3, sf3 = lib.mxfp8_quantize(y1)                   # the unfused pair gives the same bytes
    assert torch.equal(q3, q) and torch.equal(sf3, sf)
    check_against_oracle(x, g, to_np(y), to_np(q), to_np(sf))


def test_large_batch_sampled_rows(lib):
    M = 8192
    x = si.quant_sweep_input(M)
    g = si.rmsnorm_gamma(x.shape[1])
    y, q, sf = lib.mxfp8_rmsnorm_quantize(bf16_to_dev(x), bf16_to_dev(g), EPS, bf16_out=True)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M),
                                     np.random.default_rng(5).choice(M, 512, replace=False)]))
    check_against_oracle(x[rows], g, to_np(y)[rows], to_np(q)[rows], to_np(sf)[rows])


def test_rows_do_not_depend_on_batch(lib):
    """Large batches take several rows per workgroup (the next row's x in flight while a row is written), small
    ones one; a row's outputs are the same bits either way, in every output form."""
    M = 8192 + 5                                         # a ragged last workgroup
    x = si.quant_sweep_input(M)
    g = si.rmsnorm_gamma(x.shape[1])
    xd, gd = bf16_to_dev(x), bf16_to_dev(g)
    y, q, sf = lib.mxfp8_rmsnorm_quantize(xd, gd, EPS, bf16_out=True)
    q1, sf1 = lib.mxfp8_rmsnorm_quantize(xd, gd, EPS)
    assert torch.equal(q1, q) and torch.equal(sf1, sf)
    for lo, hi in ((0, 7), (4093, 4100), (M - 9, M)):
        ys, qs, sfs = lib.mxfp8_rmsnorm_quantize(xd[lo:hi], gd, EPS, bf16_out=True)
        assert torch.equal(ys, y[lo:hi]) and torch.equal(qs, q[lo:hi]) and torch.equal(sfs, sf[lo:hi]), (lo, hi)
    rows = np.concatenate([np.arange(8), np.arange(M - 8, M)])
    check_against_oracle(x[rows], g, to_np(y)[rows], to_np(q)[rows], to_np(sf)[rows])


def test_special_rows(lib):
    """All-zero rows give zeros with scale byte 0; constant rows give exactly +-gamma (r * c is 1 up to an
    fp32 rounding, which BF16 absorbs for gamma values with short mantissas); one non-zero element gives
    sqrt(K) * sign * gamma there."""
    K = 1024
    g = si.rmsnorm_gamma(K)
    rows = np.zeros((4, K), dtype=np.float32)
    rows[1, :] = 3.0
    rows[2, :] = -0.5
    rows[3, 17] = 2.0
    x = si.bf16_bits(rows)
    y, q, sf = lib.mxfp8_rmsnorm_quantize(bf16_to_dev(x), bf16_to_dev(g), EPS, bf16_out=True)
    y, q, sf = to_np(y), to_np(q), to_np(sf)
    assert np.all(y[0] == 0) and np.all(q[0] == 0) and np.all(sf[0] == 0)
    check_against_oracle(x, g, y, q, sf)


def test_strides_and_padding(lib):
    M, K = 33, 7168
    x = si.quant_sweep_input(M)
    g = si.rmsnorm_gamma(K)
    xs = torch.zeros((M, K + 256), dtype=torch.bfloat16, device=dev())
    xs[:, :K] = bf16_to_dev(x)
    y = torch.full((M, K + 128), 7.0, dtype=torch.bfloat16, device=dev())
    q = torch.full((M, K + 64), 0x55, dtype=torch.uint8, device=dev())
    sf = torch.full((M, K // 128 + 3), -1, dtype=torch.int32, device=dev())
    lib.mxfp8_rmsnorm_quantize(xs[:, :K], bf16_to_dev(g), EPS, y=y[:, :K], q=q[:, :K], sf=sf[:, :K // 128])
    assert torch.all(y[:, K:] == 7.0) and torch.all(q[:, K:] == 0x55) and torch.all(sf[:, K // 128:] == -1)
    check_against_oracle(x, g, to_np(y[:, :K]), to_np(q[:, :K]), to_np(sf[:, :K // 128]))


def test_feeds_the_fused_wqa_wkv_gemm(lib):
    """Producer then consumer: fp8_gemm_nt on the producer's (codes, scales) with a 7168 -> 2048 weight
    (the fused wqa/wkv width is not on the pages; 2048 stands in) is within 2e-2 of each row's RMS of the
    float64 result on the oracle's own MXFP8 y."""
    M, K, N = 64, 7168, 2048
    x = si.quant_sweep_input(M)
    g = si.rmsnorm_gamma(K)
    w_bits = si.chain_inputs(si.ChainShape(1, 1, K, N, 128), 4242, 0.0)["wo_a"].reshape(N, K)
    wq, wsf = mx.quantize(w_bits)
    q, sf = lib.mxfp8_rmsnorm_quantize(bf16_to_dev(x), bf16_to_dev(g), EPS)
    out = lib.fp8_gemm_nt(q, sf, torch.from_numpy(wq).to(dev()), torch.from_numpy(wsf).to(dev()))
    _, q_o, sf_o = rn.rmsnorm_quantize(x, g, EPS)
    ref = cr.gemm_nt(q_o, sf_o, wq, wsf)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    live = rms > 0
    err = np.max(np.abs(mx.bf16_decode(to_np(out)) - ref), axis=1)
    assert np.all(err[live] / rms[live] <= 2e-2)
    assert np.all(err[~live] == 0)
