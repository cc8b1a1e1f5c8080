"""GPU parity of grouped_fp8_einsum, fp8_gemm_nt and the o_proj chain against the CPU oracle.

The shapes are the DeepSeek-V4.1-Flash TP1 o_proj of vLLM PR #60118
("[Perf][DSv4.1] MegaAttn: wo_a writes wo_b's MXFP8 input", Validation):
8 groups x 4096 -> 1024, then 8192 -> 5120; plus a tiny chain (2 x 256 -> 128,
256 -> 256).  Bars:
  * exact-arithmetic regime (small codes, every partial sum exact in fp32):
    BF16 outputs, z codes and z scales bit-exact with the oracle;
  * invariants from the pages, bitwise: the fused MXFP8 z equals the quantizer
    applied to the same kernel's BF16 z (PR #60118, Tests); pre-quantized x
    equals in-kernel quantization (PR #57977, Test Result); the fused and
    unfused chains give identical outputs (PR #60118, Validation);
  * against the independent float64 oracle: z codes within 1 E4M3 ulp on at
    least 99.9% of elements, every z scale that differs explained by a block
    maximum within one BF16 step of a power-of-two threshold;
  * the wo_b GEMM fed the oracle's own z: BF16 output within 2e-2 of each row's
    RMS (max |err| / RMS);
  * the whole chain: max |out - out64| / RMS(row) <= 2e-2 on every row checked
    (the bar as stated, no allowance).  The propagation through |wo_b| of the z
    code flips that the z bar admits is printed beside it as a diagnostic.
    (gfx950's FP8 MFMA cuts each product of a group of 8 to 13 bits below the
    group's largest; the einsum feeds large and small activation codes as two
    operands so that x's outliers do not cost their neighbours bits -- see
    test_gpu_mfma_precision.py -- which keeps the chain's error at that of
    rounding the exact result to BF16.)
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from oracle import chain_ref as cr
from oracle import mxfp8_ref as mx
from tests.gpu_common import bf16_to_dev, dev, i32_to_dev, mx_ulp_distance, row_rel_err, to_np, u8_to_dev

pytestmark = pytest.mark.gpu

OUT_TOL = 2e-2


@pytest.fixture(scope="module")
def lib():
    import mxfp8_activation_quantization_amd as m
    m.device_check()
    return m


# --------------------------------------------------------------------------- exact regime

SMALL_CODES = np.array([0x00, 0x38, 0xB8, 0x40, 0xC0, 0x30, 0xB0], dtype=np.uint8)   # 0, +-1, +-2, +-0.5


def exact_operands(rng, rows, cols):
    """Codes in {0, +-0.5, +-1, +-2} and scales 2**{-1,0,1}: every product is a multiple of 2**-4 with
    magnitude <= 16, so sums over K <= 4096 need at most 20 bits and fp32 accumulates them exactly."""
    q = rng.choice(SMALL_CODES, size=(rows, cols))
    sb = rng.integers(126, 129, size=(rows, cols // 32)).astype(np.uint8)
    return q, mx.pack_scales(sb)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (7, 256, 512), (33, 384, 1024), (130, 256, 4096),
                                   (257, 128, 256), (5, 128, 1152), (40, 256, 2176), (64, 512, 8192),
                                   (300, 512, 1024), (513, 384, 512), (1024, 256, 4096), (777, 768, 128)])
def test_gemm_exact_regime_bitexact(lib, M, N, K):
    rng = np.random.default_rng(1000 + M)
    aq, asf = exact_operands(rng, M, K)
    bq, bsf = exact_operands(rng, N, K)
    d = lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(bq), i32_to_dev(bsf))
    ref = mx.bf16_round(cr.gemm_nt(aq, asf, bq, bsf))
    assert np.array_equal(to_np(d), ref)


@pytest.mark.parametrize("kind,M,G,N,K", [("gemm", 4000, 1, 5120, 256), ("einsum", 2304, 8, 1024, 256)])
def test_mixed_tile_shapes_bitexact(lib, kind, M, G, N, K):
    """Launches whose last rows of tokens use the narrower tiles (wo_b at 4000 tokens: 12 of 16 rows of 256
    tokens as 256-wide tiles; the einsum at 2304 tokens: 8 of 9): still bit-exact in the exact regime."""
    rng = np.random.default_rng(4000 + M)
    aq, asf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    if kind == "gemm":
        d = lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq), i32_to_dev(wsf))
        ref = mx.bf16_round(cr.gemm_nt(aq, asf, wq, wsf))
    else:
        d = lib.grouped_fp8_einsum(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq.reshape(G, N, K)),
                                   i32_to_dev(wsf.reshape(G, N, K // 128)), out="bf16")
        ref = mx.bf16_round(cr.grouped_einsum(aq, asf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N))
    assert np.array_equal(to_np(d), ref)


def _random_shapes(n, seed, m_range, n_steps):
    """Seeded shapes around the tile kernels' plan: tokens in m_range, 1-4 groups, weight rows in 128-steps
    from n_steps, 1-12 K-steps (fewer steps than step buffers included), einsum and GEMM."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kind = "einsum" if rng.random() < 0.5 else "gemm"
        M = int(rng.integers(*m_range))
        G = int(rng.integers(1, 5)) if kind == "einsum" else 1
        N = 128 * int(rng.integers(*n_steps))
        K = 128 * int(rng.integers(1, 13))
        out.append((kind, M, G, N, K))
    return out


@pytest.mark.parametrize("kind,M,G,N,K", _random_shapes(16, 20261202, (129, 1501), (1, 13)) +
                         _random_shapes(8, 20261203, (700, 3001), (8, 41)))
def test_random_tile_shapes_bitexact(lib, kind, M, G, N, K):
    """Seeded random shapes through the tile kernels (both families, wide and half-width tiles, ragged
    token rows, short K ranges): bit-exact against the oracle in the exact regime, every output form."""
    rng = np.random.default_rng(M * 7 + N + K)
    aq, asf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    if kind == "gemm":
        d = lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq), i32_to_dev(wsf))
        assert np.array_equal(to_np(d), mx.bf16_round(cr.gemm_nt(aq, asf, wq, wsf)))
        return
    ref = mx.bf16_round(cr.grouped_einsum(aq, asf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N))
    oq, osf = mx.quantize(ref)
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq.reshape(G, N, K)),
                                            i32_to_dev(wsf.reshape(G, N, K // 128)), out="both")
    assert np.array_equal(to_np(z_b), ref)
    assert np.array_equal(to_np(z_q), oq) and np.array_equal(to_np(z_sf), osf)


@pytest.mark.parametrize("kind,M_small,M_big,G,N,K", [("einsum", 512, 1024, 8, 1024, 4096),
                                                      ("gemm", 768, 1024, 1, 5120, 8192),
                                                      ("gemm", 300, 2000, 1, 2560, 1024)])
def test_tile_families_give_identical_bits(lib, kind, M_small, M_big, G, N, K):
    """Random operands, outside the exact regime: the same token rows computed in a launch that takes the
    128 x 128 tile family (M_small) and in one that takes the 256 x 256 family (M_big, with 128 x 256 tiles
    for its last rows) are bit-identical -- every output element is one whole-K accumulation of the same
    bytes in the same order whatever the tile shape."""
    rng = np.random.default_rng(11000 + M_big)

    def random_mxfp8(rows, cols):
        q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] ^= 1                                  # no NaN codes
        sb = rng.integers(120, 131, size=(rows, cols // 32)).astype(np.uint8)
        return q, mx.pack_scales(sb)

    aq, asf = random_mxfp8(M_big, G * K)
    wq, wsf = random_mxfp8(G * N, K)
    outs = []
    for M in (M_small, M_big):
        a_t, asf_t = u8_to_dev(aq[:M]), i32_to_dev(asf[:M])
        if kind == "gemm":
            outs.append(to_np(lib.fp8_gemm_nt(a_t, asf_t, u8_to_dev(wq), i32_to_dev(wsf))))
        else:
            z_q, z_sf, z_b = lib.grouped_fp8_einsum(a_t, asf_t, u8_to_dev(wq.reshape(G, N, K)),
                                                    i32_to_dev(wsf.reshape(G, N, K // 128)), out="both")
            outs.append((to_np(z_q), to_np(z_sf), to_np(z_b)))
    if kind == "gemm":
        assert np.array_equal(outs[0], outs[1][:M_small])
    else:
        for small, big in zip(outs[0], outs[1]):
            assert np.array_equal(small, big[:M_small])


@pytest.mark.parametrize("M", [1, 7, 12, 32])
@pytest.mark.parametrize("kind,G,N,K", [("gemm", 1, 4096, 8192), ("gemm", 1, 5120, 384), ("einsum", 8, 512, 256),
                                        ("einsum", 4, 1024, 1152), ("einsum", 8, 1024, 2048), ("gemm", 1, 8192, 1152)])
def test_whole_k_exact_regime_bitexact(lib, kind, M, G, N, K):
    """At most 32 tokens with at least 128 workgroups of 32 weight rows: each workgroup takes the whole K
    range (up to 64 steps of 128, odd step counts included) and its four waves' partial tiles are added at
    the end; the ring holds 8, 16 or 32 token rows per step (M = 1, 7 | 12 | 32), four stages deep on grids
    of 128-160 workgroups and three on grids of 256 (the last two shapes).  Bit-exact in the exact regime,
    for every output form."""
    rng = np.random.default_rng(7000 + M + K)
    aq, asf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    if kind == "gemm":
        d = lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq), i32_to_dev(wsf))
        assert np.array_equal(to_np(d), mx.bf16_round(cr.gemm_nt(aq, asf, wq, wsf)))
        return
    ref = mx.bf16_round(cr.grouped_einsum(aq, asf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N))
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq.reshape(G, N, K)),
                                            i32_to_dev(wsf.reshape(G, N, K // 128)), out="both")
    assert np.array_equal(to_np(z_b), ref)
    oq, osf = mx.quantize(ref)
    assert np.array_equal(to_np(z_q), oq) and np.array_equal(to_np(z_sf), osf)


@pytest.mark.parametrize("M", [33, 40, 64])
@pytest.mark.parametrize("kind,G,N,K", [("gemm", 1, 8192, 384), ("einsum", 8, 1024, 1152), ("einsum", 8, 1024, 8192)])
def test_whole_k_two_token_tiles_bitexact(lib, kind, M, G, N, K):
    """33 to 64 tokens on a grid of at least 256 workgroups: whole K per workgroup with two token tiles, each
    summed by two waves (even and odd steps).  Bit-exact in the exact regime, every output form."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(8000 + M + K)
    aq, asf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    if kind == "gemm":
        assert B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, M, N, K) == 0      # no split
        d = lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq), i32_to_dev(wsf))
        assert np.array_equal(to_np(d), mx.bf16_round(cr.gemm_nt(aq, asf, wq, wsf)))
        return
    assert B.lib().grouped_fp8_einsum_workspace_size(B.MXFP8_ACT_MXFP8, M, G, K, N) == 0
    ref = mx.bf16_round(cr.grouped_einsum(aq, asf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N))
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(wq.reshape(G, N, K)),
                                            i32_to_dev(wsf.reshape(G, N, K // 128)), out="both")
    assert np.array_equal(to_np(z_b), ref)
    oq, osf = mx.quantize(ref)
    assert np.array_equal(to_np(z_q), oq) and np.array_equal(to_np(z_sf), osf)


@pytest.mark.parametrize("M", [65, 97, 128])
@pytest.mark.parametrize("kind,G,N,K", [("gemm", 1, 5120, 8192), ("gemm", 1, 4096, 384), ("einsum", 8, 1024, 4096),
                                        ("einsum", 4, 1024, 1152)])
def test_whole_k_four_token_tiles_bitexact(lib, kind, M, G, N, K):
    """65 to 128 tokens on a grid of at least 128 workgroups: whole K per workgroup with four token tiles, one
    wave each over every step; token rows past M in the last tile are neither loaded nor stored (M = 65, 97).
    Bit-exact in the exact regime, every output form, no workspace."""
    test_whole_k_two_token_tiles_bitexact(lib, kind, M, G, N, K)


@pytest.mark.parametrize("M,G,K,N", [(4, 2, 256, 128), (45, 3, 512, 256), (96, 8, 128, 128), (3, 2, 1152, 128),
                                     (64, 2, 4096, 256), (600, 2, 512, 512), (257, 3, 256, 128),
                                     (520, 2, 1024, 384)])
def test_einsum_exact_regime_bitexact(lib, M, G, K, N):
    rng = np.random.default_rng(2000 + M)
    xq, xsf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(u8_to_dev(xq), i32_to_dev(xsf), u8_to_dev(wq.reshape(G, N, K)),
                                            i32_to_dev(wsf.reshape(G, N, K // 128)), out="both")
    z64 = cr.grouped_einsum(xq, xsf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N)
    zb = mx.bf16_round(z64)
    oq, osf = mx.quantize(zb)
    assert np.array_equal(to_np(z_b), zb)
    assert np.array_equal(to_np(z_q), oq)
    assert np.array_equal(to_np(z_sf), osf)


EXACT_VALUES = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0], dtype=np.float32)


def _nan_padded(rows_valid, t, fill):
    """A device tensor whose storage continues past row `rows_valid` with `fill` (a NaN pattern), viewed
    as its first rows_valid rows: a kernel that reads a row past M meets the NaN."""
    big = torch.empty((rows_valid + 64,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev())
    big.view(torch.uint8 if t.dtype == torch.uint8 else (torch.int16 if t.dtype == torch.bfloat16 else torch.int32))\
        .fill_(fill)
    big[:rows_valid] = t
    return big[:rows_valid]


@pytest.mark.parametrize("M,N,G,Ng", [(7, 512, 2, 256), (33, 512, 2, 256), (290, 512, 2, 256), (300, 512, 2, 256),
                                     (7, 4096, 8, 512), (33, 8192, 8, 1024)])
def test_rows_past_m_are_never_read(lib, M, N, G, Ng):
    """Exact regime (BF16 values that quantize exactly; sums exact in fp32) with activation storage that
    continues past row M with NaN bytes: every output must still equal the oracle bit for bit, for BF16
    activations and for E4M3 activations, in the GEMM and the einsum (split-K, tile and whole-K kernels)."""
    rng = np.random.default_rng(300 + M + N)
    K = 1024
    a = rng.choice(EXACT_VALUES, size=(M, K))
    bq, bsf = exact_operands(rng, N, K)
    ref = mx.bf16_round(a.astype(np.float64) @ (mx.E4M3_TABLE[bq] * np.repeat(
        np.ldexp(1.0, mx.unpack_scales(bsf).astype(np.int64) - 127), 32, axis=1)).T)
    at = _nan_padded(M, torch.from_numpy(a).to(torch.bfloat16).to(dev()), 0x7FC0)
    b_t, bsf_t = u8_to_dev(bq), i32_to_dev(bsf)
    assert np.array_equal(to_np(lib.fp8_gemm_nt(at, None, b_t, bsf_t)), ref)
    aq, asf = lib.mxfp8_quantize(at)
    aq_p, asf_p = _nan_padded(M, aq, 0x7F), _nan_padded(M, asf, -1)
    assert np.array_equal(to_np(lib.fp8_gemm_nt(aq_p, asf_p, b_t, bsf_t)), ref)
    # einsum, BF16 and E4M3 x
    x = rng.choice(EXACT_VALUES, size=(M, G * K))
    wq, wsf = exact_operands(rng, G * Ng, K)
    w_t, wsf_t = u8_to_dev(wq.reshape(G, Ng, K)), i32_to_dev(wsf.reshape(G, Ng, K // 128))
    xq_o, xsf_o = mx.quantize(mx.bf16_round(x))
    z_ref = mx.bf16_round(cr.grouped_einsum(xq_o, xsf_o, wq.reshape(G, Ng, K), wsf.reshape(G, Ng, K // 128),
                                            G, K, Ng))
    xt = _nan_padded(M, torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(dev()), 0x7FC0)
    assert np.array_equal(to_np(lib.grouped_fp8_einsum(xt, None, w_t, wsf_t, out="bf16")), z_ref)
    xq, xsf = lib.mxfp8_quantize(xt)
    zq = lib.grouped_fp8_einsum(_nan_padded(M, xq, 0x7F), _nan_padded(M, xsf, -1), w_t, wsf_t, out="bf16")
    assert np.array_equal(to_np(zq), z_ref)


def test_split_k_workspace_counters_return_to_zero(lib):
    """The split-K arrival counters are back at zero after each call, so the workspace can be reused."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(77)
    M, N, K = 48, 256, 4096
    aq, asf = exact_operands(rng, M, K)
    bq, bsf = exact_operands(rng, N, K)
    need = B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, M, N, K)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    outs = [lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(bq), i32_to_dev(bsf), workspace=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(o, outs[0]) for o in outs)
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0           # the whole counter region
    assert np.array_equal(to_np(outs[0]), mx.bf16_round(cr.gemm_nt(aq, asf, bq, bsf)))


@pytest.mark.parametrize("kind,M,G,N,K", [("gemm", 48, 1, 256, 4096), ("gemm", 64, 1, 5120, 8192),
                                          ("gemm", 5, 1, 128, 2176), ("einsum", 64, 4, 1024, 4096),
                                          ("einsum", 33, 3, 256, 1024), ("gemm", 64, 1, 6144, 4096),
                                          ("gemm", 40, 1, 5120, 2048), ("gemm", 64, 1, 4096, 4096)])
def test_split_k_combine_modes_give_identical_bits(lib, kind, M, G, N, K):
    """The decode kernels combine split-K partials through one XCD's L2 (default), through memory, or by
    recomputing the other splits (the fallback when a tile's splits ran on different XCDs): all three give
    the same bits, equal to the oracle in the exact regime, and leave the counters at zero.  The shapes
    take 2, 3, 4 and 8 splits; with 2 or 3 the last split is the longer one (wo_b: 20/20/24 of 64 steps;
    6144 x 4096: 14/18; 5120 x 2048: 4/4/8; the 33-token einsum: 2/6), with 4 or 8 they are equal."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(300 + M + N)
    aq, asf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    a_t, asf_t = u8_to_dev(aq), i32_to_dev(asf)
    if kind == "gemm":
        w_t, wsf_t = u8_to_dev(wq), i32_to_dev(wsf)
    else:
        w_t, wsf_t = u8_to_dev(wq.reshape(G, N, K)), i32_to_dev(wsf.reshape(G, N, K // 128))
    need = (B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, M, N, K) if kind == "gemm"
            else B.lib().grouped_fp8_einsum_workspace_size(B.MXFP8_ACT_MXFP8, M, G, K, N))
    assert need > 0                                                       # the shape is split along K
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    outs = {}
    for mode in ("local", "through", "recompute", "local"):
        if kind == "gemm":
            outs[mode] = to_np(lib.fp8_gemm_nt(a_t, asf_t, w_t, wsf_t, workspace=ws, splitk_combine=mode))
        else:
            outs[mode] = to_np(lib.grouped_fp8_einsum(a_t, asf_t, w_t, wsf_t, out="bf16", workspace=ws,
                                                      splitk_combine=mode))
        torch.cuda.synchronize()
        assert int(ws[:4096].view(torch.int32).abs().sum()) == 0, mode
    assert np.array_equal(outs["through"], outs["local"])
    assert np.array_equal(outs["recompute"], outs["local"])
    if kind == "gemm":
        ref = mx.bf16_round(cr.gemm_nt(aq, asf, wq, wsf))
    else:
        ref = mx.bf16_round(cr.grouped_einsum(aq, asf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N))
    assert np.array_equal(outs["local"], ref)


def _modes_bitexact(lib, kind, M, G, N, K, seed, modes=("local", "through", "recompute", "local")):
    """Runs one exact-regime call per combine mode on one workspace; every output form must equal the oracle
    bit for bit and the counter region must be zero again after each call."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(seed)
    aq, asf = exact_operands(rng, M, G * K)
    wq, wsf = exact_operands(rng, G * N, K)
    a_t, asf_t = u8_to_dev(aq), i32_to_dev(asf)
    need = (B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, M, N, K) if kind == "gemm"
            else B.lib().grouped_fp8_einsum_workspace_size(B.MXFP8_ACT_MXFP8, M, G, K, N))
    ws = torch.zeros(max(need, 65536), dtype=torch.uint8, device=dev())
    if kind == "gemm":
        ref = mx.bf16_round(cr.gemm_nt(aq, asf, wq, wsf))
        w_t, wsf_t = u8_to_dev(wq), i32_to_dev(wsf)
    else:
        ref = mx.bf16_round(cr.grouped_einsum(aq, asf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N))
        oq, osf = mx.quantize(ref)
        w_t, wsf_t = u8_to_dev(wq.reshape(G, N, K)), i32_to_dev(wsf.reshape(G, N, K // 128))
    for mode in modes:
        if kind == "gemm":
            d = lib.fp8_gemm_nt(a_t, asf_t, w_t, wsf_t, workspace=ws, splitk_combine=mode)
            assert np.array_equal(to_np(d), ref), mode
        else:
            z_q, z_sf, z_b = lib.grouped_fp8_einsum(a_t, asf_t, w_t, wsf_t, out="both", workspace=ws,
                                                    splitk_combine=mode)
            assert np.array_equal(to_np(z_b), ref), mode
            assert np.array_equal(to_np(z_q), oq) and np.array_equal(to_np(z_sf), osf), mode
            z_q2, z_sf2 = lib.grouped_fp8_einsum(a_t, asf_t, w_t, wsf_t, out="mxfp8", workspace=ws,
                                                 splitk_combine=mode)
            assert torch.equal(z_q2, z_q) and torch.equal(z_sf2, z_sf), mode
            z_b2 = lib.grouped_fp8_einsum(a_t, asf_t, w_t, wsf_t, out="bf16", workspace=ws, splitk_combine=mode)
            assert torch.equal(z_b2, z_b), mode
        torch.cuda.synchronize()
        assert int(ws[:65536].view(torch.int32).abs().sum()) == 0, mode


@pytest.mark.parametrize("M", [1, 20, 33, 64])
@pytest.mark.parametrize("kind,G,N,K", [("einsum", 8, 1024, 4096), ("gemm", 1, 5120, 8192)])
def test_decode_shapes_bitexact(lib, kind, M, G, N, K):
    """The decode shapes (wo_a 8 x 4096 -> 1024 and wo_b 8192 -> 5120) at up to 64 tokens, whichever decode
    kernel takes them: in the exact regime every output form equals the oracle bit for bit in each combine
    mode, and the counter region of the workspace is zero again after every call."""
    _modes_bitexact(lib, kind, M, G, N, K, 9100 + M + N)


@pytest.mark.parametrize("kind,M,G,N,K", [("gemm", 65, 1, 5120, 8192), ("gemm", 300, 1, 5120, 2048),
                                          ("gemm", 512, 1, 2560, 4096), ("gemm", 300, 1, 384, 1024),
                                          ("einsum", 129, 8, 1024, 4096), ("einsum", 256, 4, 1024, 2048),
                                          ("einsum", 700, 2, 1024, 1024), ("einsum", 97, 3, 384, 1152),
                                          ("gemm", 200, 1, 5120, 8192), ("gemm", 767, 1, 5120, 1152),
                                          ("einsum", 385, 8, 1024, 4096), ("gemm", 1100, 1, 640, 2048),
                                          ("einsum", 130, 5, 640, 640), ("gemm", 1100, 1, 5120, 1152),
                                          ("gemm", 130, 1, 256, 4096),
                                          # either side of each switch of the plan on the o_proj shapes:
                                          # split-K kernel | 128 x 128 tiles | 256 x 256 tiles
                                          ("gemm", 128, 1, 5120, 8192), ("gemm", 129, 1, 5120, 8192),
                                          ("einsum", 512, 8, 1024, 4096), ("einsum", 513, 8, 1024, 4096),
                                          ("gemm", 768, 1, 5120, 8192), ("gemm", 769, 1, 5120, 8192)])
def test_mid_range_shapes_bitexact(lib, kind, M, G, N, K):
    """65 to about 1000 tokens: the split-K streaming kernel (up to 128 tokens, and up to 256 on small grids),
    128-token rows
    of 128- and 64-wide weight tiles (while the 256 x 256 grid would cover at most a quarter of the CUs),
    256-token rows of 256- and 128-wide tiles above; ragged token counts, K ranges that are not multiples of
    four steps, weight counts that are odd multiples of 128: bit-exact against the oracle in the exact regime
    in each combine mode, for every output form; counters return to zero."""
    _modes_bitexact(lib, kind, M, G, N, K, 9300 + M + N)


# --------------------------------------------------------------------------- configs

class Case:
    """Inputs, weights (GPU-quantized and oracle-quantized) for one chain configuration."""

    def __init__(self, shape, seed, outlier_rate, lib):
        print(f"case M={shape.M} G={shape.G} K={shape.K} N={shape.N} P={shape.P} seed={seed}", flush=True)
        self.shape = shape
        inp = si.chain_inputs(shape, seed, outlier_rate)
        self.x_bits = inp["x"]
        G, N, K = shape.G, shape.N, shape.K
        # GPU path: the library's quantizer prepares the weights
        self.wa_q, self.wa_sf = lib.quantize_weight(bf16_to_dev(inp["wo_a"]))
        self.wb_q, self.wb_sf = lib.quantize_weight(bf16_to_dev(inp["wo_b"]))
        # oracle path: its own quantizer
        self.o_w = cr.quantize_weights(inp["wo_a"], inp["wo_b"])
        self.x = bf16_to_dev(self.x_bits)
        torch.cuda.synchronize()

    def oracle(self, rows=None):
        if rows is None:
            return cr.o_proj_chain(self.x_bits, *self.o_w)
        return cr.o_proj_chain_rows(self.x_bits, *self.o_w, rows=rows)


_cases = {}


def get_case(name, lib):
    if name not in _cases:
        if name == "ragged":
            c = si.CHAIN_CONFIGS["decode"]
            _cases[name] = Case(si.ChainShape(300, 8, 4096, 1024, 5120), c.seed, c.outlier_rate, lib)
        else:
            c = si.CHAIN_CONFIGS[name]
            _cases[name] = Case(c.shape, c.seed, c.outlier_rate, lib)
    return _cases[name]


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_weights_quantized_on_gpu_match_oracle(lib, name):
    c = get_case(name, lib)
    wa_q, wa_sf, wb_q, wb_sf = c.o_w
    assert np.array_equal(to_np(c.wa_q), wa_q) and np.array_equal(to_np(c.wa_sf), wa_sf)
    assert np.array_equal(to_np(c.wb_q), wb_q) and np.array_equal(to_np(c.wb_sf), wb_sf)


def check_z_against_oracle(z_q, z_sf, z_b, ref):
    """z codes within 1 ulp on >= 99.9%; scale mismatches only at threshold-straddling block maxima."""
    gq, gsf, gb = to_np(z_q), to_np(z_sf), to_np(z_b)
    d = mx_ulp_distance(gq, gsf, ref.z_q, ref.z_sf)
    frac_ok = np.mean(d <= 1)
    gs, os_ = mx.unpack_scales(gsf), mx.unpack_scales(ref.z_sf)
    bad = np.argwhere(gs != os_)
    for r, b in bad:
        amax = np.max(np.abs(ref.z64[r, 32 * b:32 * b + 32]))
        k = min(int(gs[r, b]), int(os_[r, b])) - 127
        thr = 448.0 * 2.0 ** k
        assert abs(int(gs[r, b]) - int(os_[r, b])) == 1
        assert abs(amax - thr) <= thr * 2.0 ** -7, (r, b, amax, thr)
    print(f"z: {frac_ok * 100:.4f}% within 1 ulp, {len(bad)} of {gs.size} scales differ (threshold cases)",
          flush=True)
    assert frac_ok >= 0.999
    # BF16 z against float64 z: one BF16 rounding plus fp32 accumulation error
    zg = mx.bf16_decode(gb)
    rms = np.sqrt(np.mean(ref.z64 ** 2, axis=1, keepdims=True))
    err = np.abs(zg - ref.z64) - np.abs(ref.z64) * 2.0 ** -8
    assert np.all(err <= 1e-3 * rms)


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_einsum_vs_oracle(lib, name):
    c = get_case(name, lib)
    ref = c.oracle()
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="both")
    check_z_against_oracle(z_q, z_sf, z_b, ref)


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_fused_z_equals_quantized_own_bf16(lib, name):
    c = get_case(name, lib)
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="both")
    oq, osf = mx.quantize(to_np(z_b))
    assert np.array_equal(to_np(z_q), oq) and np.array_equal(to_np(z_sf), osf)
    gq, gsf = lib.mxfp8_quantize(z_b)                       # the consumer's own quantizer on the device
    assert torch.equal(gq, z_q) and torch.equal(gsf, z_sf)
    # output mode does not change the accumulation
    z_q2, z_sf2 = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="mxfp8")
    z_b2 = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="bf16")
    assert torch.equal(z_q2, z_q) and torch.equal(z_sf2, z_sf) and torch.equal(z_b2, z_b)


@pytest.mark.parametrize("name,M", [("tiny", None), ("decode", None), ("ragged", None), ("ragged", 1),
                                    ("ragged", 7), ("ragged", 32)])
def test_prequantized_x_equals_in_kernel_quantization(lib, name, M):
    """Holds on every kernel: the split-K streaming kernel and (up to 32 tokens at the decode depths) the
    whole-K kernel quantize BF16 in their load path; before the tile kernel (many tokens) and the whole-K
    kernel at other depths the quantizer runs into the workspace."""
    c = get_case(name, lib)
    x = c.x if M is None else c.x[:M]
    xq, xsf = lib.mxfp8_quantize(x)
    a = lib.grouped_fp8_einsum(x, None, c.wa_q, c.wa_sf, out="both")
    b = lib.grouped_fp8_einsum(xq, xsf, c.wa_q, c.wa_sf, out="both")
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # same for the GEMM's activation operand
    z_b = a[2]
    zq, zsf = lib.mxfp8_quantize(z_b)
    assert torch.equal(lib.fp8_gemm_nt(z_b, None, c.wb_q, c.wb_sf), lib.fp8_gemm_nt(zq, zsf, c.wb_q, c.wb_sf))


@pytest.mark.parametrize("M", [1, 5, 8, 9, 16, 17, 31, 32])
@pytest.mark.parametrize("kind,G,N,K", [("einsum", 8, 1024, 4096), ("gemm", 1, 5120, 8192), ("einsum", 4, 1024, 8192)])
def test_whole_k_bf16_activations_equal_prequantized(lib, kind, M, G, N, K):
    """Up to 16 tokens on the decode depths (K of 32 or 64 steps) the whole-K kernel quantizes BF16
    activations in its load path (no workspace, no separate launch); from 17 to 32 the quantizer runs into
    the workspace first.  Either way every output is bit-identical to the same call on pre-quantized
    activations, for every row-group size and ragged token count; BF16 storage past row M is NaN and never
    read."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(9500 + M + K)
    xf = rng.standard_normal((M, G * K)).astype(np.float32)
    xf[rng.random(xf.shape) < 1e-3] *= 100.0
    x = _nan_padded(M, torch.from_numpy(xf).to(torch.bfloat16).to(dev()), 0x7FC0)
    wq, wsf = exact_operands(rng, G * N, K)
    xq, xsf = lib.mxfp8_quantize(x)
    if kind == "gemm":
        assert (B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_BF16, M, N, K) == 0) == (M <= 16)
        w_t, wsf_t = u8_to_dev(wq), i32_to_dev(wsf)
        assert torch.equal(lib.fp8_gemm_nt(x, None, w_t, wsf_t), lib.fp8_gemm_nt(xq, xsf, w_t, wsf_t))
        return
    assert (B.lib().grouped_fp8_einsum_workspace_size(B.MXFP8_ACT_BF16, M, G, K, N) == 0) == (M <= 16)
    w_t, wsf_t = u8_to_dev(wq.reshape(G, N, K)), i32_to_dev(wsf.reshape(G, N, K // 128))
    a = lib.grouped_fp8_einsum(x, None, w_t, wsf_t, out="both")
    b = lib.grouped_fp8_einsum(xq, xsf, w_t, wsf_t, out="both")
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    zq, zsf = lib.grouped_fp8_einsum(x, None, w_t, wsf_t, out="mxfp8")
    assert torch.equal(zq, a[0]) and torch.equal(zsf, a[1])


def check_out_against_oracle(c, out, z_q, z_sf, ref, label=""):
    """Chain output: max |out - out64| / RMS(row) <= 2e-2 on every row.  The statistics (max, p99.9, rows over
    the bar) and, as a diagnostic only, how far the z code flips propagate through |wo_b| are printed first."""
    o = mx.bf16_decode(to_np(out))
    rms = np.sqrt(np.mean(ref.out64 ** 2, axis=1, keepdims=True))
    err = np.abs(o - ref.out64)
    rel = np.max(err / np.maximum(rms, 1e-30), axis=1)
    dz = np.abs(mx.dequantize(to_np(z_q), to_np(z_sf)) - mx.dequantize(ref.z_q, ref.z_sf))
    wb = np.abs(mx.dequantize(c.o_w[2], c.o_w[3]))
    prop = dz @ wb.T
    print(f"out {label}: {len(rel)} rows, max |err|/RMS {rel.max():.5f}, p99.9 {np.quantile(rel, 0.999):.5f}, "
          f"median {np.median(rel):.5f}; rows above {OUT_TOL}: {int(np.sum(rel > OUT_TOL))}; "
          f"max z-flip propagation / RMS {np.max(prop / rms):.5f}", flush=True)
    assert rel.max() <= OUT_TOL, (label, float(rel.max()), int(np.argmax(rel)))


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_gemm_stage_on_oracle_z(lib, name):
    """wo_b alone, on the oracle's own MXFP8 z: max |err| / row RMS <= 2e-2."""
    c = get_case(name, lib)
    ref = c.oracle()
    out = lib.fp8_gemm_nt(u8_to_dev(ref.z_q), i32_to_dev(ref.z_sf), c.wb_q, c.wb_sf)
    rel = row_rel_err(to_np(out), ref.out64)
    print(f"wo_b on oracle z: max |err|/RMS {rel.max():.4f}", flush=True)
    assert rel.max() <= OUT_TOL


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_chain_vs_oracle_and_modes_identical(lib, name):
    c = get_case(name, lib)
    ref = c.oracle()
    outs = {m: lib.o_proj_chain(c.x, c.wa_q, c.wa_sf, c.wb_q, c.wb_sf, mode=m) for m in lib.CHAIN_MODES}
    again = lib.o_proj_chain(c.x, c.wa_q, c.wa_sf, c.wb_q, c.wb_sf, mode="chain")
    assert torch.equal(outs["chain"], again)                 # deterministic
    for m in lib.CHAIN_MODES:
        assert torch.equal(outs[m], outs["chain"]), m
    z_q, z_sf = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="mxfp8")
    check_out_against_oracle(c, outs["chain"], z_q, z_sf, ref, name)


@pytest.mark.parametrize("M", [1, 7, 33, 129, 300])
def test_ragged_token_counts(lib, M):
    c = get_case("ragged", lib)
    x = c.x[:M]
    out = lib.o_proj_chain(x, c.wa_q, c.wa_sf, c.wb_q, c.wb_sf, mode="chain")
    rows = list(range(M))
    ref = cr.o_proj_chain_rows(c.x_bits, *c.o_w, rows=rows)
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(x, None, c.wa_q, c.wa_sf, out="both")
    check_z_against_oracle(z_q, z_sf, z_b, ref)
    check_out_against_oracle(c, out, z_q, z_sf, ref, f"ragged M={M}")
    # rows are independent: the first M rows of the 300-row batch agree with the M-row call to within the
    # accumulation order (different token counts take different kernels: 300 rows the tile kernel, up to
    # 32 the whole-K kernel, in between the split-K one)
    full = lib.o_proj_chain(c.x, c.wa_q, c.wa_sf, c.wb_q, c.wb_sf, mode="chain")
    assert row_rel_err(to_np(out), mx.bf16_decode(to_np(full[:M])).astype(np.float64)).max() <= OUT_TOL


def test_outputs_respect_strides_and_guards(lib):
    c = get_case("tiny", lib)
    M, G, N = c.shape.M, c.shape.G, c.shape.N
    zq = torch.full((M, G * N + 32), 0xA5, dtype=torch.uint8, device=dev())
    zsf = torch.full((M, G * N // 128 + 2), 0x5A5A5A5A, dtype=torch.int32, device=dev())
    zb = torch.zeros((M, G * N + 24), dtype=torch.bfloat16, device=dev())
    zb[:, G * N:] = 7.0
    lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="both", z_q=zq[:, :G * N], z_sf=zsf[:, :G * N // 128],
                           z_bf16=zb[:, :G * N])
    a_q, a_sf, a_b = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="both")
    assert torch.equal(zq[:, :G * N], a_q) and torch.equal(zsf[:, :G * N // 128], a_sf)
    assert torch.equal(zb[:, :G * N], a_b)
    assert bool((zq[:, G * N:] == 0xA5).all()) and bool((zsf[:, G * N // 128:] == 0x5A5A5A5A).all())
    assert bool((zb[:, G * N:] == 7.0).all())


# The chain over the 20 token counts the benchmark sweeps (1-256 decode, 384, 512-32768 prefill), as
# prefixes of the long configuration's x (BF16 N(0, 1) with 0.1% of entries x100).
SWEEP_SIZES = (1, 2, 4, 8, 16, 32, 64, 128, 192, 256, 384, 512, 768, 1024, 2048, 4096, 8192, 16384, 24576, 32768)


def test_chain_modes_bitwise_identical_at_sweep_sizes(lib):
    """vLLM PR #60118, Validation: the fused and unfused chains give bitwise identical outputs at every size
    measured.  At each of the 20 sizes the three arrangements -- standalone quantize + einsum with MXFP8
    epilogue + GEMM, the einsum on BF16 x (x_fused), and the einsum writing BF16 z re-quantized by a
    separate launch (unfused) -- give the same output bytes, and the fused z equals the quantizer applied to
    the same kernel's BF16 z (PR #60118, Tests).  Sixteen sampled rows of each size also meet the output bar
    against the oracle."""
    c = get_case("long", lib)
    rng = np.random.default_rng(60118)
    for M in SWEEP_SIZES:
        x = c.x[:M]
        outs = {m: lib.o_proj_chain(x, c.wa_q, c.wa_sf, c.wb_q, c.wb_sf, mode=m) for m in lib.CHAIN_MODES}
        for m in lib.CHAIN_MODES:
            assert torch.equal(outs[m], outs["chain"]), (M, m)
        z_q, z_sf, z_b = lib.grouped_fp8_einsum(x, None, c.wa_q, c.wa_sf, out="both")
        q2, s2 = lib.mxfp8_quantize(z_b)
        assert torch.equal(q2, z_q) and torch.equal(s2, z_sf), M
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 14), replace=False)]))
        ref = c.oracle(rows)
        idx = torch.from_numpy(rows).to(dev())
        check_out_against_oracle(c, outs["chain"][idx], z_q[idx], z_sf[idx], ref, f"sweep M={M}")
        del outs, z_q, z_sf, z_b, q2, s2
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 129, 8193])
def test_fused_z_identity_under_graph_replay(lib, M):
    """vLLM PR #60118, Tests: at 1, 129 and 8193 tokens, with the einsum and wo_b captured in a HIP graph and
    replayed, the FP8 data and scales the einsum's epilogue writes are byte-identical to what wo_b's own
    quantization of the BF16 z gives, and the chain's output equals wo_b run on that BF16 z.  Every replay
    (three, with eager work between them) equals the eager result."""
    c = get_case("long", lib)
    x = c.x[:M].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def body():
        z_q, z_sf, z_b = lib.grouped_fp8_einsum(x, None, c.wa_q, c.wa_sf, out="both", stream=s)
        out = lib.fp8_gemm_nt(z_q, z_sf, c.wb_q, c.wb_sf, stream=s)
        out_b = lib.fp8_gemm_nt(z_b, None, c.wb_q, c.wb_sf, stream=s)      # wo_b quantizing the BF16 z itself
        q_b, sf_b = lib.mxfp8_quantize(z_b, stream=s)
        return z_q, z_sf, z_b, out, out_b, q_b, sf_b

    with torch.cuda.stream(s):
        eager = [t.clone() for t in body()]                # also sizes the stream's workspace before capture
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        static = body()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in static:
            t.zero_()
        s.wait_stream(torch.cuda.current_stream())         # the fills come before the replay
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        z_q, z_sf, z_b, out, out_b, q_b, sf_b = static
        assert torch.equal(z_q, q_b) and torch.equal(z_sf, sf_b), (M, rep)
        assert torch.equal(out, out_b), (M, rep)
        for a, b in zip(static, eager):
            assert torch.equal(a, b), (M, rep)
        lib.o_proj_chain(c.x[:M], c.wa_q, c.wa_sf, c.wb_q, c.wb_sf)     # eager work between replays
        torch.cuda.synchronize()
    oq, osf = mx.quantize(to_np(z_b))                          # and the oracle's quantizer agrees
    assert np.array_equal(to_np(z_q), oq) and np.array_equal(to_np(z_sf), osf)
    del g


@pytest.mark.parametrize("name", ["prefill", "long"])
def test_large_configs_against_oracle(lib, name):
    """Prefill: every one of the 4096 rows against the oracle.  Long: a seeded sample of 2048 rows plus the
    first and last 128 (the oracle's float64 x for all 32768 rows would take 8.6 GB)."""
    c = get_case(name, lib)
    M = c.shape.M
    out = lib.o_proj_chain(c.x, c.wa_q, c.wa_sf, c.wb_q, c.wb_sf, mode="chain")
    z_q, z_sf, z_b = lib.grouped_fp8_einsum(c.x, None, c.wa_q, c.wa_sf, out="both")
    if name == "prefill":
        rows = np.arange(M)
    else:
        rng = np.random.default_rng(20260004)
        rows = np.unique(np.concatenate([np.arange(128), np.arange(M - 128, M),
                                         rng.choice(np.arange(128, M - 128), 2048, replace=False)]))
    print(f"{name}: oracle on {len(rows)} rows of {M}", flush=True)
    ref = c.oracle(rows)
    idx = torch.from_numpy(rows).to(dev())
    check_z_against_oracle(z_q[idx], z_sf[idx], z_b[idx], ref)
    check_out_against_oracle(c, out[idx], z_q[idx], z_sf[idx], ref, name)
    out_oz = lib.fp8_gemm_nt(u8_to_dev(ref.z_q), i32_to_dev(ref.z_sf), c.wb_q, c.wb_sf)
    assert row_rel_err(to_np(out_oz), ref.out64).max() <= OUT_TOL
    # invariants at full size
    zq2, zsf2 = lib.mxfp8_quantize(z_b)
    assert torch.equal(zq2, z_q) and torch.equal(zsf2, z_sf)
    del c.x
    _cases.pop(name)


def test_bf16_staging_keeps_split_k_counters(lib):
    """A BF16 call with many tokens (quantized into the workspace first) leaves the split-K counter region of a
    shared workspace untouched, so a following decode-size split-K call on the same workspace stays exact."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(93)
    Q, BF = B.MXFP8_ACT_MXFP8, B.MXFP8_ACT_BF16
    need = max(B.lib().fp8_gemm_nt_workspace_size(BF, 300, 256, 2048),
               B.lib().fp8_gemm_nt_workspace_size(Q, 48, 256, 4096))
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    vals = rng.choice(EXACT_VALUES, size=(300, 2048)).astype(np.float32)
    a_bf = bf16_to_dev(mx.bf16_round(vals))
    bq, bsf = exact_operands(rng, 256, 2048)
    lib.fp8_gemm_nt(a_bf, None, u8_to_dev(bq), i32_to_dev(bsf), workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0
    aq, asf = exact_operands(rng, 48, 4096)
    cq, csf = exact_operands(rng, 256, 4096)
    d = lib.fp8_gemm_nt(u8_to_dev(aq), i32_to_dev(asf), u8_to_dev(cq), i32_to_dev(csf), workspace=ws)
    assert np.array_equal(to_np(d), mx.bf16_round(cr.gemm_nt(aq, asf, cq, csf)))


def test_shared_workspace_across_shapes(lib):
    """One workspace reused by einsum and GEMM calls of different shapes keeps every result exact."""
    from mxfp8_activation_quantization_amd import binding as B
    rng = np.random.default_rng(91)
    shapes = [(129, 8, 4096, 1024, 5120), (64, 8, 4096, 1024, 5120), (200, 2, 2048, 256, 640)]
    need = max(max(B.lib().grouped_fp8_einsum_workspace_size(B.MXFP8_ACT_MXFP8, M, G, K, N),
                   B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, M, P, G * N)) for M, G, K, N, P in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    for rep in range(2):
        for M, G, K, N, P in shapes:
            xq, xsf = exact_operands(rng, M, G * K)
            wq, wsf = exact_operands(rng, G * N, K)
            bq, bsf = exact_operands(rng, P, G * N)
            zb = lib.grouped_fp8_einsum(u8_to_dev(xq), i32_to_dev(xsf), u8_to_dev(wq.reshape(G, N, K)),
                                        i32_to_dev(wsf.reshape(G, N, K // 128)), out="bf16", workspace=ws)
            z64 = cr.grouped_einsum(xq, xsf, wq.reshape(G, N, K), wsf.reshape(G, N, K // 128), G, K, N)
            assert np.array_equal(to_np(zb), mx.bf16_round(z64)), (rep, M)
            zq = rng.choice(SMALL_CODES, size=(M, G * N))
            zsf = mx.pack_scales(rng.integers(126, 129, size=(M, G * N // 32)).astype(np.uint8))
            d = lib.fp8_gemm_nt(u8_to_dev(zq), i32_to_dev(zsf), u8_to_dev(bq), i32_to_dev(bsf), workspace=ws)
            assert np.array_equal(to_np(d), mx.bf16_round(cr.gemm_nt(zq, zsf, bq, bsf))), (rep, M)
    torch.cuda.synchronize()
    assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("M,mode", [(1, "x_fused"), (8, "x_fused"), (24, "chain"), (64, "chain"), (64, "unfused"),
                                    (128, "chain"), (300, "chain")])
def test_graph_replays_equal_eager(lib, M, mode):
    """The chain captured in a HIP graph on its own stream, as the benchmark times it, gives the eager result
    on every replay: three replays with eager chain calls on other inputs and host synchronizations between
    them, then a replay after new contents are copied into the captured input.  The token counts take every
    kernel of the path (load-path quantization, whole-K, split-K with its arrival counters, tiles); the
    split-K counters must be back at zero after the replays for the next replay to be exact."""
    c = get_case("ragged", lib)
    args = (c.wa_q, c.wa_sf, c.wb_q, c.wb_sf)
    x_static = c.x[:M].clone()
    other = torch.flip(c.x, [0])[:M].contiguous()
    eager = lib.o_proj_chain(x_static, *args, mode=mode)
    eager_other = lib.o_proj_chain(other, *args, mode=mode)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.o_proj_chain(x_static, *args, mode=mode, stream=s)       # the stream's workspace, before capture
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out_static = lib.o_proj_chain(x_static, *args, mode=mode, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        out_static.fill_(7.0)
        s.wait_stream(torch.cuda.current_stream())         # the fill comes before the replay
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static, eager), (M, mode, rep)
        assert torch.equal(lib.o_proj_chain(other, *args, mode=mode), eager_other), (M, mode, rep)
        torch.cuda.synchronize()
    x_static.copy_(other)
    s.wait_stream(torch.cuda.current_stream())             # the new input is in place before the replay
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out_static, eager_other), (M, mode)
    from mxfp8_activation_quantization_amd import binding as B
    for ws in B._workspaces.values():
        assert int(ws[:65536].view(torch.int32).abs().sum()) == 0


def test_graph_survives_workspace_growth(lib):
    """A chain captured at 64 tokens (split-K wo_b: counters and partials in the stream's workspace) still
    replays to the eager result after a larger call on the same stream has grown that stream's workspace and
    other allocations have been made: the outgrown workspace the graph writes into stays allocated."""
    from mxfp8_activation_quantization_amd import binding as B
    c = get_case("ragged", lib)
    args = (c.wa_q, c.wa_sf, c.wb_q, c.wb_sf)
    x_static = c.x[:64].clone()
    eager = lib.o_proj_chain(x_static, *args)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.o_proj_chain(x_static, *args, stream=s)
    s.synchronize()
    key = (dev().index or 0, s.cuda_stream)
    ws_before = B._workspaces[key]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out_static = lib.o_proj_chain(x_static, *args, stream=s)
    torch.cuda.synchronize()
    # a BF16 GEMM with many tokens stages its activations in the workspace: more bytes than split-K needs
    big = torch.randn(2048, 8192, device=dev()).to(torch.bfloat16)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.fp8_gemm_nt(big, None, c.wb_q, c.wb_sf, stream=s)
    s.synchronize()
    assert B._workspaces[key].data_ptr() != ws_before.data_ptr()     # the workspace did grow
    junk = [torch.full((1 << 20,), 0x7F, dtype=torch.uint8, device=dev()) for _ in range(16)]
    for rep in range(2):
        out_static.fill_(7.0)
        s.wait_stream(torch.cuda.current_stream())         # the fill comes before the replay
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_static, eager), rep
    assert all(bool((j == 0x7F).all()) for j in junk)


def test_capture_on_a_cold_stream_raises(lib):
    """A split-K call captured on a stream that has no workspace yet raises a clear error instead of capturing
    a zero fill whose counters would stay undefined until the first replay; after one eager call on the
    stream the same capture works."""
    c = get_case("ragged", lib)
    args = (c.wa_q, c.wa_sf, c.wb_q, c.wb_sf)
    x_static = c.x[:64].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="workspace"):
        with torch.cuda.graph(g, stream=s):
            lib.o_proj_chain(x_static, *args, stream=s)
    del g
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        eager = lib.o_proj_chain(x_static, *args, stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        out = lib.o_proj_chain(x_static, *args, stream=s)
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager)


def test_outgrown_workspaces_are_released_unless_captured(lib):
    """Growing a stream's workspace releases the old buffer when no graph captured it, so a sweep of growing
    shapes holds one buffer per stream; a captured buffer is retained until release_retained_workspaces()."""
    from mxfp8_activation_quantization_amd import binding as B
    c = get_case("ragged", lib)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    key = (dev().index or 0, s.cuda_stream)
    n0 = len(B._retained)
    with torch.cuda.stream(s):
        for M in (17, 64, 100, 300):                           # staged BF16 activations: growing workspaces
            lib.fp8_gemm_nt(c.x[:M, :8192], None, c.wb_q, c.wb_sf, stream=s)
    s.synchronize()
    assert len(B._retained) == n0
    assert B._workspaces[key].numel() >= B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_BF16, 300, 5120, 8192)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lib.fp8_gemm_nt(c.x[:64, :8192], None, c.wb_q, c.wb_sf, stream=s)
    torch.cuda.synchronize()
    big = torch.randn(1024, 8192, device=dev()).to(torch.bfloat16)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lib.fp8_gemm_nt(big, None, c.wb_q, c.wb_sf, stream=s)      # grows past the captured buffer
    s.synchronize()
    assert len(B._retained) == n0 + 1
    with torch.cuda.stream(s):
        g.replay()
    torch.cuda.synchronize()
    del g
    assert lib.release_retained_workspaces() >= 1
    assert len(B._retained) == 0
