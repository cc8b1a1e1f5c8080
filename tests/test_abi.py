"""Host-side tests of the C ABI (no GPU needed): the built library loads, exports
every function include/mxfp8.h declares, and rejects bad arguments with the
documented status codes before any HIP call.

Pointers below are fake addresses: validation never dereferences them, and on
a host without a gfx950 the only call that reaches HIP is the device check.
"""
import ctypes
import os
import re

import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))

mx = pytest.importorskip("mxfp8_activation_quantization_amd",
                         reason="libmxfp8.so is not built (run the build first)")
from mxfp8_activation_quantization_amd import binding as B  # noqa: E402

LIB = B.lib()
HAVE_GPU = torch.cuda.is_available()


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_chain_entry_points():
    names = declared_functions()
    for n in ("mxfp8_quantize", "grouped_fp8_einsum", "fp8_gemm_nt", "mxfp8_status_string",
              "mxfp8_device_check", "mxfp8_version", "mxfp8_rmsnorm_quantize"):
        assert n in names


def test_library_exports_every_declared_symbol():
    assert len(HEADERS) >= 2
    for n in declared_functions():
        assert hasattr(LIB, n), n
        assert n in B.SIGNATURES, n


def test_product_header_has_no_global_state_setter():
    """The product ABI keeps no mutable global state: the split-K combine is a per-call argument of the
    test-only entry points (include/mxfp8_testing.h), not a process-wide switch."""
    product = declared_functions([os.path.join(INCLUDE, "mxfp8.h")])
    assert not any("set_" in n for n in product)
    assert not hasattr(LIB, "mxfp8_set_splitk_mode")
    testing = declared_functions([os.path.join(INCLUDE, "mxfp8_testing.h")])
    assert testing == ["mxfp8_testing_fp8_gemm_nt", "mxfp8_testing_grouped_fp8_einsum"]


def test_status_strings():
    for s in range(8):
        assert LIB.mxfp8_status_string(s)
    assert LIB.mxfp8_status_string(99) == b"unknown status"
    assert LIB.mxfp8_version() >= 100


@pytest.mark.skipif(HAVE_GPU, reason="a GPU is present")
def test_device_check_without_gpu():
    assert LIB.mxfp8_device_check() == B.MXFP8_ERR_DEVICE


# fake, well-aligned addresses far apart
X, Q, SF, W, WSF, Z, ZSF, ZB, D = (0x10000000 * (i + 1) for i in range(9))


def quant(M=4, K=256, ld_x=None, ld_q=None, ld_sf=None, x=X, q=Q, sf=SF):
    return LIB.mxfp8_quantize(x, M, K, ld_x or K, q, ld_q or K, sf, ld_sf or K // 128, None)


def test_quantize_argument_errors():
    assert quant(M=-1) == B.MXFP8_ERR_SHAPE
    assert quant(K=0) == B.MXFP8_ERR_SHAPE
    assert quant(K=96) == B.MXFP8_ERR_SHAPE
    assert quant(ld_x=200) == B.MXFP8_ERR_SHAPE
    assert quant(ld_sf=1) == B.MXFP8_ERR_SHAPE
    assert quant(ld_x=260) == B.MXFP8_ERR_ALIGN           # 520-byte rows break 16-byte alignment
    assert quant(ld_q=264) == B.MXFP8_ERR_ALIGN
    assert quant(x=None) == B.MXFP8_ERR_NULL
    assert quant(sf=None) == B.MXFP8_ERR_NULL
    assert quant(x=X + 8) == B.MXFP8_ERR_ALIGN
    assert quant(sf=SF + 2) == B.MXFP8_ERR_ALIGN
    assert quant(q=X + 512) == B.MXFP8_ERR_ALIAS          # codes written into the input
    assert quant(sf=Q + 64) == B.MXFP8_ERR_ALIAS
    assert quant(M=0, x=None, q=None, sf=None) == B.MXFP8_OK   # empty batch is a no-op


def rms(M=4, K=256, ld_x=None, gamma=W, eps=1e-6, y=None, ld_y=0, q=Q, ld_q=None, sf=SF, ld_sf=None, x=X):
    return LIB.mxfp8_rmsnorm_quantize(x, M, K, ld_x or K, gamma, eps, y, ld_y, q, ld_q or K, sf, ld_sf or K // 128,
                                      None)


def test_rmsnorm_quantize_argument_errors():
    assert rms(M=-1) == B.MXFP8_ERR_SHAPE
    assert rms(K=96) == B.MXFP8_ERR_SHAPE
    assert rms(eps=0.0) == B.MXFP8_ERR_SHAPE                # eps must be positive
    assert rms(eps=-1e-6) == B.MXFP8_ERR_SHAPE
    assert rms(eps=float("nan")) == B.MXFP8_ERR_SHAPE
    assert rms(eps=float("inf")) == B.MXFP8_ERR_SHAPE
    assert rms(ld_x=200) == B.MXFP8_ERR_SHAPE
    assert rms(y=ZB, ld_y=100) == B.MXFP8_ERR_SHAPE
    assert rms(ld_x=260) == B.MXFP8_ERR_ALIGN
    assert rms(gamma=None) == B.MXFP8_ERR_NULL
    assert rms(sf=None) == B.MXFP8_ERR_NULL
    assert rms(gamma=W + 8) == B.MXFP8_ERR_ALIGN
    assert rms(y=ZB + 8, ld_y=256) == B.MXFP8_ERR_ALIGN
    assert rms(q=X + 256) == B.MXFP8_ERR_ALIAS             # codes written into the input
    assert rms(q=W) == B.MXFP8_ERR_ALIAS                   # codes written into gamma
    assert rms(y=Q + 64, ld_y=256) == B.MXFP8_ERR_ALIAS    # BF16 output over the codes
    assert rms(q=None, sf=None) == B.MXFP8_ERR_UNSUPPORTED    # no output at all
    assert rms(q=None) == B.MXFP8_ERR_NULL                     # codes and scales come together
    assert rms(M=0, x=None, gamma=None, q=None, sf=None, y=ZB, ld_y=256) == B.MXFP8_OK


@pytest.mark.skipif(HAVE_GPU, reason="a GPU is present")
def test_valid_rmsnorm_quantize_reports_missing_device():
    assert rms() == B.MXFP8_ERR_DEVICE
    assert rms(y=ZB, ld_y=256) == B.MXFP8_ERR_DEVICE


WS = 0x10000000 * 12


def einsum(kind=B.MXFP8_ACT_MXFP8, M=4, G=2, K=256, N=128, x=X, ld_x=None, x_sf=SF, ld_xsf=None, w=W,
           w_sf=WSF, z=Z, ld_z=None, z_sf=ZSF, ld_zsf=None, zb=None, ld_zb=0, ws=WS, ws_bytes=1 << 30):
    return LIB.grouped_fp8_einsum(kind, x, ld_x or G * K, x_sf, ld_xsf or G * K // 128, M, G, K, N, w, w_sf,
                                  z, ld_z or G * N, z_sf, ld_zsf or G * N // 128, zb, ld_zb, ws, ws_bytes, None)


def test_einsum_argument_errors():
    assert einsum(kind=7) == B.MXFP8_ERR_UNSUPPORTED
    assert einsum(G=0) == B.MXFP8_ERR_SHAPE
    assert einsum(N=96) == B.MXFP8_ERR_SHAPE                    # o_lora_rank % 128 gate
    assert einsum(K=64) == B.MXFP8_ERR_SHAPE
    assert einsum(ld_x=100) == B.MXFP8_ERR_SHAPE
    assert einsum(z=None, z_sf=None, zb=None) == B.MXFP8_ERR_UNSUPPORTED
    assert einsum(z_sf=None) == B.MXFP8_ERR_NULL
    assert einsum(w=None) == B.MXFP8_ERR_NULL
    assert einsum(x_sf=None) == B.MXFP8_ERR_NULL
    assert einsum(ld_z=100) == B.MXFP8_ERR_SHAPE
    assert einsum(ld_z=264) == B.MXFP8_ERR_ALIGN
    assert einsum(w=W + 4) == B.MXFP8_ERR_ALIGN
    assert einsum(z=X) == B.MXFP8_ERR_ALIAS
    assert einsum(z_sf=Z + 16) == B.MXFP8_ERR_ALIAS
    assert einsum(zb=ZSF, ld_zb=256) == B.MXFP8_ERR_ALIAS
    assert einsum(kind=B.MXFP8_ACT_BF16, x_sf=None, ld_x=516) == B.MXFP8_ERR_ALIGN   # 1032-byte rows
    assert einsum(M=0, x=None, z=Z, z_sf=ZSF) == B.MXFP8_OK


@pytest.mark.skipif(HAVE_GPU, reason="a GPU is present")
def test_valid_einsum_reports_missing_device():
    assert einsum() == B.MXFP8_ERR_DEVICE
    assert einsum(kind=B.MXFP8_ACT_BF16, x_sf=None) == B.MXFP8_ERR_DEVICE


def gemm(kind=B.MXFP8_ACT_MXFP8, M=4, N=256, K=256, a=X, ld_a=None, a_sf=SF, ld_asf=None, b=W, b_sf=WSF, d=D,
         ld_d=None, ws=WS, ws_bytes=1 << 30):
    return LIB.fp8_gemm_nt(kind, a, ld_a or K, a_sf, ld_asf or K // 128, M, N, K, b, b_sf, d, ld_d or N, ws, ws_bytes,
                           None)


def test_gemm_argument_errors():
    assert gemm(M=-3) == B.MXFP8_ERR_SHAPE
    assert gemm(N=100) == B.MXFP8_ERR_SHAPE
    assert gemm(ld_d=100) == B.MXFP8_ERR_SHAPE
    assert gemm(ld_d=260) == B.MXFP8_ERR_ALIGN
    assert gemm(d=None) == B.MXFP8_ERR_NULL
    assert gemm(b_sf=None) == B.MXFP8_ERR_NULL
    assert gemm(d=W + 64) == B.MXFP8_ERR_ALIAS
    assert gemm(kind=3) == B.MXFP8_ERR_UNSUPPORTED
    assert gemm(M=0, a=None, d=None) == B.MXFP8_OK


def test_size_limits_of_tile_addressing():
    """256-row tiles are addressed with 32-bit offsets: row strides above 2^23 bytes and K above 2^22 are
    rejected before any launch (the documented limits)."""
    assert gemm(ld_a=(1 << 23) + 16) == B.MXFP8_ERR_SHAPE                   # E4M3 rows, bytes
    assert gemm(kind=B.MXFP8_ACT_BF16, ld_a=(1 << 22) + 8) == B.MXFP8_ERR_SHAPE   # BF16 rows: 2 bytes each
    assert gemm(ld_asf=(1 << 16)) == B.MXFP8_ERR_SHAPE                      # scale rows: 4 bytes per word
    assert gemm(K=(1 << 22) + 128) == B.MXFP8_ERR_SHAPE
    assert einsum(K=(1 << 22) + 128) == B.MXFP8_ERR_SHAPE
    assert LIB.fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, 4, 256, (1 << 22) + 128) == -1
    assert LIB.grouped_fp8_einsum_workspace_size(B.MXFP8_ACT_MXFP8, 4, 2, (1 << 22) + 128, 128) == -1


@pytest.mark.skipif(HAVE_GPU, reason="a GPU is present")
def test_valid_gemm_reports_missing_device():
    assert gemm() == B.MXFP8_ERR_DEVICE


def test_workspace_sizes():
    Q, BF = B.MXFP8_ACT_MXFP8, B.MXFP8_ACT_BF16
    # a K range shorter than two 256-deep super-steps per split is never split (no scratch); deeper K is
    # split across workgroups in the decode range only
    assert LIB.grouped_fp8_einsum_workspace_size(Q, 64, 2, 512, 1024) == 0
    need = LIB.grouped_fp8_einsum_workspace_size(Q, 64, 4, 4096, 1024)
    assert need > 0 and need % 256 == 0
    assert LIB.grouped_fp8_einsum_workspace_size(BF, 64, 4, 4096, 1024) == need   # split K: quantized in the kernel
    assert LIB.fp8_gemm_nt_workspace_size(Q, 64, 5120, 8192) > 0
    # up to 64 tokens on a grid of 256 workgroups of 32 weight rows (wo_a): whole K per workgroup, no scratch;
    # BF16 activations are quantized into the workspace first
    assert LIB.grouped_fp8_einsum_workspace_size(Q, 64, 8, 4096, 1024) == 0
    assert LIB.grouped_fp8_einsum_workspace_size(BF, 64, 8, 4096, 1024) == 65536 + 64 * 32768 + 64 * 1024
    assert LIB.fp8_gemm_nt_workspace_size(Q, 4096, 5120, 8192) == 0        # many tokens: no split
    # many BF16 tokens: the activations are quantized into the workspace first (codes + packed scales),
    # after the counter region that split-K calls sharing the workspace keep
    assert LIB.fp8_gemm_nt_workspace_size(BF, 4096, 5120, 8192) == 65536 + 4096 * 8192 + 4096 * 8192 // 32
    assert LIB.grouped_fp8_einsum_workspace_size(BF, 300, 8, 4096, 1024) >= 300 * 32768 * (1 + 1 / 32)
    assert LIB.fp8_gemm_nt_workspace_size(Q, 0, 5120, 8192) == 0
    # at most 32 tokens on a wide enough weight: one workgroup per 32 weight rows and the whole K range,
    # no split (E4M3: no scratch); BF16 activations are quantized into the workspace first
    assert LIB.fp8_gemm_nt_workspace_size(Q, 32, 5120, 8192) == 0
    assert LIB.grouped_fp8_einsum_workspace_size(Q, 1, 8, 4096, 1024) == 0
    assert LIB.fp8_gemm_nt_workspace_size(Q, 33, 5120, 8192) > 0           # 160 workgroups: split K past 32
    assert LIB.fp8_gemm_nt_workspace_size(Q, 33, 8192, 8192) == 0
    # ... except up to 16 tokens with K of 32 or 64 steps (the decode shapes): quantized in the load path
    assert LIB.fp8_gemm_nt_workspace_size(BF, 1, 5120, 8192) == 0
    assert LIB.grouped_fp8_einsum_workspace_size(BF, 7, 8, 4096, 1024) == 0
    assert LIB.grouped_fp8_einsum_workspace_size(BF, 16, 8, 4096, 1024) == 0
    assert LIB.grouped_fp8_einsum_workspace_size(BF, 17, 8, 4096, 1024) == 65536 + 17 * 32768 + 17 * 1024
    # 65-128 tokens on >= 128 workgroups: whole K, E4M3 activations need nothing, BF16 ones are staged
    assert LIB.fp8_gemm_nt_workspace_size(Q, 128, 5120, 8192) == 0
    assert LIB.grouped_fp8_einsum_workspace_size(Q, 65, 8, 4096, 1024) == 0
    assert LIB.fp8_gemm_nt_workspace_size(BF, 100, 5120, 8192) == 65536 + 100 * 8192 + 100 * 8192 // 32
    assert LIB.fp8_gemm_nt_workspace_size(BF, 16, 4096, 6144) == 65536 + 16 * 6144 + 16 * 6144 // 32   # 48 steps
    # too narrow for the machine (64 workgroups) or K past the scale tables: split K as before
    assert LIB.fp8_gemm_nt_workspace_size(Q, 8, 2048, 8192) > 0
    assert LIB.fp8_gemm_nt_workspace_size(Q, 8, 5120, 8192 + 128) > 0
    assert LIB.grouped_fp8_einsum_workspace_size(Q, 64, 8, 4000, 1024) == -1
    assert LIB.fp8_gemm_nt_workspace_size(Q, 64, 100, 8192) == -1
    assert LIB.fp8_gemm_nt_workspace_size(7, 64, 128, 8192) == -1          # unknown activation kind


def test_workspace_errors():
    need = LIB.fp8_gemm_nt_workspace_size(B.MXFP8_ACT_MXFP8, 4, 256, 4096)
    assert need > 0
    assert gemm(K=4096, ws=None) == B.MXFP8_ERR_WORKSPACE
    assert gemm(K=4096, ws_bytes=need - 1) == B.MXFP8_ERR_WORKSPACE
    assert gemm(K=4096, ws=WS + 128) == B.MXFP8_ERR_WORKSPACE            # 256-byte alignment
    assert gemm(K=4096, ws=D) == B.MXFP8_ERR_ALIAS                        # workspace over the output
    assert einsum(K=4096, ws=X) == B.MXFP8_ERR_ALIAS                      # workspace over the input
    assert gemm(K=512, ws=None, ws_bytes=0) != B.MXFP8_ERR_WORKSPACE      # one K slice: none needed


def test_splitk_combine_argument_of_the_testing_entry_points():
    """Modes 0-2 pass validation (and then need the device); anything else is rejected before any HIP call."""
    def t_gemm(mode, **kw):
        return LIB.mxfp8_testing_fp8_gemm_nt(mode, B.MXFP8_ACT_MXFP8, X, 4096, SF, 32, 4, 256, 4096, W, WSF, D, 256,
                                             WS, 1 << 30, None)

    def t_einsum(mode):
        return LIB.mxfp8_testing_grouped_fp8_einsum(mode, B.MXFP8_ACT_MXFP8, X, 512, SF, 4, 4, 2, 256, 128, W, WSF,
                                                    Z, 256, ZSF, 2, None, 0, WS, 1 << 30, None)

    for f in (t_gemm, t_einsum):
        assert f(3) == B.MXFP8_ERR_UNSUPPORTED
        assert f(-1) == B.MXFP8_ERR_UNSUPPORTED
        if not HAVE_GPU:
            for m in (0, 1, 2):
                assert f(m) == B.MXFP8_ERR_DEVICE
    # an argument error is reported as such whatever the mode
    assert LIB.mxfp8_testing_fp8_gemm_nt(1, B.MXFP8_ACT_MXFP8, X, 4096, SF, 32, 4, 100, 4096, W, WSF, D, 256,
                                         WS, 1 << 30, None) == B.MXFP8_ERR_SHAPE


def test_binding_raises_value_error_on_argument_status():
    with pytest.raises(ValueError):
        B._check(B.MXFP8_ERR_SHAPE, "test")
    with pytest.raises(RuntimeError):
        B._check(B.MXFP8_ERR_DEVICE, "test")
