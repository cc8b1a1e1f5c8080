"""fp8_gemm_nt_noalloc (the entry point for callers that cannot allocate) against fp8_gemm_nt: the same
kernels with the library's fixed per-GPU scratch in place of the workspace, so every output must be identical
bit for bit.  Two calls in a row on each path, the second with fewer tokens (the scratch keeps the first
call's contents); the split-K counters must be usable again by the next call."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_common import dev, i32_to_dev, to_np, u8_to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import mxfp8_activation_quantization_amd as m
    from mxfp8_activation_quantization_amd import binding
    m.device_check()
    return binding


def random_mxfp8(rng, rows, cols):
    q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 1                                   # no NaN codes
    sb = rng.integers(118, 128, size=(rows, cols // 32)).astype(np.uint8)
    return q, np.ascontiguousarray(sb).view(np.int32).reshape(rows, cols // 128)


def noalloc_call(B, a, a_sf, b, b_sf, d, stream=None):
    """The C entry point itself, through ctypes (no workspace argument exists)."""
    kind = B.MXFP8_ACT_BF16 if a.dtype == torch.bfloat16 else B.MXFP8_ACT_MXFP8
    sp = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    return B.lib().fp8_gemm_nt_noalloc(kind, a.data_ptr(), a.stride(0), a_sf.data_ptr() if a_sf is not None else None,
                                       a_sf.stride(0) if a_sf is not None else 0, a.shape[0], b.shape[0],
                                       b.shape[1], b.data_ptr(), b_sf.data_ptr(), d.data_ptr(), d.stride(0), sp)


@pytest.mark.parametrize("N,K,Ms", [(5120, 8192, (64, 33)),      # decode wo_b: split-K partials in the scratch
                                    (256, 4096, (48, 5)),        # narrow weight: split K at every token count
                                    (5120, 8192, (300, 129))])   # tile kernels: no scratch needed
def test_noalloc_equals_workspace_path_mxfp8(B, N, K, Ms):
    rng = np.random.default_rng(700 + N + K)
    bq, bsf = random_mxfp8(rng, N, K)
    b_t, bsf_t = u8_to_dev(bq), i32_to_dev(bsf)
    aq, asf = random_mxfp8(rng, max(Ms), K)
    for M in Ms:                                                 # two calls in a row, the second smaller
        a_t, asf_t = u8_to_dev(aq[:M]), i32_to_dev(asf[:M])
        ref = B.fp8_gemm_nt(a_t, asf_t, b_t, bsf_t)
        d = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev())
        assert noalloc_call(B, a_t, asf_t, b_t, bsf_t, d) == B.MXFP8_OK
        torch.cuda.synchronize()
        assert torch.equal(d, ref), (N, K, M)


def test_noalloc_equals_workspace_path_bf16(B):
    """BF16 activations: quantized into the scratch first (the tile and whole-K kernels read MXFP8)."""
    rng = np.random.default_rng(71)
    N, K = 5120, 8192
    bq, bsf = random_mxfp8(rng, N, K)
    b_t, bsf_t = u8_to_dev(bq), i32_to_dev(bsf)
    x = torch.from_numpy(rng.standard_normal((300, K)).astype(np.float32)).to(torch.bfloat16).to(dev())
    for M in (300, 100, 20, 8):
        assert B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_BF16, M, N, K) <= B.NOALLOC_SCRATCH_BYTES
        ref = B.fp8_gemm_nt(x[:M], None, b_t, bsf_t)
        d = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        assert noalloc_call(B, x[:M], None, b_t, bsf_t, d) == B.MXFP8_OK
        torch.cuda.synchronize()
        assert torch.equal(d, ref), M


def test_noalloc_rejects_shapes_beyond_its_scratch(B):
    """BF16 activations of 4096 rows at K = 8192 would stage 34 MB: MXFP8_ERR_SCRATCH, nothing written."""
    N, K, M = 256, 8192, 4096
    assert B.lib().fp8_gemm_nt_workspace_size(B.MXFP8_ACT_BF16, M, N, K) > B.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev())
    b_t = torch.zeros((N, K), dtype=torch.uint8, device=dev())
    bsf_t = torch.zeros((N, K // 128), dtype=torch.int32, device=dev())
    d = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=dev())
    assert noalloc_call(B, x, None, b_t, bsf_t, d) == B.MXFP8_ERR_SCRATCH
    assert "scratch" in B.lib().mxfp8_status_string(B.MXFP8_ERR_SCRATCH).decode()
    with pytest.raises(ValueError):
        B.fp8_gemm_nt_noalloc(x, None, b_t, bsf_t, d)
    torch.cuda.synchronize()
    assert bool((d == 7.0).all())


def test_noalloc_under_graph_capture_on_a_fresh_stream(B):
    """Captured on a stream that has never run it (no workspace to size first): replays equal the eager
    result, with eager calls of another size between them."""
    rng = np.random.default_rng(72)
    N, K = 5120, 8192
    bq, bsf = random_mxfp8(rng, N, K)
    b_t, bsf_t = u8_to_dev(bq), i32_to_dev(bsf)
    aq, asf = random_mxfp8(rng, 64, K)
    a_t, asf_t = u8_to_dev(aq), i32_to_dev(asf)
    ref = B.fp8_gemm_nt(a_t, asf_t, b_t, bsf_t)
    other = B.fp8_gemm_nt(a_t[:40], asf_t[:40], b_t, bsf_t)
    d = torch.empty((64, N), dtype=torch.bfloat16, device=dev())
    d2 = torch.empty((40, N), dtype=torch.bfloat16, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        assert noalloc_call(B, a_t, asf_t, b_t, bsf_t, d, stream=s) == B.MXFP8_OK
    torch.cuda.synchronize()
    for rep in range(3):
        d.fill_(7.0)
        s.wait_stream(torch.cuda.current_stream())         # the fill comes before the replay
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d, ref), rep
        assert noalloc_call(B, a_t[:40], asf_t[:40], b_t, bsf_t, d2) == B.MXFP8_OK
        torch.cuda.synchronize()
        assert torch.equal(d2, other), rep
    del g
