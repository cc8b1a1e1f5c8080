"""ctypes binding of libmxfp8.so: the C ABI in include/mxfp8.h with torch tensors as containers.

Argument marshalling only: shapes are read off the tensors, outputs are
allocated with torch when the caller does not pass them, and every call goes to
the library on the current torch stream.  All arithmetic happens in the HIP
kernels.  There is no fallback: without the built library the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

MXFP8_OK = 0
MXFP8_ERR_NULL = 1
MXFP8_ERR_SHAPE = 2
MXFP8_ERR_ALIGN = 3
MXFP8_ERR_UNSUPPORTED = 4
MXFP8_ERR_ALIAS = 5
MXFP8_ERR_DEVICE = 6
MXFP8_ERR_LAUNCH = 7
MXFP8_ERR_WORKSPACE = 8
MXFP8_ERR_SCRATCH = 9

MXFP8_ACT_BF16 = 0
MXFP8_ACT_MXFP8 = 1

_ARG_ERRORS = {MXFP8_ERR_NULL, MXFP8_ERR_SHAPE, MXFP8_ERR_ALIGN, MXFP8_ERR_UNSUPPORTED, MXFP8_ERR_ALIAS,
               MXFP8_ERR_WORKSPACE, MXFP8_ERR_SCRATCH}

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p

# C signatures (include/mxfp8.h)
SIGNATURES = {
    "mxfp8_status_string": (ctypes.c_char_p, [c_int]),
    "mxfp8_version": (c_int, []),
    "mxfp8_device_check": (c_int, []),
    "mxfp8_quantize": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "mxfp8_rmsnorm_quantize": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_float, c_vp, c_i64, c_vp, c_i64,
                                       c_vp, c_i64, c_vp]),
    "grouped_fp8_einsum": (c_int, [c_int, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp,
                                   c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "grouped_fp8_einsum_workspace_size": (c_i64, [c_int, c_i64, c_i64, c_i64, c_i64]),
    "fp8_gemm_nt": (c_int, [c_int, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_i64,
                            c_vp, c_i64, c_vp]),
    "fp8_gemm_nt_workspace_size": (c_i64, [c_int, c_i64, c_i64, c_i64]),
    "fp8_gemm_nt_noalloc": (c_int, [c_int, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_i64,
                                    c_vp]),
    # include/mxfp8_testing.h: the same calls with the split-K combine chosen per call
    "mxfp8_testing_grouped_fp8_einsum": (c_int, [c_int, c_int, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64,
                                                 c_vp, c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "mxfp8_testing_fp8_gemm_nt": (c_int, [c_int, c_int, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp,
                                          c_vp, c_i64, c_vp, c_i64, c_vp]),
}


class MXFP8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.mxfp8_status_string(status).decode()} (status {status})")


class MXFP8ArgumentError(MXFP8Error, ValueError):
    pass


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python mxfp8_activation_quantization_amd/build.py` "
            "(there is no CPU or framework fallback)")
    # torch (imported above) has already loaded its HIP runtime; the library binds to the same
    # libamdhip64.so.7 by soname, so torch's streams and device pointers are valid in it.
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _check(status: int, where: str) -> None:
    if status != MXFP8_OK:
        raise (MXFP8ArgumentError if status in _ARG_ERRORS else MXFP8Error)(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _rows(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name}: expected a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")


# Scratch of the GEMM calls (split-K counters and partials, staged activations): one
# zero-filled buffer per (device, stream), grown on demand.  The kernels leave its
# counters at zero, so a buffer is reusable by later calls on the same stream (stream
# order serializes them).  A buffer handed out while its stream was being captured
# into a graph is marked: the graph replays into its address, so when the stream's
# workspace later grows, a marked buffer is kept (in _retained) and an unmarked one is
# released.  A workspace cannot be created or grown during capture (the zero fill would
# only be recorded, leaving the counters undefined until the first replay): warm the
# capture stream with one eager call of the largest shape first, or pass `workspace=`.
_workspaces: dict = {}
_captured: set = set()          # keys of _workspaces whose current buffer a graph holds
_retained: list = []            # outgrown buffers that a captured graph may still use


def _stream_obj(stream_ptr: int):
    cur = torch.cuda.current_stream()
    return cur if cur.cuda_stream == stream_ptr else torch.cuda.ExternalStream(stream_ptr)


def workspace_for(nbytes: int, device: torch.device, stream_ptr: int) -> torch.Tensor | None:
    if nbytes <= 0:
        return None
    key = (device.index if device.index is not None else torch.cuda.current_device(), stream_ptr)
    ws = _workspaces.get(key)
    st = _stream_obj(stream_ptr)
    with torch.cuda.stream(st):
        capturing = torch.cuda.is_current_stream_capturing()
        if ws is None or ws.numel() < nbytes:
            if capturing:
                raise RuntimeError(
                    f"the GEMM needs a {nbytes}-byte workspace on a stream that is being captured, and none of "
                    "that size exists yet; make one eager call of the largest shape on this stream before "
                    "capturing, or pass workspace=")
            if ws is not None and key in _captured:
                _retained.append(ws)
            _captured.discard(key)
            # allocated and zero-filled on the stream its kernels run on: the fill is stream-ordered before
            # them, and the caching allocator reuses a released buffer only in that stream's order
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            _workspaces[key] = ws
    if capturing:
        _captured.add(key)
    return ws


def release_retained_workspaces() -> int:
    """Drops the outgrown workspaces kept for captured graphs; call once those graphs are destroyed.
    Returns how many buffers were released."""
    n = len(_retained)
    _retained.clear()
    return n


def _ws_args(need: int, device, stream_ptr: int, workspace: torch.Tensor | None):
    if need <= 0:
        return None, 0
    ws = workspace if workspace is not None else workspace_for(need, device, stream_ptr)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def device_check() -> None:
    _check(_lib.mxfp8_device_check(), "mxfp8_device_check")


# How the decode kernels combine split-K partials; every mode gives the same bits.  Anything but
# "local" goes through the test-only entry points of include/mxfp8_testing.h.
SPLITK_MODES = {"local": 0, "through": 1, "recompute": 2}


# ----------------------------------------------------------------------------- quantize

def mxfp8_quantize(x: torch.Tensor, q: torch.Tensor | None = None, sf: torch.Tensor | None = None,
                   stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """BF16 [M, K] -> (E4M3 codes uint8 [M, K], packed UE8M0 scales int32 [M, K/128])."""
    _rows(x, torch.bfloat16, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((M, max(K // 128, 1)), dtype=torch.int32, device=x.device)
    _rows(q, torch.uint8, "q")
    _rows(sf, torch.int32, "sf")
    _check(_lib.mxfp8_quantize(_ptr(x), M, K, x.stride(0), _ptr(q), q.stride(0), _ptr(sf), sf.stride(0),
                               _stream(stream)), "mxfp8_quantize")
    return q, sf


def mxfp8_rmsnorm_quantize(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, *, bf16_out: bool = False,
                           mxfp8_out: bool = True, y: torch.Tensor | None = None, q: torch.Tensor | None = None,
                           sf: torch.Tensor | None = None, stream=None):
    """RMSNorm of BF16 rows, leaving as MXFP8: (q uint8 [M, K], sf int32 [M, K/128]); (y, q, sf) with the BF16
    y when bf16_out (or y) is given; y alone with mxfp8_out=False.  gamma: BF16 [K]."""
    _rows(x, torch.bfloat16, "x")
    M, K = x.shape
    if gamma.dtype != torch.bfloat16 or gamma.dim() != 1 or gamma.numel() != K or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous BF16 vector of the row length")
    if y is None and (bf16_out or not mxfp8_out):
        y = torch.empty((M, K), dtype=torch.bfloat16, device=x.device)
    if y is not None:
        _rows(y, torch.bfloat16, "y")
    if mxfp8_out:
        if q is None:
            q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        if sf is None:
            sf = torch.empty((M, max(K // 128, 1)), dtype=torch.int32, device=x.device)
        _rows(q, torch.uint8, "q")
        _rows(sf, torch.int32, "sf")
    else:
        q = sf = None
    _check(_lib.mxfp8_rmsnorm_quantize(_ptr(x), M, K, x.stride(0), _ptr(gamma), float(eps), _ptr(y),
                                       y.stride(0) if y is not None else 0, _ptr(q),
                                       q.stride(0) if q is not None else 0, _ptr(sf),
                                       sf.stride(0) if sf is not None else 0, _stream(stream)),
           "mxfp8_rmsnorm_quantize")
    if not mxfp8_out:
        return y
    return (y, q, sf) if y is not None else (q, sf)


def quantize_weight(w: torch.Tensor, stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """BF16 weight [..., K] -> MXFP8 along K with the same leading shape (codes, packed scales)."""
    lead = w.shape[:-1]
    K = w.shape[-1]
    q, sf = mxfp8_quantize(w.reshape(-1, K), stream=stream)
    return q.reshape(*lead, K), sf.reshape(*lead, K // 128)


# ----------------------------------------------------------------------------- einsum

def _act_args(x: torch.Tensor, x_sf: torch.Tensor | None):
    if x.dtype == torch.bfloat16:
        _rows(x, torch.bfloat16, "x")
        return MXFP8_ACT_BF16, _ptr(x), x.stride(0), None, 0
    _rows(x, torch.uint8, "x")
    if x_sf is None:
        raise ValueError("E4M3 activations need their packed scales")
    _rows(x_sf, torch.int32, "x_sf")
    return MXFP8_ACT_MXFP8, _ptr(x), x.stride(0), _ptr(x_sf), x_sf.stride(0)


def grouped_fp8_einsum(x: torch.Tensor, x_sf: torch.Tensor | None, w: torch.Tensor, w_sf: torch.Tensor, *,
                       out: str = "mxfp8", z_q: torch.Tensor | None = None, z_sf: torch.Tensor | None = None,
                       z_bf16: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
                       splitk_combine: str = "local"):
    """wo_a: z[m, g*N+n] = sum_k x[m, g*K+k] w[g, n, k].

    x: BF16 [M, G*K] (quantized in the kernel) or E4M3 uint8 [M, G*K] with x_sf int32 [M, G*K/128].
    w: uint8 [G, N, K], w_sf: int32 [G, N, K/128].
    out: "mxfp8" -> (z_q, z_sf); "bf16" -> z_bf16; "both" -> (z_q, z_sf, z_bf16).
    splitk_combine: "local" (the product path), or "through" / "recompute" (test-only entry point).
    """
    if w.dim() != 3 or w.dtype != torch.uint8 or w_sf.dtype != torch.int32:
        raise ValueError("w must be uint8 [G, N, K] and w_sf int32 [G, N, K/128]")
    if not (w.is_contiguous() and w_sf.is_contiguous()):
        raise ValueError("w and w_sf must be contiguous")
    G, N, K = w.shape
    kind, xp, ldx, xsfp, ldxsf = _act_args(x, x_sf)
    M = x.shape[0]
    want_mx = out in ("mxfp8", "both")
    want_bf = out in ("bf16", "both")
    if not (want_mx or want_bf):
        raise ValueError(f"unknown out mode {out!r}")
    dev = x.device
    if want_mx:
        if z_q is None:
            z_q = torch.empty((M, G * N), dtype=torch.uint8, device=dev)
        if z_sf is None:
            z_sf = torch.empty((M, G * N // 128), dtype=torch.int32, device=dev)
        _rows(z_q, torch.uint8, "z_q")
        _rows(z_sf, torch.int32, "z_sf")
    else:
        z_q = z_sf = None
    if want_bf:
        if z_bf16 is None:
            z_bf16 = torch.empty((M, G * N), dtype=torch.bfloat16, device=dev)
        _rows(z_bf16, torch.bfloat16, "z_bf16")
    else:
        z_bf16 = None
    sp = _stream(stream)
    wsp, wsn = _ws_args(_lib.grouped_fp8_einsum_workspace_size(kind, M, G, K, N), dev, sp, workspace)
    args = (kind, xp, ldx, xsfp, ldxsf, M, G, K, N, _ptr(w), _ptr(w_sf),
            _ptr(z_q), z_q.stride(0) if z_q is not None else 0,
            _ptr(z_sf), z_sf.stride(0) if z_sf is not None else 0,
            _ptr(z_bf16), z_bf16.stride(0) if z_bf16 is not None else 0, wsp, wsn, sp)
    if splitk_combine == "local":
        _check(_lib.grouped_fp8_einsum(*args), "grouped_fp8_einsum")
    else:
        _check(_lib.mxfp8_testing_grouped_fp8_einsum(SPLITK_MODES[splitk_combine], *args),
               "mxfp8_testing_grouped_fp8_einsum")
    if out == "mxfp8":
        return z_q, z_sf
    if out == "bf16":
        return z_bf16
    return z_q, z_sf, z_bf16


# ----------------------------------------------------------------------------- gemm

def fp8_gemm_nt(a: torch.Tensor, a_sf: torch.Tensor | None, b: torch.Tensor, b_sf: torch.Tensor,
                d: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
                splitk_combine: str = "local") -> torch.Tensor:
    """wo_b: d[m, n] = bf16(sum_k a[m, k] b[n, k]); a BF16 or E4M3 (+ a_sf), b uint8 [N, K] + b_sf int32 [N, K/128].
    splitk_combine as in grouped_fp8_einsum."""
    if b.dim() != 2 or b.dtype != torch.uint8 or b_sf.dtype != torch.int32:
        raise ValueError("b must be uint8 [N, K] and b_sf int32 [N, K/128]")
    if not (b.is_contiguous() and b_sf.is_contiguous()):
        raise ValueError("b and b_sf must be contiguous")
    N, K = b.shape
    kind, ap, lda, asfp, ldasf = _act_args(a, a_sf)
    M = a.shape[0]
    if d is None:
        d = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _rows(d, torch.bfloat16, "d")
    sp = _stream(stream)
    wsp, wsn = _ws_args(_lib.fp8_gemm_nt_workspace_size(kind, M, N, K), a.device, sp, workspace)
    args = (kind, ap, lda, asfp, ldasf, M, N, K, _ptr(b), _ptr(b_sf), _ptr(d), d.stride(0), wsp, wsn, sp)
    if splitk_combine == "local":
        _check(_lib.fp8_gemm_nt(*args), "fp8_gemm_nt")
    else:
        _check(_lib.mxfp8_testing_fp8_gemm_nt(SPLITK_MODES[splitk_combine], *args), "mxfp8_testing_fp8_gemm_nt")
    return d


NOALLOC_SCRATCH_BYTES = 16 << 20     # MXFP8_NOALLOC_SCRATCH_BYTES


def fp8_gemm_nt_noalloc(a: torch.Tensor, a_sf: torch.Tensor | None, b: torch.Tensor, b_sf: torch.Tensor,
                        d: torch.Tensor, stream=None) -> torch.Tensor:
    """fp8_gemm_nt without a workspace: the library's fixed per-GPU scratch serves the kernels instead (for
    callers that cannot allocate; calls that overlap in time on one GPU race on it).  `d` is required."""
    if b.dim() != 2 or b.dtype != torch.uint8 or b_sf.dtype != torch.int32:
        raise ValueError("b must be uint8 [N, K] and b_sf int32 [N, K/128]")
    if not (b.is_contiguous() and b_sf.is_contiguous()):
        raise ValueError("b and b_sf must be contiguous")
    N, K = b.shape
    kind, ap, lda, asfp, ldasf = _act_args(a, a_sf)
    _rows(d, torch.bfloat16, "d")
    _check(_lib.fp8_gemm_nt_noalloc(kind, ap, lda, asfp, ldasf, a.shape[0], N, K, _ptr(b), _ptr(b_sf), _ptr(d),
                                    d.stride(0), _stream(stream)), "fp8_gemm_nt_noalloc")
    return d


# ----------------------------------------------------------------------------- chain

CHAIN_MODES = ("chain", "x_fused", "unfused")


def o_proj_chain(x: torch.Tensor, wo_a: torch.Tensor, wo_a_sf: torch.Tensor, wo_b: torch.Tensor,
                 wo_b_sf: torch.Tensor, mode: str = "chain", stream=None) -> torch.Tensor:
    """The o_proj chain on one stream, no host synchronization; returns BF16 [M, P].

    mode "chain":   mxfp8_quantize(x); the einsum writes z as MXFP8 in its epilogue; the GEMM consumes
                    (z, sf) as is (vLLM PR #60118, Overview: wo_a writes wo_b's MXFP8 input).
    mode "x_fused": as "chain", but the einsum quantizes BF16 x in its own load path (two launches).
    mode "unfused": the arrangement the fused epilogue replaces: the einsum writes BF16 z and a standalone
                    mxfp8_quantize of z feeds the GEMM (PR #60118, Conversation).
    All three give identical bytes.
    """
    if mode == "chain":
        x_q, x_sf = mxfp8_quantize(x, stream=stream)
        z_q, z_sf = grouped_fp8_einsum(x_q, x_sf, wo_a, wo_a_sf, out="mxfp8", stream=stream)
    elif mode == "x_fused":
        z_q, z_sf = grouped_fp8_einsum(x, None, wo_a, wo_a_sf, out="mxfp8", stream=stream)
    elif mode == "unfused":
        x_q, x_sf = mxfp8_quantize(x, stream=stream)
        z = grouped_fp8_einsum(x_q, x_sf, wo_a, wo_a_sf, out="bf16", stream=stream)
        z_q, z_sf = mxfp8_quantize(z, stream=stream)
    else:
        raise ValueError(f"mode must be one of {CHAIN_MODES}")
    return fp8_gemm_nt(z_q, z_sf, wo_b, wo_b_sf, stream=stream)
