"""Shared helpers for the GPU parity tests (host-side conversions and comparisons only)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import mxfp8_ref as mx


def dev():
    return torch.device("cuda", 0)


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns -> bfloat16 device tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(dev())


def u8_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def i32_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def e4m3_ordinal(codes: np.ndarray) -> np.ndarray:
    """Sign-magnitude E4M3 codes -> integers ordered like their values (+0 and -0 both map to 0)."""
    c = codes.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def mx_ulp_distance(q_a, sf_a, q_b, sf_b) -> np.ndarray:
    """Distance in E4M3 ulps between two MXFP8 tensors, in units of the finer of the two block scales.

    Equal scales: difference of ordinals.  Different scales: both dequantized
    values are expressed on the finer scale's grid position by value.
    """
    ea = np.repeat(mx.unpack_scales(sf_a).astype(np.int64), 32, axis=1)
    eb = np.repeat(mx.unpack_scales(sf_b).astype(np.int64), 32, axis=1)
    same = ea == eb
    d = np.abs(e4m3_ordinal(q_a) - e4m3_ordinal(q_b))
    if not same.all():
        va = mx.E4M3_TABLE[q_a] * np.ldexp(1.0, ea - 127)
        vb = mx.E4M3_TABLE[q_b] * np.ldexp(1.0, eb - 127)
        fine = np.minimum(ea, eb)
        # value of one E4M3 ulp at |v| on the finer block's grid
        def ulp(v, e):
            s = np.abs(v) * np.ldexp(1.0, 127 - e)
            _, ex = np.frexp(s)
            return np.ldexp(1.0, np.maximum(ex - 4, -9) + e - 127)
        u = np.minimum(ulp(va, fine), ulp(vb, fine))
        dd = np.abs(va - vb) / np.where(u > 0, u, 1.0)
        d = np.where(same, d, np.ceil(dd))
    return d


def row_rel_err(out_bf16_bits: np.ndarray, ref64: np.ndarray) -> np.ndarray:
    """Per-row max |out - ref| / RMS(ref row) (RMS floored at 1e-30)."""
    out = mx.bf16_decode(out_bf16_bits)
    rms = np.sqrt(np.mean(ref64 ** 2, axis=1))
    return np.max(np.abs(out - ref64), axis=1) / np.maximum(rms, 1e-30)
