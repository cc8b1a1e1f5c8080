"""CPU oracle: MXFP8 encoding of BF16 data (test infrastructure, never product code).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the GPU library and imports nothing from it.

What it computes (vLLM PR #60118 "[Perf][DSv4.1] MegaAttn: wo_a writes wo_b's
MXFP8 input", sections Conversation and Overview; vLLM PR #57977 "[Perf][DSv4.1]
Keep activations MXFP8 between DeepGEMM kernels", sections Purpose and Pieces):
an MXFP8 tensor is FP8 E4M3 codes plus one UE8M0 power-of-two scale per 32
contiguous elements of a row, the scales packed four to an int32.

The pages name the format but not the scale rule, the rounding or the packing
order.  Readings taken here (each listed with its reason in the design notes):
  * scale exponent e = the smallest integer with amax <= 448 * 2**e, clamped to
    [-127, 127]; an all-zero block gets e = -127 (byte 0x00);
  * codes = round-to-nearest-even of v * 2**-e onto the OCP E4M3FN grid,
    magnitudes above 448 saturate to 448, the sign is kept (-0 -> 0x80), and
    0x7F / 0xFF (NaN) are never produced;
  * scale byte = e + 127; word w of a row holds blocks 4w..4w+3, block 4w+j in
    bits [8j, 8j+8);
  * non-finite input is outside the contract and raises ValueError.

Two implementations live here and are tested bit-identical to each other:
  * the ``*_scalar`` functions are the specification, in exact rational
    arithmetic (``fractions.Fraction``), one element at a time;
  * the vectorized numpy functions are what the chain oracle uses; every step is
    an exact float64 operation (frexp / ldexp / round-half-even).
"""
from __future__ import annotations

from bisect import bisect_left
from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32           # elements per UE8M0 scale
PACK = 4             # scale bytes per int32 word
WORD_SPAN = BLOCK * PACK
E_MIN, E_MAX = -127, 127
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# --------------------------------------------------------------------------
# Formats: OCP FP8 E4M3FN and BF16, decoded from their definitions
# --------------------------------------------------------------------------

def e4m3_decode_scalar(code: int) -> float:
    """Value of an OCP E4M3FN byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 encodes subnormals m/8 * 2**-6; 0x7F and 0xFF are NaN; the
    format has no infinities, so 0x7E (exponent 15, mantissa 6) = 448 is the
    largest finite value.
    """
    code &= 0xFF
    s = -1.0 if code & 0x80 else 1.0
    ef = (code >> 3) & 0xF
    m = code & 0x7
    if ef == 0xF and m == 0x7:
        return float("nan")
    if ef == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (ef - 7)


E4M3_TABLE = np.array([e4m3_decode_scalar(c) for c in range(256)], dtype=np.float64)
# finite non-negative grid, ascending with the code: codes 0x00..0x7E
_POS_CODES = list(range(0x7F))
_POS_VALUES = [Fraction(E4M3_TABLE[c]) for c in _POS_CODES]


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float64, exactly (BF16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_decode_scalar(bits: int) -> float:
    return float(bf16_decode(np.array([bits], dtype=np.uint16))[0])


def bf16_round(v: np.ndarray) -> np.ndarray:
    """float64 -> BF16 bit patterns with one round-to-nearest-even step.

    BF16 keeps 8 significant bits; below 2**-126 its grid is the subnormal
    spacing 2**-133.  Rounding is done on the float64 value itself (no detour
    through float32, which would round twice).  Overflow past the largest BF16
    raises ValueError (outside the contract).
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("bf16_round: non-finite input")
    a = np.abs(v)
    _, e = np.frexp(a)                       # a = f * 2**e, f in [0.5, 1)
    q = np.maximum(e - 8, -133)              # exponent of one BF16 ulp at a
    r = np.ldexp(np.round(np.ldexp(a, -q)), q)   # np.round: half to even
    if np.any(r > BF16_MAX):
        raise ValueError("bf16_round: overflow")
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return bits | (np.signbit(v).astype(np.uint16) << 15)


# --------------------------------------------------------------------------
# Specification: one block at a time, exact rational arithmetic
# --------------------------------------------------------------------------

def scale_exponent_scalar(amax) -> int:
    """Smallest e in [-127, 127] with amax <= 448 * 2**e (e = -127 when amax == 0).

    A search over the UE8M0 range, compared exactly.  If even 448 * 2**127 is
    too small (impossible for BF16 input) the clamp gives 127.
    """
    a = Fraction(amax)
    if a < 0:
        raise ValueError("amax must be >= 0")
    e = E_MIN
    while e < E_MAX and a > _LIMITS[e - E_MIN]:
        e += 1
    return e


_LIMITS = [448 * Fraction(2) ** e for e in range(E_MIN, E_MAX + 1)]   # 448 * 2**e, exact


def e4m3_encode_scalar(mag: Fraction, negative: bool) -> int:
    """Nearest finite E4M3FN value to ``mag`` (>= 0), ties to the even code; sign bit from ``negative``.

    Magnitudes above 448 saturate to 448 (0x7E).  A negative value that rounds
    to zero keeps its sign (0x80).
    """
    if mag < 0:
        raise ValueError("mag must be >= 0")
    if mag >= _POS_VALUES[-1]:
        code = 0x7E
    else:
        i = bisect_left(_POS_VALUES, mag)          # _POS_VALUES[i-1] < mag <= _POS_VALUES[i]
        if _POS_VALUES[i] == mag:
            code = _POS_CODES[i]
        else:
            lo, hi = i - 1, i
            dlo = mag - _POS_VALUES[lo]
            dhi = _POS_VALUES[hi] - mag
            if dlo < dhi:
                code = _POS_CODES[lo]
            elif dhi < dlo:
                code = _POS_CODES[hi]
            else:                                   # exact tie: even mantissa
                code = _POS_CODES[lo] if _POS_CODES[lo] % 2 == 0 else _POS_CODES[hi]
    return code | (0x80 if negative else 0)


def quantize_block_scalar(bits32) -> tuple[int, list[int]]:
    """One block of BF16 bit patterns -> (UE8M0 scale byte, E4M3 codes)."""
    vals = []
    for b in bits32:
        b = int(b) & 0xFFFF
        x = bf16_decode_scalar(b)
        if x != x or x in (float("inf"), float("-inf")):
            raise ValueError("non-finite input")
        vals.append((Fraction(abs(x)), bool(b & 0x8000)))
    amax = max(m for m, _ in vals)
    e = scale_exponent_scalar(amax)
    inv = Fraction(2) ** (-e)
    codes = [e4m3_encode_scalar(m * inv, neg) for m, neg in vals]
    return e + 127, codes


def quantize_scalar(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Rows of BF16 bits [R, C] -> (codes uint8 [R, C], scale bytes uint8 [R, C/32]); C % 32 == 0."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    R, C = x_bits.shape
    if C % BLOCK:
        raise ValueError("row length must be a multiple of 32")
    codes = np.zeros((R, C), dtype=np.uint8)
    sf = np.zeros((R, C // BLOCK), dtype=np.uint8)
    for r in range(R):
        for b in range(C // BLOCK):
            s, q = quantize_block_scalar(x_bits[r, b * BLOCK:(b + 1) * BLOCK])
            sf[r, b] = s
            codes[r, b * BLOCK:(b + 1) * BLOCK] = q
    return codes, sf


# --------------------------------------------------------------------------
# Vectorized numpy version (bit-identical to the specification)
# --------------------------------------------------------------------------

def scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Vectorized smallest e with amax <= 448 * 2**e, clamped to [-127, 127]; int32.

    With amax = f * 2**E (f in [0.5, 1)) and 448 = 0.875 * 2**9 the condition is
    E <= 9 + e when f <= 0.875, else E < 9 + e.
    """
    a = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(a)
    e = E.astype(np.int64) - 9 + (f > 0.875)
    e = np.where(a == 0.0, E_MIN, e)
    return np.clip(e, E_MIN, E_MAX).astype(np.int32)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Vectorized RNE + saturation of exact float64 values onto the E4M3FN grid; uint8 codes.

    E4M3 keeps 4 significant bits; below 2**-6 its grid is the subnormal spacing
    2**-9.  np.round rounds halves to even, which on this grid is the even code.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)
    q = np.maximum(e - 4, -9)                            # exponent of one E4M3 ulp at a
    r = np.minimum(np.ldexp(np.round(np.ldexp(a, -q)), q), E4M3_MAX)
    # value -> code
    f2, e2 = np.frexp(r)                                 # r = f2 * 2**e2
    normal = r >= 2.0 ** -6
    ef = np.where(normal, e2 - 1 + 7, 0)                 # biased exponent field
    mant = np.where(normal, np.ldexp(r, -(e2 - 1) + 3) - 8, np.ldexp(r, 9))
    code = (ef.astype(np.int64) << 3) | mant.astype(np.int64)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def pack_scales(sf_bytes: np.ndarray) -> np.ndarray:
    """Scale bytes [R, C/32] -> int32 words [R, C/128]; block 4w+j lands in bits [8j, 8j+8) of word w."""
    sf_bytes = np.asarray(sf_bytes, dtype=np.uint8)
    R, nb = sf_bytes.shape
    if nb % PACK:
        raise ValueError("row length must be a multiple of 128")
    b = sf_bytes.reshape(R, nb // PACK, PACK).astype(np.uint32)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    return w.view(np.int32)


def unpack_scales(sf_words: np.ndarray) -> np.ndarray:
    """int32 words [R, C/128] -> scale bytes [R, C/32] (inverse of pack_scales)."""
    w = np.asarray(sf_words, dtype=np.int32).view(np.uint32)
    R, nw = w.shape
    out = np.empty((R, nw, PACK), dtype=np.uint8)
    for j in range(PACK):
        out[..., j] = (w >> (8 * j)) & 0xFF
    return out.reshape(R, nw * PACK)


def _quantize_chunk(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    R, C = v.shape
    blk = v.reshape(R, C // BLOCK, BLOCK)
    amax = np.abs(blk).max(axis=-1)
    e = scale_exponent(amax)
    codes = e4m3_encode(np.ldexp(blk, -e[..., None]))    # exact power-of-two scaling
    return codes.reshape(R, C), (e + 127).astype(np.uint8)


def quantize(x_bits: np.ndarray, chunk_elems: int = 1 << 23) -> tuple[np.ndarray, np.ndarray]:
    """Rows of BF16 bits [R, C] -> (codes uint8 [R, C], packed scales int32 [R, C/128]); C % 128 == 0."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2:
        raise ValueError("quantize expects a 2-D array of rows")
    R, C = x_bits.shape
    if C % WORD_SPAN:
        raise ValueError("row length must be a multiple of 128")
    codes = np.empty((R, C), dtype=np.uint8)
    sfb = np.empty((R, C // BLOCK), dtype=np.uint8)
    step = max(1, chunk_elems // max(C, 1))
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        v = bf16_decode(x_bits[r0:r1])
        if not np.all(np.isfinite(v)):
            raise ValueError("quantize: non-finite input")
        codes[r0:r1], sfb[r0:r1] = _quantize_chunk(v)
    return codes, pack_scales(sfb)


def quantize_bytes(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Like quantize, but returns the unpacked scale bytes [R, C/32] (C % 32 == 0)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    v = bf16_decode(x_bits)
    if not np.all(np.isfinite(v)):
        raise ValueError("quantize: non-finite input")
    return _quantize_chunk(v)


def dequantize(codes: np.ndarray, sf_words: np.ndarray) -> np.ndarray:
    """codes [R, C] + packed scales [R, C/128] -> float64 [R, C]: decode(code) * 2**(byte - 127)."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, C = codes.shape
    e = unpack_scales(sf_words).astype(np.int64) - 127
    vals = E4M3_TABLE[codes].reshape(R, C // BLOCK, BLOCK)
    return np.ldexp(vals, e[..., None]).reshape(R, C)
