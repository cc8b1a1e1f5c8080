"""Pins of the oracle's number formats against definitions, a library and brute force.

The vLLM pages on MXFP8 activations (PR #60118 "[Perf][DSv4.1] MegaAttn: wo_a
writes wo_b's MXFP8 input"; PR #57977 "[Perf][DSv4.1] Keep activations MXFP8
between DeepGEMM kernels") name the format (E4M3 codes, UE8M0 scale per 32
elements, four scales per int32) but print no values.  These tests tie the
oracle to things outside itself: torch's CPU float8_e4m3fn / bfloat16 casts,
closed forms of the format definitions, and exhaustive search.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import mxfp8_ref as mx


def _all_bf16():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _finite_bf16():
    b = _all_bf16()
    return b[np.isfinite(mx.bf16_decode(b))]


# ---------------------------------------------------------------- E4M3 table

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mx.E4M3_TABLE))
    assert np.array_equal(ref[~nan], mx.E4M3_TABLE[~nan])
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}


def test_e4m3_table_closed_forms():
    t = mx.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                       # codes ordered like values
    assert np.array_equal(t[0x80:0xFF], -pos)             # sign bit is a pure sign
    assert np.nanmax(np.abs(t)) == mx.E4M3_MAX


# ---------------------------------------------------------------- BF16

def test_bf16_decode_matches_torch():
    b = _all_bf16()
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = mx.bf16_decode(b)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    f32 = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(50000) * 1e-39).astype(np.float32),      # fp32 subnormals -> BF16 subnormals
        (rng.standard_normal(50000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 448.4375, 2.0 ** -133, -(2.0 ** -134)], dtype=np.float32),
    ])
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mx.bf16_round(f32.astype(np.float64)), ref)


def _bf16_round_bruteforce(v: float) -> int:
    """Nearest finite BF16 to v by exact rational comparison with its two neighbours; ties to even."""
    t = torch.tensor([v], dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    b0 = int(t.view(torch.int16).item()) & 0xFFFF
    cands = {b0}
    for d in (-2, -1, 1, 2):
        mag = (b0 & 0x7FFF) + d
        if 0 <= mag <= 0x7F7F:
            cands.add((b0 & 0x8000) | mag)
            cands.add(mag if b0 & 0x8000 else (0x8000 | mag))
    fv = Fraction(v)
    best = sorted(cands, key=lambda c: (abs(Fraction(mx.bf16_decode_scalar(c)) - fv), c & 1))
    r = best[0]
    if mx.bf16_decode_scalar(r) == 0.0:                 # keep the sign of v on zero
        r = 0x8000 if np.signbit(v) else 0
    return r


def test_bf16_round_float64_exact_single_rounding():
    # midpoints between BF16 neighbours, and one float64 ulp either side of them:
    # a detour through float32 would round these twice and miss by one ulp.
    rng = np.random.default_rng(11)
    base = rng.integers(0x0001, 0x7F7E, size=400).astype(np.uint16)
    lo = mx.bf16_decode(base)
    hi = mx.bf16_decode(base + 1)
    mid = (lo + hi) / 2
    vals = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid,
                           rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, size=300)])
    got = mx.bf16_round(vals)
    for v, g in zip(vals, got):
        assert int(g) == _bf16_round_bruteforce(float(v)), v


def test_bf16_round_rejects_overflow_and_nan():
    with pytest.raises(ValueError):
        mx.bf16_round(np.array([3.5e38]))
    with pytest.raises(ValueError):
        mx.bf16_round(np.array([np.nan]))


# ---------------------------------------------------------------- E4M3 RNE cast

def _cast_domain():
    """All distinct |bf16| * 2**-e magnitudes that the cast can see and that matter.

    Magnitudes below 2**-11 round to zero and above 448 saturate, so the domain
    is every BF16 significand at every exponent in [2**-12, 2**10), plus zero.
    """
    sig = np.arange(128, 256, dtype=np.float64)                # 8-bit significands
    vals = [0.0]
    for j in range(-12 - 7, 10 - 7):
        vals.extend((sig * 2.0 ** j).tolist())
    return np.array(sorted(set(vals)), dtype=np.float64)


def test_e4m3_scalar_cast_matches_torch_in_range():
    dom = _cast_domain()
    dom = dom[dom <= 448.0]
    ref = torch.from_numpy(np.concatenate([dom, -dom]).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    ours = [mx.e4m3_encode_scalar(Fraction(float(v)), False) for v in dom]
    ours += [mx.e4m3_encode_scalar(Fraction(float(v)), True) for v in dom]
    assert np.array_equal(np.array(ours, dtype=np.uint8), ref)


def test_e4m3_scalar_cast_saturates():
    for v in (448.0, 449.0, 464.0, 480.0, 1e6, 3e38):
        assert mx.e4m3_encode_scalar(Fraction(v), False) == 0x7E
        assert mx.e4m3_encode_scalar(Fraction(v), True) == 0xFE


def test_e4m3_vector_cast_matches_scalar_on_domain():
    dom = _cast_domain()
    dom = np.concatenate([dom, [449.0, 464.0, 465.0, 1e9]])
    vec = mx.e4m3_encode(np.concatenate([dom, -dom]))
    sc = [mx.e4m3_encode_scalar(Fraction(float(v)), False) for v in dom]
    sc += [mx.e4m3_encode_scalar(Fraction(float(v)), True) for v in dom]
    assert np.array_equal(vec, np.array(sc, dtype=np.uint8))


def test_e4m3_vector_cast_exhaustive_bf16_times_scale():
    """Every BF16 value times every UE8M0 scale 2**-e, e in [-127, 127] (16.7M casts)."""
    v = mx.bf16_decode(_finite_bf16())
    for e in range(-127, 128):
        s = np.ldexp(v, -e)
        codes = mx.e4m3_encode(s)
        inr = np.abs(s) <= 448.0
        ref = torch.from_numpy(s[inr].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[inr], ref), e
        sat = codes[~inr]
        assert np.all((sat & 0x7F) == 0x7E), e
        assert np.array_equal(sat >> 7, np.signbit(s[~inr]).astype(np.uint8)), e
        assert not np.any((codes & 0x7F) == 0x7F)


# ---------------------------------------------------------------- scale rule

def test_scale_rule_vector_matches_search_exhaustive():
    b = _finite_bf16()
    b = b[b < 0x8000]                                     # non-negative amax values
    amax = mx.bf16_decode(b)
    vec = mx.scale_exponent(amax)
    # the definitional search is slow in Python; it depends only on the value,
    # so run it once per (exponent field, mantissa) pattern -- i.e. all of them
    ref = np.array([mx.scale_exponent_scalar(float(a)) for a in amax], dtype=np.int32)
    assert np.array_equal(vec, ref)


def test_scale_rule_integer_closed_form():
    """e = -127 for BF16 exponent field 0, else max(-127, E - 135 + [mantissa > 0x60])."""
    b = _finite_bf16()
    b = b[b < 0x8000].astype(np.int64)
    E = b >> 7
    m = b & 0x7F
    closed = np.where(E == 0, -127, np.maximum(-127, E - 135 + (m > 0x60)))
    assert np.array_equal(mx.scale_exponent(mx.bf16_decode(b.astype(np.uint16))), closed)


def test_scale_rule_invariant_scaled_amax_in_upper_half():
    b = _finite_bf16()
    b = b[(b < 0x8000) & (b > 0)]
    amax = mx.bf16_decode(b)
    e = mx.scale_exponent(amax)
    s = np.ldexp(amax, -e)
    assert np.all(s <= 448.0)
    unclamped = e > -127
    assert np.all(s[unclamped] > 224.0)
    assert e.max() == 120                                  # BF16 never reaches the upper clamp


@pytest.mark.parametrize("k", [-127, -100, -8, -1, 0, 1, 17, 119])
def test_scale_rule_at_448_times_power_of_two(k):
    a = 448.0 * 2.0 ** k
    assert mx.scale_exponent(np.array([a]))[0] == k
    nb = mx.bf16_round(np.array([float(a)]))[0] + 1          # next BF16 above a
    assert mx.scale_exponent(mx.bf16_decode(np.array([nb])))[0] == k + 1


@pytest.mark.parametrize("j", list(range(-133, 128, 7)))
def test_scale_rule_powers_of_two(j):
    # 2**j * 2**-(j-8) = 256 <= 448 and 512 > 448, so e = j - 8 (clamped)
    assert mx.scale_exponent(np.array([2.0 ** j]))[0] == max(-127, j - 8)
