"""Pins for the oracle's symmetric INT4 quantizer and its P code (CPU only).

The P code is RotateAttention's range-optimized P quantization (RotateAttention
page, Abstract): P = exp(s - max) lies in (0, 1], so a fixed scale of 1/15 and
zero point 0 map it onto all 16 unsigned 4-bit levels.  The oracle evaluates
rne(15 * 2^x) through float32 thresholds; these tests check the thresholds and
the code against exact (mpmath) arithmetic and against numpy's exp2.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle as O

F32 = np.float32


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _from_bits(b):
    return np.asarray(b, np.uint32).view(np.float32)


# ---------------------------------------------------------------- quantizer

def _brute_code(v):
    """Integer in [-7, 7] nearest to the float v, ties to the even integer."""
    best = None
    for c in range(-7, 8):
        d = abs(Fraction(float(v)) - c)
        key = (d, c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_quantizer_brute_force_tiny_blocks():
    """P4: codes, scale and inverse scale match exact rational arithmetic."""
    rng = np.random.default_rng(10)
    z = (rng.standard_normal((300, 8)) * rng.uniform(0.01, 50, size=(300, 1))).astype(F32)
    codes, scale, inv = O.quantize_blocks(z, block=128)
    for b in range(3):
        blk = z[b * 128:(b + 1) * 128]
        amax = max(abs(float(x)) for x in blk.ravel())
        assert scale[b] == O.nearest_f32(mpmath.mpf(amax) / 7)
        assert inv[b] == O.nearest_f32(7 / mpmath.mpf(amax))
        for i in range(blk.shape[0]):
            for j in range(blk.shape[1]):
                v = F32(blk[i, j]) * inv[b]          # one float32 rounding
                assert codes[b * 128 + i, j] == _brute_code(v)


def test_quantizer_laws():
    """P4: codes in [-7, 7]; the amax element maps to +-7; error <= scale/2."""
    rng = np.random.default_rng(11)
    for trial in range(20):
        n = int(rng.integers(1, 400))
        z = (rng.standard_normal((n, 16)) * np.exp(rng.standard_normal())).astype(F32)
        codes, scale, _ = O.quantize_blocks(z)
        assert codes.min() >= -7 and codes.max() <= 7
        for b in range(len(scale)):
            blk = z[b * 128:(b + 1) * 128]
            cb = codes[b * 128:(b + 1) * 128]
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert abs(int(cb[i])) == 7 and np.sign(cb[i]) == np.sign(blk[i])
            err = np.abs(blk.astype(np.float64) - cb * np.float64(scale[b]))
            assert np.all(err <= 0.5 * scale[b] * (1 + 2.0 ** -20))


def test_quantizer_zero_and_partial_blocks():
    z = np.zeros((200, 8), F32)
    z[150, 3] = -2.5
    codes, scale, inv = O.quantize_blocks(z)
    assert scale[0] == 0 and inv[0] == 0 and not codes[:128].any()
    assert codes[150, 3] == -7 and scale[1] == F32(2.5) / F32(7)
    assert np.count_nonzero(codes) == 1


def test_kappa_matches_exact():
    for D, approx in ((128, 0.12751743), (64, 0.18033688)):
        k = O.kappa(D)
        assert abs(float(k) - approx) < 1e-8
        exact = mpmath.log(mpmath.e, 2) / mpmath.sqrt(D)
        assert abs(mpmath.mpf(float(k)) - exact) <= mpmath.mpf(float(np.spacing(k))) / 2


# ---------------------------------------------------------------- P code

def test_thresholds_bracket_the_half_levels():
    """P5: tau_k is the smallest float32 with 15 * 2^tau_k >= k - 1/2 (mpmath)."""
    tau = O.pcode_thresholds()
    assert tau.dtype == np.float32 and tau.shape == (15,)
    assert np.all(np.diff(tau) > 0)
    for k in range(1, 16):
        t = tau[k - 1]
        prev = np.nextafter(t, F32(-np.inf), dtype=F32)
        half = mpmath.mpf(2 * k - 1) / 2
        assert 15 * mpmath.power(2, mpmath.mpf(float(t))) >= half
        assert 15 * mpmath.power(2, mpmath.mpf(float(prev))) < half
    assert tau[7] == F32(-1.0)      # the only exact tie: 7.5 -> 8


def _exact_code_f64(x):
    """rne(15 * 2^x) via float64 exp2, exact away from the half levels."""
    y = 15.0 * np.exp2(np.asarray(x, np.float64))
    c = np.floor(y + 0.5)
    near = np.abs(y - (np.floor(y) + 0.5)) < 1e-9
    return np.clip(c, 0, 15), near


def test_pcode_windows_around_every_threshold():
    """P5: every float32 within 2^14 ulps of each tau_k, against exp2 and mpmath."""
    tau = O.pcode_thresholds()
    for t in tau:
        b = int(_bits(t))
        bits = np.arange(b - (1 << 14), b + (1 << 14), dtype=np.int64)
        xs = _from_bits(bits.astype(np.uint32))
        got = O.pcode(xs)
        want, near = _exact_code_f64(xs)
        for i in np.nonzero(near)[0]:
            y = 15 * mpmath.power(2, mpmath.mpf(float(xs[i])))
            fl = int(mpmath.floor(y))
            frac = y - fl
            want[i] = fl + (1 if frac > 0.5 or (frac == 0.5 and fl % 2 == 1) else 0)
        assert np.array_equal(got, want.astype(np.uint8))


def test_pcode_random_sweep_and_special_values():
    """P5: a random sweep of [-8, 0] and the special points of the code."""
    rng = np.random.default_rng(12)
    xs = (-8.0 * rng.random(2_000_000)).astype(F32)
    got = O.pcode(xs)
    want, near = _exact_code_f64(xs)
    ok = ~near
    assert np.array_equal(got[ok], want[ok].astype(np.uint8))
    tau = O.pcode_thresholds()
    assert O.pcode(F32(0.0)) == 15
    assert O.pcode(F32(-0.0)) == 15
    assert O.pcode(F32(-1.0)) == 8
    assert O.pcode(np.nextafter(F32(-1.0), F32(-2.0), dtype=F32)) == 7
    assert O.pcode(tau[0]) == 1
    assert O.pcode(np.nextafter(tau[0], F32(-9.0), dtype=F32)) == 0
    assert O.pcode(F32(-np.inf)) == 0
    assert O.pcode(F32(-100.0)) == 0


def test_pcode_monotone_and_uses_every_level():
    xs = np.sort((-6.0 * np.random.default_rng(13).random(100_000)).astype(F32))
    c = O.pcode(xs)
    assert np.all(np.diff(c.astype(np.int16)) >= 0)
    assert set(np.unique(c)) == set(range(16))


def test_symmetric_p_code_wastes_half_the_range():
    """The motivating fact: P >= 0, so a symmetric 4-bit code of P in (0, 1]
    reaches at most 8 distinct levels, while the range-optimized code reaches 16."""
    p = np.linspace(1e-6, 1.0, 100_001)
    sym = np.clip(np.rint(p * 7), -7, 7)           # symmetric, scale 1/7
    assert len(np.unique(sym)) == 8
    x = np.log2(p).astype(F32)
    assert len(np.unique(O.pcode(x))) == 16
