"""Pins for the oracle's int4-g64 quantiser and planar packer.

Rule (page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战", section 权重转换):
groups of 64 along the input dimension, qmax 7, q = clip(rint(w/s), -8, 7) stored as
unsigned q+8, one fp32 scale per group, planar nibbles (byte k of a group holds element
k in the low nibble and element k+32 in the high nibble).

The oracle is checked against things other than itself: the hand-worked vectors in
tests/golden/, an exact-rational re-derivation of the fp32 results, closed-form bounds
and invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._golden import load_quant_case

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- exact helpers


def f32_round(fr: Fraction) -> float:
    """Round an exact rational to the nearest fp32 value (ties to even), exactly."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = round(a / quantum)  # Fraction.__round__ is round-half-even
    v = n * quantum
    if v >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(v)  # exactly representable in fp32, hence in fp64


def quant_exact(w: np.ndarray):
    """Independent statement of the quantiser with exact rational arithmetic."""
    rows, cols = w.shape
    G = -(-cols // 64)
    packed = np.zeros((rows, G * 32), dtype=np.uint8)
    scales = np.zeros((rows, G), dtype=np.float32)
    for r in range(rows):
        for g in range(G):
            vals = [Fraction(float(w[r, c])) if c < cols else Fraction(0)
                    for c in range(g * 64, g * 64 + 64)]
            amax = max(abs(v) for v in vals)
            s = f32_round(amax / 7)
            u = []
            for v in vals:
                if s == 0:
                    u.append(8)
                    continue
                qf = Fraction(f32_round(v / Fraction(s)))
                q = min(7, max(-8, round(qf)))
                u.append(q + 8)
            scales[r, g] = s
            for k in range(32):
                packed[r, g * 32 + k] = u[k] | (u[k + 32] << 4)
    return packed, scales


def unpack_planar(packed: np.ndarray, cols: int) -> np.ndarray:
    """Planar unpack written independently of the oracle: [rows, cols] nibbles."""
    rows = packed.shape[0]
    G = packed.shape[1] // 32
    b = packed.reshape(rows, G, 32)
    u = np.concatenate([b & 0x0F, b >> 4], axis=2).reshape(rows, G * 64)
    return u[:, :cols].astype(np.int64)


def f32_bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))


# ---------------------------------------------------------------- hand-worked cases


@pytest.mark.parametrize("name", ["quant_E1.txt", "quant_E2.txt", "quant_E3.txt",
                                  "quant_E4.txt"])
def test_golden_group(name):
    w, want_bytes, want_scale = load_quant_case(name)
    packed, scales, st = oracle.quant_int4_g64(w)
    assert st == 0
    assert bytes(packed[0]) == want_bytes
    assert f32_bits(scales[0, 0]) == want_scale


def test_golden_not_interleaved():
    """Planar, not the converter snippet's even/odd interleave (which gives 0x1F)."""
    w, want, _ = load_quant_case("quant_E1.txt")
    packed, _, _ = oracle.quant_int4_g64(w)
    assert packed[0, 0] == 0xCF and want[0] == 0xCF
    u = unpack_planar(packed, 64)[0]
    interleaved_byte0 = int(u[0] | (u[1] << 4))
    assert interleaved_byte0 == 0x1F and packed[0, 0] != interleaved_byte0


def test_golden_e3_fp32_quotient_matters():
    """E3's premise, re-derived exactly: the fp32 quotient is a tie, the exact one not."""
    w, _, want_scale = load_quant_case("quant_E3.txt")
    amax, w1 = Fraction(float(w[0, 0])), Fraction(float(w[0, 1]))
    s = f32_round(amax / 7)
    assert f32_bits(s) == want_scale
    assert f32_round(w1 / Fraction(s)) == -4.5
    assert w1 / Fraction(s) < Fraction(-9, 2)  # exact quotient is below -4.5


# ---------------------------------------------------------------- exact re-derivation


def test_scale_bits_exact_rational():
    """s = fl32(amax/7) bit-exactly, over 1e5 amax values incl. subnormals."""
    rng = np.random.default_rng(12345)
    n = 100_000
    bits = rng.integers(1, 0x7F800000, size=n, dtype=np.uint32)  # all positive finite
    bits[:2000] = rng.integers(1, 0x00800000, size=2000, dtype=np.uint32)  # subnormal
    amax = bits.view(np.float32)
    w = np.zeros((n, 64), dtype=np.float32)
    w[:, 5] = amax
    w[:, 40] = -amax * np.float32(0.5)
    _, scales, st = oracle.quant_int4_g64(w)
    assert st == 0
    # exact check on a subsample (Fractions are slow), plus a cheap full check
    for i in range(0, n, 7):
        s = f32_round(Fraction(float(amax[i])) / 7)
        assert f32_bits(scales[i, 0]) == f32_bits(s), (i, hex(bits[i]))
    ref = (amax.astype(np.float64) / 7.0).astype(np.float32)
    assert np.array_equal(scales[:, 0].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("cols", [64, 200, 1, 130])
def test_quant_matches_exact_rational(cols):
    """Bit-exact against the exact-rational statement, incl. ragged last groups."""
    rng = np.random.default_rng(cols)
    w = (rng.standard_normal((6, cols)) * 0.02).astype(np.float32)
    # plant exact ties: w = s*(k+1/2) with s a power of two
    if cols >= 64:
        w[0, :8] = np.float32(2.0 ** -6) * np.array([7, -7, .5, 1.5, 2.5, -.5, -1.5, -6.5],
                                                   dtype=np.float32)
    p, s, st = oracle.quant_int4_g64(w)
    pe, se = quant_exact(w)
    assert st == 0
    assert np.array_equal(p, pe)
    assert np.array_equal(s.view(np.uint32), se.view(np.uint32))


# ---------------------------------------------------------------- invariants


def test_invariants_random():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((64, 640)) * 0.02).astype(np.float32)
    p, s, st = oracle.quant_int4_g64(w)
    assert st == 0
    u = unpack_planar(p, 640)
    assert u.min() >= 1 and u.max() <= 15  # |q| <= 7 for non-zero groups
    q = u - 8
    sg = np.repeat(s.astype(np.float64), 64, axis=1)[:, :640]
    # the element with |w| = amax maps to +-7
    wg = w.reshape(64, 10, 64)
    am = np.argmax(np.abs(wg), axis=2)
    qg = q.reshape(64, 10, 64)
    top = np.take_along_axis(qg, am[..., None], axis=2)[..., 0]
    sign = np.sign(np.take_along_axis(wg, am[..., None], axis=2)[..., 0])
    assert np.array_equal(top, 7 * sign.astype(np.int64))
    # rounding error bound |w - s q| <= s/2 (1 + 2^-22)
    err = np.abs(w.astype(np.float64) - sg * q)
    assert np.all(err <= sg / 2 * (1 + 2.0 ** -22))


def test_requantise_is_identity_when_exact():
    """Quantising s*q again returns the same bytes and scale (7s, s*q exact in fp32)."""
    rng = np.random.default_rng(3)
    q = rng.integers(-7, 8, size=(8, 256))
    q[:, ::64] = 7  # every group attains amax = 7 s
    s = (2.0 ** rng.integers(-20, 4, size=(8, 4))).repeat(64, axis=1)
    w = (q * s).astype(np.float32)
    p, sc, _ = oracle.quant_int4_g64(w)
    assert np.array_equal(unpack_planar(p, 256) - 8, q)
    p2, sc2, _ = oracle.quant_int4_g64(oracle.dequant_int4_g64(p, sc, 256).astype(np.float32))
    assert np.array_equal(p, p2) and np.array_equal(sc.view(np.uint32), sc2.view(np.uint32))


def test_planar_round_trip_and_dequant():
    """Packing then unpacking the planar layout is the identity; dequant = s (u - 8)."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((5, 192)) * 0.3).astype(np.float32)
    p, s, _ = oracle.quant_int4_g64(w)
    u = unpack_planar(p, 192)
    # re-pack with an independent planar writer
    G = 3
    uu = u.reshape(5, G, 64)
    rep = (uu[:, :, :32] | (uu[:, :, 32:] << 4)).astype(np.uint8).reshape(5, G * 32)
    assert np.array_equal(rep, p)
    d = oracle.dequant_int4_g64(p, s, 192)
    assert np.array_equal(d, np.repeat(s.astype(np.float64), 64, axis=1) * (u - 8))


def test_zero_and_ragged_padding():
    w = np.zeros((2, 70), dtype=np.float32)
    w[1, 69] = -1.0  # alone in the ragged second group
    p, s, st = oracle.quant_int4_g64(w)
    assert st == 0
    assert np.all(p[0] == 0x88) and np.all(s[0] == 0)
    assert f32_bits(s[1, 1]) == f32_bits(np.float32(1.0 / 7.0))
    u = unpack_planar(p, 128)
    assert u[1, 69] == 1 and np.all(np.delete(u[1], 69) == 8)  # pad nibbles are 8


def test_nonfinite_group_fails_closed():
    w = (np.arange(256, dtype=np.float32) * 0.01).reshape(2, 128)
    w[0, 3] = np.nan
    w[1, 100] = np.inf
    p, s, st = oracle.quant_int4_g64(w)
    assert st == 1
    assert np.isnan(s[0, 0]) and np.isnan(s[1, 1])
    assert np.all(p[0, :32] == 0x88) and np.all(p[1, 32:] == 0x88)
    assert np.isfinite(s[0, 1]) and np.isfinite(s[1, 0])  # other groups untouched


def test_minus_zero_and_no_nibble_zero():
    """rint(-0.4) is -0 -> nibble 8; with s = amax/7 nibble 0 (q=-8) never appears."""
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 7.0
    w[0, 1] = -0.4
    w[0, 2] = -7.0
    p, _, _ = oracle.quant_int4_g64(w)
    u = unpack_planar(p, 64)[0]
    assert u[1] == 8 and u[2] == 1 and u.min() >= 1


# ---------------------------------------------------------------- the identity


def test_identity_integer_exact():
    """dot(u, x) - 8 sum(x) == dot(q, x) exactly for integer x (the VNNI identity)."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    p, s, _ = oracle.quant_int4_g64(w)
    u = unpack_planar(p, 256)
    q = np.rint(oracle.dequant_int4_g64(p, s, 256) / np.repeat(s, 64, axis=1)).astype(np.int64)
    x = rng.integers(-128, 128, size=256).astype(np.int64)
    assert np.array_equal(u @ x - 8 * x.sum(), q @ x)


def test_identity_float_within_bound():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    p, s, _ = oracle.quant_int4_g64(w)
    u = unpack_planar(p, 256).astype(np.float64)
    q = u - 8
    x = rng.standard_normal(256)
    lhs = u @ x - 8 * x.sum()
    rhs = q @ x
    bound = 2 * 256 * 2.0 ** -52 * (np.abs(u) @ np.abs(x) + 8 * np.abs(x).sum())
    assert np.all(np.abs(lhs - rhs) <= bound)
