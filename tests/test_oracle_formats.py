"""Pins for the sibling-format oracle (oracle/formats.py), from what the pages and the
published format definitions fix:

* the registry's byte arithmetic (page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射
  实战", section 权重转换): int3 with a per-group scale is 3.5 bits per weight (page
  "Colibrì 深度解析", section 八), int4-g64 4.5, raw f32 has no scale array (section
  十五, issue 1434); MXFP4 is 4.25 bits per weight (32 four-bit elements + one byte);
* inference from byte counts is unique on the layer shapes of these workloads and
  refuses the shapes where two formats have the same byte counts;
* E4M3 encoding equals torch's float8_e4m3fn conversion (a library routine) on
  saturated inputs, and the OCP E4M3 constants (448, 2^-9, the NaN code);
* E2M1 encoding: every representable value maps to itself, every midpoint to its
  even neighbour, beyond 6 saturates (the OCP MX element rules), checked against a
  rounding written per binade with Python's round();
* the MXFP4 shared exponent is floor(log2 max|v|) - 2 (math.frexp), and a block
  whose values are representable after scaling dequantises exactly;
* int3-g64: brute force nearest-even over {-4..3}, the group's amax element maps to
  +-3, the bit planes unpack with numpy's unpackbits;
* the matrix-vector product against exact rational arithmetic.
A wrong index, a dropped term or a transposed operand in any of these fails one."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F


# ---------------------------------------------------------------- sizes, inference

def bits_per_weight(fmt, O, I):
    w, s = F.sizes(fmt, O, I)
    return 8.0 * (w + s) / (O * I)


def test_bits_per_weight_stated_by_the_pages():
    O, I = 2048, 6144
    assert bits_per_weight(5, O, I) == 3.5   # "3.5 bit/weight int3 per-group scale"
    assert bits_per_weight(4, O, I) == 4.5   # 4-bit nibbles + one f32 per 64
    assert bits_per_weight(7, O, I) == 4.25  # OCP MXFP4
    assert F.sizes(0, O, I) == (4 * O * I, 0)  # raw f32: no scale array
    assert F.sizes(6, O, I) is None            # E8/IQ3: never inferred
    # the int4-g64 expert matrix of the decode layer: 6,291,456 nibble bytes + 196,608 scales
    assert F.sizes(4, 2048, 6144) == (6_291_456, 786_432)


@pytest.mark.parametrize("O,I", [(2048, 6144), (6144, 2048), (256, 6144), (72, 200),
                                 (1000, 330), (129, 257)])
def test_inference_is_unique_on_layer_shapes(O, I):
    for fmt in (0, 1, 2, 3, 4, 5, 7, 8):
        got, cands = F.resolve(O, I, *F.sizes(fmt, O, I))
        assert got == fmt, (fmt, cands)
    assert F.resolve(O, I, 1, 1) == (None, [])


def test_inference_refuses_ambiguous_shapes():
    # int4-row and int4-g64 of a 64-wide row: 32 bytes + one f32 per row each
    assert F.resolve(10, 64, 320, 40) == (None, [2, 4])
    # int4-row and MXFP4 of a 128-wide row: 64 bytes + 4 bytes per row each
    assert F.resolve(3, 128, 192, 12) == (None, [2, 7])
    # int8-row and fp8-b128 of one row: I bytes + one f32
    assert F.resolve(1, 100, 100, 4) == (None, [1, 8])


# ---------------------------------------------------------------- E4M3

def test_e4m3_constants():
    assert F.E4M3[-1] == 448.0 and F.E4M3[1] == 2.0 ** -9 and F.E4M3[8] == 2.0 ** -6
    assert len(F.E4M3) == 127 and np.all(np.diff(F.E4M3) > 0)
    assert F.e4m3_encode(np.array([448.0, -448.0, 0.0, -0.0], np.float32)).tolist() == \
        [0x7E, 0xFE, 0x00, 0x80]
    assert np.isnan(F.e4m3_decode(np.array([0x7F, 0xFF]))).all()


def test_e4m3_matches_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 3, 60, 400)])
    v = np.concatenate([v, F.E4M3, -F.E4M3, (F.E4M3[1:] + F.E4M3[:-1]) / 2,
                        np.array([1e-4, 2.0 ** -10, 3 * 2.0 ** -11, 440.0, 447.9])])
    v = v.astype(np.float32)
    vc = np.clip(v, -448, 448)  # torch's conversion does not saturate
    ref = torch.from_numpy(vc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(vc), ref)
    assert np.array_equal(F.e4m3_encode(np.array([500.0, -1e9], np.float32)), [0x7E, 0xFE])
    assert np.array_equal(F.e4m3_decode(ref), torch.from_numpy(ref).view(
        torch.float8_e4m3fn).double().numpy())


# ---------------------------------------------------------------- E2M1

def e2m1_round_per_binade(x: float) -> float:
    """RNE onto the E2M1 grid written with Python's round() per binade."""
    a = abs(x)
    if a >= 6.0:
        return 6.0
    if a < 1.0:
        return round(a * 2) / 2          # step 0.5 on [0, 1) (subnormal 0.5)
    if a < 2.0:
        return round(a * 2) / 2          # step 0.5 on [1, 2)
    if a < 4.0:
        return float(round(a))           # step 1 on [2, 4)
    return round(a / 2) * 2.0            # step 2 on [4, 6)


def test_e2m1_rounding():
    vals = np.concatenate([F.E2M1, (F.E2M1[1:] + F.E2M1[:-1]) / 2,
                           np.random.default_rng(4).uniform(0, 8, 5000)]).astype(np.float32)
    codes = F.e2m1_encode(vals)
    got = F.e2m1_decode(codes)
    want = np.array([e2m1_round_per_binade(float(x)) for x in vals])
    assert np.array_equal(got, want)
    assert np.array_equal(F.e2m1_encode(F.E2M1.astype(np.float32)), np.arange(8))
    # midpoints go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert F.e2m1_decode(F.e2m1_encode(mids)).tolist() == [0, 1, 1, 2, 2, 4, 4]
    assert F.e2m1_encode(np.array([-0.1, -6.5], np.float32)).tolist() == [8, 15]


# ---------------------------------------------------------------- MXFP4

def test_mxfp4_shared_exponent_and_exact_blocks():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((7, 100)) * 0.02).astype(np.float32)
    pk, sc = F.quant_mxfp4(w)
    assert pk.shape == (7, 64) and sc.shape == (7, 4)
    for o in range(7):
        for b in range(4):
            blk = np.zeros(32, np.float32)
            seg = w[o, 32 * b:32 * (b + 1)]
            blk[:seg.size] = seg
            amax = float(np.abs(blk).max())
            assert int(sc[o, b]) - 127 == math.floor(math.log2(amax)) - 2
    # a block of representable values times a power of two comes back exactly
    grid = np.resize(np.concatenate([F.E2M1, -F.E2M1[1:]]), 32)
    for k in (-20, -3, 0, 7):
        blk = (grid * 2.0 ** k).astype(np.float32)[None, :]
        pk, sc = F.quant_mxfp4(blk)
        assert int(sc[0, 0]) - 127 == k  # amax 6 = 1.5 * 2^2
        assert np.array_equal(F.dequant_mxfp4(pk, sc, 32)[0], blk[0].astype(np.float64))
    # element 2j low nibble, 2j + 1 high nibble
    blk = np.zeros((1, 32), np.float32)
    blk[0, 0], blk[0, 1], blk[0, 31] = 6.0, -1.0, 0.5
    pk, sc = F.quant_mxfp4(blk)
    assert sc[0, 0] == 127 and pk[0, 0] == (0x7 | (0xA << 4)) and pk[0, 15] == (0x1 << 4)
    # all-zero block: E = 0, codes 0; non-finite: E = 255
    pk, sc = F.quant_mxfp4(np.zeros((1, 32), np.float32))
    assert sc[0, 0] == 0 and not pk.any()
    bad = np.ones((1, 64), np.float32)
    bad[0, 40] = np.inf
    pk, sc = F.quant_mxfp4(bad)
    assert sc.tolist() == [[125, 255]]  # amax 1: floor(log2 1) - 2 = -2


def test_mxfp4_error_bound():
    # with X = 2^(floor(log2 amax) - 2), v / X < 8: values up to 6 X round with at
    # most half a step (X at the top binade), above 6 X they saturate
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    pk, sc = F.quant_mxfp4(w)
    W = F.dequant_mxfp4(pk, sc, 256)
    X = np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
    err = np.abs(W - w)
    top = np.abs(w) > 6 * X
    assert np.all(err[~top] <= X[~top] + 1e-30)
    assert np.all(np.abs(W[top]) == 6 * X[top])


# ---------------------------------------------------------------- int3-g64

def test_int3_brute_force_and_closed_forms():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((5, 150)) * 0.02).astype(np.float32)
    w[1, 64:128] = 0.0  # an all-zero group
    pk, sc = F.quant_int3_g64(w)
    assert pk.shape == (5, 72) and sc.shape == (5, 3)
    u = unpack_planes(pk, 5, 3)
    for o in range(5):
        for g in range(3):
            seg = np.zeros(64, np.float32)
            part = w[o, 64 * g:64 * (g + 1)]
            seg[:part.size] = part
            amax = np.float32(np.abs(seg).max())
            s = np.float32(amax / np.float32(3))
            assert sc[o, g] == s
            if s == 0:
                assert np.all(u[o, g] == 4)
                continue
            for j in range(64):
                qf = float(np.float32(seg[j] / s))
                cand = sorted(range(-4, 4), key=lambda q: (abs(q - qf), q % 2))
                assert u[o, g, j] == cand[0] + 4, (o, g, j, qf)
            k = int(np.argmax(np.abs(seg)))
            assert u[o, g, k] in (1, 7)  # the amax element maps to -3 or +3
    W = F.dequant_int3_g64(pk, sc, 150)
    assert np.all(np.abs(W - w) <= sc.repeat(64, axis=1)[:, :150] / 2 * (1 + 1e-6))


def test_int3_ties_to_even():
    # s = 3 / 3 = 1: quotients 0.5, 1.5, 2.5, -2.5, -3.5 and 2.9 (amax 3)
    w = np.zeros((1, 64), np.float32)
    w[0, :6] = [0.5, 1.5, 2.5, -2.5, -3.0, 3.0]
    w[0, 6] = -0.5
    pk, sc = F.quant_int3_g64(w)
    assert sc[0, 0] == 1.0
    u = unpack_planes(pk, 1, 1)[0, 0]
    assert (u[:7].astype(int) - 4).tolist() == [0, 2, 2, -2, -3, 3, 0]


def unpack_planes(pk, O, G):
    """The bit-plane layout read with numpy's unpackbits (little-endian bit order)."""
    b = pk.reshape(O, G, 3, 8)
    bits = np.unpackbits(b, axis=3, bitorder="little")  # [O, G, 3, 64]
    return bits[:, :, 0] | (bits[:, :, 1] << 1) | (bits[:, :, 2] << 2)


def test_int3_non_finite_group():
    w = np.ones((1, 128), np.float32)
    w[0, 70] = np.nan
    pk, sc = F.quant_int3_g64(w)
    assert sc[0, 0] == np.float32(1 / 3) and np.isnan(sc[0, 1])
    assert np.all(unpack_planes(pk, 1, 2)[0, 1] == 4)


# ---------------------------------------------------------------- fp8-e4m3-b128

def test_fp8_tiles_and_scales():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((200, 300)) * 0.02).astype(np.float32)
    codes, sc = F.quant_fp8_b128(w)
    assert codes.shape == (200, 300) and sc.shape == (2, 3)
    for a in range(2):
        for b in range(3):
            tile = w[128 * a:128 * (a + 1), 128 * b:128 * (b + 1)]
            s = np.float32(np.abs(tile).max() / np.float32(448))
            assert sc[a, b] == s
            r = np.clip((tile / s).astype(np.float32), -448, 448)
            ref = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[128 * a:128 * (a + 1), 128 * b:128 * (b + 1)], ref)
    W = F.dequant_fp8_b128(codes, sc)
    rel = np.abs(W - w) / np.maximum(np.abs(w), 1e-30)
    big = np.abs(w) > np.repeat(np.repeat(sc, 128, 0), 128, 1)[:200, :300] * 2.0 ** -6
    assert rel[big].max() <= 2.0 ** -4  # 3 mantissa bits: half an ulp is 2^-4 relative


def test_fp8_zero_and_non_finite_tiles():
    w = np.zeros((130, 10), np.float32)
    w[129, 3] = np.inf
    codes, sc = F.quant_fp8_b128(w)
    assert sc[0, 0] == 0 and np.isnan(sc[1, 0]) and not codes.any()


# ---------------------------------------------------------------- product

def test_matvec_exact_rational():
    rng = np.random.default_rng(9)
    for fmt in (5, 7, 8):
        w = (rng.standard_normal((3, 70)) * 0.02).astype(np.float32)
        pk, sc = F.quant(fmt, w)
        W = F.dequant(fmt, pk, sc, 3, 70)
        x = rng.standard_normal((2, 70)).astype(np.float32)
        y = F.matvec(W, x)
        for t in range(2):
            for o in range(3):
                exact = sum(Fraction(float(W[o, i])) * Fraction(float(x[t, i]))
                            for i in range(70))
                assert abs(Fraction(float(y[t, o])) - exact) <= abs(exact) * Fraction(1, 2 ** 45) \
                    + Fraction(1, 2 ** 80)


# ---------------------------------------------------------------- a layer in a format

def test_layer_in_int4_matches_the_c_oracle():
    """The format layer (numpy composition) with int4-g64 experts equals the C
    oracle's fp64 layer on the same bytes: two independent statements of the same
    routing and FFN."""
    import oracle
    rng = np.random.default_rng(12)
    H, I, E, K, T = 128, 64, 8, 3, 4
    ws = [[(rng.standard_normal(s) * 0.02).astype(np.float32) for s in ((I, H), (I, H), (H, I))]
          for _ in range(E + 1)]
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    fx = [F.quant_expert(4, *w) for w in ws]
    cx = [oracle.Expert(fx[e][0][0], fx[e][0][1], fx[e][1][0], fx[e][1][1], fx[e][2][0],
                        fx[e][2][1]) for e in range(E + 1)]
    for scoring, bias in ((0, None), (1, (rng.standard_normal(E) * 0.1).astype(np.float32))):
        y1, i1, g1 = F.moe_forward_fmt(4, x, wr, bias, fx[:E], fx[E], H, I, K, scoring)
        y2, i2, g2 = oracle.moe_forward(x, wr, bias, cx[:E], cx[E], H, I, K, scoring)
        assert np.array_equal(i1, i2)
        assert np.allclose(g1, g2, rtol=1e-14, atol=0)
        assert np.allclose(y1, y2, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("fmt", (5, 7, 8))
def test_layer_closed_forms(fmt):
    rng = np.random.default_rng(13)
    H, I, E, K, T = 128, 64, 6, 2, 3
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    zero = F.quant_expert(fmt, np.zeros((I, H), np.float32), np.zeros((I, H), np.float32),
                          np.zeros((H, I), np.float32))
    y, idx, g = F.moe_forward_fmt(fmt, x, wr, None, [zero] * E, zero, H, I, K)
    assert not y.any()  # all-zero experts give y = 0
    assert np.allclose(g.sum(axis=1), 1.0)
    # the composition itself is the one pinned against the C oracle with int4 experts;
    # here each format's dequantised matrices enter it (dequant is pinned above)
