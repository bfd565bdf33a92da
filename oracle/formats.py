"""The oracle of the sibling weight formats: the byte arithmetic of the format
registry, format inference from byte counts, and the int3-g64, MXFP4 and
fp8-e4m3-b128 quantisers, their dequantisers and the matrix-vector product.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): only the tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.

Sources (page titles and sections):
* "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战", section 权重转换: the
  registry (0 f32, 1 int8-row, 2 int4-row, 3 int2-row, 4 int4-grouped, 5 int3-g64,
  6 E8/IQ3, 7 MXFP4, 8 fp8-e4m3-b128), and the rule that a tensor's format follows
  from its weight byte count, its scale byte count and its [O, I] shape alone.
* "Colibrì 深度解析", section 十五 (issue 1434): raw f32 has no scale array;
  section 八: int3 with a per-group scale costs 3.5 bits per weight; section 十: the
  quantised matrix kernels, from int4 up to MXFP4.
* MXFP4: the OCP Microscaling Formats (MX) specification v1.0: blocks of 32 FP4
  E2M1 elements share one E8M0 scale 2^(E - 127); the conversion from fp32 takes
  the shared exponent floor(log2(max |v|)) minus the element format's largest
  exponent (2 for E2M1), then rounds each v / 2^shared to the element format,
  to nearest even, saturating at the largest normal (6).
* fp8 e4m3: the OCP 8-bit floating point specification: E4M3 with bias 7, no
  infinities, largest finite 448, smallest subnormal 2^-9.

Readings, where the pages give a format's name only:
* F1 sizes, G = ceil(I / 64): 0 f32: 4 O I bytes, no scales; 1 int8-row: O I, f32
  per row; 2 int4-row: O ceil(I/2), f32 per row; 3 int2-row: O ceil(I/4), f32 per
  row; 4 int4-g64: 32 O G, f32 per group; 5 int3-g64: 24 O G (64 three-bit codes),
  f32 per group; 6 E8/IQ3: layout unknown, never inferred; 7 MXFP4: 16 O ceil(I/32),
  one E8M0 byte per 32-block; 8 fp8-e4m3-b128: O I bytes, one f32 per 128 x 128
  tile (the block shape of the fp8 checkpoints of the model families the pages run).
* F2 inference: the formats whose two byte counts match; exactly one is the answer,
  none or several is an error (fail closed), with the candidates reported.
* F3 int3-g64, by analogy with the int4-g64 rule: s = fl32(amax / 3); q =
  clip(rint_even(fl32(w / s)), -4, 3), u = q + 4 (all u = 4 when s = 0); a group's 24
  bytes are three little-endian 64-bit bit planes: bit j of plane p is bit p of u[j].
  As for int4-g64, a group holding a non-finite value gets a NaN scale and all u = 4.
* F4 MXFP4 packing: byte j of a block holds element 2j in its low nibble and
  element 2j + 1 in its high nibble; nibble = sign << 3 | E2M1 magnitude code; the
  sign is the sign bit of fl32(v / X); an all-zero block has E = 0; a block with a
  non-finite value has E = 255 (the NaN scale).
* F5 fp8-e4m3-b128: s = fl32(amax / 448) over the tile; code = E4M3 round to
  nearest even of fl32(w / s), saturated at 448, sign from fl32(w / s); all codes 0
  when s = 0, and a NaN scale with all codes 0 when the tile holds a non-finite value.
The matrix-vector product y[t, o] = sum_i W^[o, i] x[t, i] is fp64 on the exactly
dequantised W^.
"""
from __future__ import annotations

import math

import numpy as np

NAMES = {0: "f32", 1: "int8-row", 2: "int4-row", 3: "int2-row", 4: "int4-g64",
         5: "int3-g64", 6: "e8-iq3", 7: "mxfp4", 8: "fp8-e4m3-b128"}


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def sizes(fmt: int, O: int, I: int):
    """(weight bytes, scale bytes) of an [O, I] tensor in `fmt`, or None (F1)."""
    G = _cdiv(I, 64)
    table = {
        0: (4 * O * I, 0),
        1: (O * I, 4 * O),
        2: (O * _cdiv(I, 2), 4 * O),
        3: (O * _cdiv(I, 4), 4 * O),
        4: (32 * O * G, 4 * O * G),
        5: (24 * O * G, 4 * O * G),
        7: (16 * O * _cdiv(I, 32), O * _cdiv(I, 32)),
        8: (O * I, 4 * _cdiv(O, 128) * _cdiv(I, 128)),
    }
    return table.get(fmt)


def resolve(O: int, I: int, weight_bytes: int, scale_bytes: int):
    """-> (fmt or None, sorted candidate list) (F2)."""
    cands = [f for f in NAMES if sizes(f, O, I) == (weight_bytes, scale_bytes)]
    return (cands[0] if len(cands) == 1 else None), cands


# ---------------------------------------------------------------- element formats

def _e4m3_table() -> np.ndarray:
    """Magnitudes of the E4M3 codes 0..126 (127 is NaN), from the definition."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3 = _e4m3_table()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _nearest_even_code(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Code of the table value nearest to each magnitude (ascending table), ties to
    the even code; magnitudes beyond the last value take the last code."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(table, mag, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dl = np.abs(mag - table[lo])
    dh = np.abs(table[hi] - mag)
    code = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    return np.where(mag >= table[-1], len(table) - 1, code).astype(np.int64)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> E4M3 bytes: round to nearest even, saturate at 448 (F5)."""
    v = np.asarray(v, dtype=np.float32)
    sign = np.signbit(v).astype(np.int64) << 7
    code = _nearest_even_code(np.abs(v.astype(np.float64)), E4M3)
    out = sign | code
    return np.where(np.isnan(v), 0x7F | sign, out).astype(np.uint8)


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.int64)
    mag = np.where((b & 0x7F) == 0x7F, np.nan, E4M3[np.minimum(b & 0x7F, 126)])
    return np.where(b & 0x80, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> 4-bit E2M1 codes (sign << 3 | magnitude code), saturating."""
    v = np.asarray(v, dtype=np.float32)
    sign = np.signbit(v).astype(np.int64) << 3
    return (sign | _nearest_even_code(np.abs(v.astype(np.float64)), E2M1)).astype(np.uint8)


def e2m1_decode(c: np.ndarray) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    mag = E2M1[c & 7]
    return np.where(c & 8, -mag, mag)


# ---------------------------------------------------------------- int3-g64 (fmt 5)

def _rint_even_f32(q: np.ndarray) -> np.ndarray:
    return np.rint(q)  # numpy rounds half to even


def quant_int3_g64(w: np.ndarray):
    """fp32 [O, I] -> (packed uint8 [O, 24 G], scales f32 [O, G]) (F3)."""
    w = np.asarray(w, dtype=np.float32)
    O, I = w.shape
    G = _cdiv(I, 64)
    pad = np.zeros((O, G * 64), dtype=np.float32)
    pad[:, :I] = w
    grp = pad.reshape(O, G, 64)
    finite = np.isfinite(grp).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(grp), grp, 0)).max(axis=2), 0)
    s = (amax.astype(np.float32) / np.float32(3.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = (grp / s[:, :, None]).astype(np.float32)
    q = np.clip(_rint_even_f32(np.where(np.isfinite(qf), qf, 0)), -4, 3)
    neutral = (s[:, :, None] == 0) | ~finite[:, :, None]
    u = np.where(neutral, 4, q + 4).astype(np.uint64)
    s = np.where(finite, s, np.float32(np.nan)).astype(np.float32)
    packed = np.zeros((O, G, 24), dtype=np.uint8)
    for p in range(3):
        plane = np.zeros((O, G), dtype=np.uint64)
        for j in range(64):
            plane |= ((u[:, :, j] >> np.uint64(p)) & np.uint64(1)) << np.uint64(j)
        for byte in range(8):
            packed[:, :, 8 * p + byte] = ((plane >> np.uint64(8 * byte)) & np.uint64(0xFF))
    return packed.reshape(O, G * 24), s


def dequant_int3_g64(packed: np.ndarray, scales: np.ndarray, I: int) -> np.ndarray:
    O, G = scales.shape
    pk = packed.reshape(O, G, 24).astype(np.uint64)
    u = np.zeros((O, G, 64), dtype=np.int64)
    for p in range(3):
        plane = np.zeros((O, G), dtype=np.uint64)
        for byte in range(8):
            plane |= pk[:, :, 8 * p + byte] << np.uint64(8 * byte)
        for j in range(64):
            u[:, :, j] |= (((plane >> np.uint64(j)) & np.uint64(1)).astype(np.int64)) << p
    w = scales.astype(np.float64)[:, :, None] * (u - 4).astype(np.float64)
    return w.reshape(O, G * 64)[:, :I]


# ---------------------------------------------------------------- MXFP4 (fmt 7)

def quant_mxfp4(w: np.ndarray):
    """fp32 [O, I] -> (packed uint8 [O, 16 NB], E8M0 scales uint8 [O, NB]) (F4)."""
    w = np.asarray(w, dtype=np.float32)
    O, I = w.shape
    NB = _cdiv(I, 32)
    pad = np.zeros((O, NB * 32), dtype=np.float32)
    pad[:, :I] = w
    blk = pad.reshape(O, NB, 32)
    finite = np.isfinite(blk).all(axis=2)
    amax = np.where(finite, np.abs(np.where(np.isfinite(blk), blk, 0)).max(axis=2), 0)
    m, ex = np.frexp(amax.astype(np.float64))        # amax = m 2^ex, m in [0.5, 1)
    shared = np.clip((ex - 1) - 2, -127, 127)        # floor(log2 amax) - 2
    E = np.where(~finite, 255, np.where(amax == 0, 0, shared + 127)).astype(np.uint8)
    # v / 2^shared, exact: a multiplication by the normal number 2^-shared
    inv = np.ldexp(np.float32(1.0), (-shared).astype(np.int32)).astype(np.float32)
    r = (blk * inv[:, :, None]).astype(np.float32)
    codes = e2m1_encode(r).astype(np.int64)
    codes[~finite | (amax == 0)] = 0
    packed = (codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)).astype(np.uint8)
    return packed.reshape(O, NB * 16), E


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray, I: int) -> np.ndarray:
    O, NB = scales.shape
    pk = packed.reshape(O, NB, 16).astype(np.int64)
    codes = np.zeros((O, NB, 32), dtype=np.int64)
    codes[:, :, 0::2] = pk & 0xF
    codes[:, :, 1::2] = pk >> 4
    X = np.where(scales == 255, np.nan, np.ldexp(1.0, scales.astype(np.int64) - 127))
    w = X[:, :, None] * e2m1_decode(codes)
    return w.reshape(O, NB * 32)[:, :I]


# ---------------------------------------------------------------- fp8-e4m3-b128 (fmt 8)

def quant_fp8_b128(w: np.ndarray):
    """fp32 [O, I] -> (codes uint8 [O, I], scales f32 [ceil(O/128), ceil(I/128)]) (F5)."""
    w = np.asarray(w, dtype=np.float32)
    O, I = w.shape
    TO, TI = _cdiv(O, 128), _cdiv(I, 128)
    codes = np.zeros((O, I), dtype=np.uint8)
    scales = np.zeros((TO, TI), dtype=np.float32)
    for a in range(TO):
        for b in range(TI):
            tile = w[128 * a:128 * (a + 1), 128 * b:128 * (b + 1)]
            if not np.isfinite(tile).all():
                scales[a, b] = np.nan
                continue
            amax = np.abs(tile).max()
            s = np.float32(amax / np.float32(448.0))
            scales[a, b] = s
            if s == 0:
                continue
            with np.errstate(divide="ignore", invalid="ignore"):
                r = (tile / s).astype(np.float32)
            codes[128 * a:128 * (a + 1), 128 * b:128 * (b + 1)] = e4m3_encode(r)
    return codes, scales


def dequant_fp8_b128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    O, I = codes.shape
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=0), 128, axis=1)[:O, :I]
    return s * e4m3_decode(codes)


# ---------------------------------------------------------------- product

def dequant(fmt: int, packed, scales, O: int, I: int) -> np.ndarray:
    if fmt == 5:
        return dequant_int3_g64(packed, scales, I)
    if fmt == 7:
        return dequant_mxfp4(packed, scales, I)
    if fmt == 8:
        return dequant_fp8_b128(packed, scales)
    raise ValueError(f"no dequantiser for fmt {fmt} here")


def quant(fmt: int, w):
    return {5: quant_int3_g64, 7: quant_mxfp4, 8: quant_fp8_b128}[fmt](w)


def matvec(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y [T, O] = x [T, I] W^T in fp64 (W already dequantised)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


# ---------------------------------------------------------------- a layer in a format

def quant_expert(fmt: int, wg, wu, wd):
    """The three matrices of one expert in fmt: [(packed, scales)] for gate [I, H],
    up [I, H], down [H, I]."""
    if fmt == 4:
        import oracle
        return [oracle.quant_int4_g64(w)[:2] for w in (wg, wu, wd)]
    return [quant(fmt, w) for w in (wg, wu, wd)]


def dequant_expert(fmt: int, ex, H: int, I: int):
    """-> (Wg [I, H], Wu [I, H], Wd [H, I]) fp64, exactly dequantised."""
    shapes = ((I, H), (I, H), (H, I))
    out = []
    for (pk, sc), (O, C) in zip(ex, shapes):
        if fmt == 4:
            import oracle
            out.append(oracle.dequant_int4_g64(pk, sc, C))
        else:
            out.append(dequant(fmt, pk, sc, O, C))
    return out


def moe_forward_fmt(fmt: int, x, wr, bias, experts: list, shared, H: int, I: int, K: int,
                    scoring: int = 0):
    """The layer with its experts in fmt: the routing of the oracle's layer (softmax
    or sigmoid scoring), then per token y = sum_k g_k FFN_{e_k}(x) + FFN_shared(x),
    FFN(x) = Wd (silu(Wg x) * (Wu x)), silu(z) = z / (1 + e^-z), all fp64 on the
    exactly dequantised matrices.  experts: E entries of quant_expert output (None
    where unused).  -> (y fp64 [T, H], idx [T, K], gates fp64 [T, K])."""
    import oracle
    logits = oracle.router_logits(x, wr, bias if scoring == 0 else None)
    if scoring == 0:
        idx, gates, _ = oracle.topk(logits, K)
    else:
        idx, gates, _ = oracle.topk_sigmoid(logits, K, bias)
    xf = np.asarray(x, dtype=np.float64) if np.asarray(x).dtype != np.uint16 else \
        (np.asarray(x, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)

    deq = {}  # each expert's matrices dequantised once per call

    def ffn(ex, v):
        if id(ex) not in deq:
            deq[id(ex)] = dequant_expert(fmt, ex, H, I)
        Wg, Wu, Wd = deq[id(ex)]
        g = Wg @ v
        u = Wu @ v
        return Wd @ (g / (1.0 + np.exp(-g)) * u)

    T = xf.shape[0]
    y = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            ex = experts[int(idx[t, k])]
            if ex is None:
                raise ValueError("a selected expert was not supplied")
            y[t] += gates[t, k] * ffn(ex, xf[t])
        y[t] += ffn(shared, xf[t])
    return y, idx, gates
