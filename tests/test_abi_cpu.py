"""Host-side checks of the C ABI (no GPU): the library loads, exports every symbol
include/coli.h declares, the format arithmetic is right, and argument errors are
rejected on the host before any HIP call (fail closed)."""
import ctypes
import os
import re

import pytest

import int4_grouped_expert_amd as coli

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "coli.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(coli_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(coli.lib, n), n
    assert sorted(coli.EXPORTS) == names


def test_strerror_covers_codes():
    for c in range(-10, 1):
        assert coli.lib.coli_strerror(c)
    assert coli.lib.coli_strerror(-99) == b"unknown status"


def test_format_sizes():
    assert coli.coli_int4_g64_packed_bytes(2048, 6144) == 6291456
    assert coli.coli_int4_g64_scale_count(2048, 6144) == 196608
    assert coli.coli_int4_g64_packed_bytes(3, 65) == 3 * 2 * 32
    assert coli.coli_int4_g64_packed_bytes(0, 10) == 0
    assert coli.coli_int4_g64_packed_bytes(4, 0) == 0
    # 21,233,664 bytes per expert at H=6144, I=2048 (nibbles + fp32 scales), plus
    # the scales again group-major and blocked by 8 rows (6 x 786,432) and the
    # 256-byte finish tag section
    assert coli.coli_expert_blob_bytes(6144, 2048) == 21233664 + 6 * 786432 + 256
    assert coli.coli_expert_blob_bytes(256, 128) == 55296 + 6 * 2048 + 256
    assert coli.coli_expert_blob_bytes(0, 128) == 0
    # ragged shapes: ceil(cols / 64) groups per row, every section 256-byte aligned
    nb = coli.coli_expert_blob_bytes(200, 72)
    assert nb > 0 and nb % 256 == 0


def test_expert_views_offsets():
    base = 1 << 40
    (gq, gs), (uq, us), (dq, ds) = coli.coli_expert_views(base, 6144, 2048)
    assert gq - base == 0 and uq - base == 6291456 and dq - base == 2 * 6291456
    assert gs - base == 3 * 6291456 and us - gs == 786432 and ds - us == 786432
    for a in (gq, gs, uq, us, dq, ds):
        assert (a - base) % 256 == 0


def test_expert_finish_rejects_before_launch():
    L = coli.lib
    assert L.coli_expert_finish(None, 256, 128, None) == coli.COLI_EINVAL
    assert L.coli_expert_finish(ctypes.c_void_p(1 << 40), 0, 128, None) == coli.COLI_ESHAPE
    assert L.coli_expert_finish(ctypes.c_void_p(1 << 40), 256, 1 << 20, None) == coli.COLI_ESHAPE
    assert L.coli_expert_finish(ctypes.c_void_p((1 << 40) + 64), 256, 128, None) == coli.COLI_EALIGN


def test_workspace_bytes():
    lay = coli.coli_moe_layer(6144, 2048, 256, 8, 1 << 20, coli.COLI_BF16, None, 1 << 30, 1 << 31)
    d = coli.lib.coli_moe_workspace_bytes(ctypes.byref(lay), 1, coli.COLI_DECODE)
    assert d >= (8 + 1) * 2048 * 4
    p = coli.lib.coli_moe_workspace_bytes(ctypes.byref(lay), 2048, coli.COLI_PREFILL)
    assert p >= (2048 * 9) * (2048 + 6144) * 2
    # decode beyond 256 tokens runs in 256-token sub-batches: the workspace of one
    d256 = coli.lib.coli_moe_workspace_bytes(ctypes.byref(lay), 256, coli.COLI_DECODE)
    assert coli.lib.coli_moe_workspace_bytes(ctypes.byref(lay), 257, coli.COLI_DECODE) == d256
    assert coli.lib.coli_moe_workspace_bytes(ctypes.byref(lay), 5000, coli.COLI_DECODE) == d256
    bad = coli.coli_moe_layer(6144, 2048, 256, 300, 1, 1, None, 1, 1)
    assert coli.lib.coli_moe_workspace_bytes(ctypes.byref(bad), 1, coli.COLI_DECODE) == 0


def test_buffer_offset_limit_rejected_before_launch():
    """A prefill of 65536 tokens of the decode-shaped layer would need (T*K + T) *
    I * 2 = 2.4e9 bytes of staged h: past the kernels' 2^31 buffer offsets.  The
    size query says 0 and the forward returns ESHAPE before any launch (the
    pointers here are not device memory: a launch would fault)."""
    L = coli.lib
    lay = coli.coli_moe_layer(6144, 2048, 256, 8, 1 << 20, coli.COLI_BF16, None, 1 << 30, 1 << 31)
    assert L.coli_moe_workspace_bytes(ctypes.byref(lay), 65536, coli.COLI_PREFILL) == 0
    assert L.coli_moe_workspace_bytes(ctypes.byref(lay), 8192, coli.COLI_PREFILL) > 0
    a = P(1 << 20)
    rc = L.coli_moe_forward(ctypes.byref(lay), coli.COLI_PREFILL, a, 65536, a, None, None, None,
                            a, 1 << 40, None)
    assert rc == coli.COLI_ESHAPE


P = ctypes.c_void_p


def test_quant_rejects_before_launch():
    L = coli.lib
    a = P(4096)
    assert L.coli_quant_int4_g64(None, 1, 64, a, a, None, None) == coli.COLI_EINVAL
    assert L.coli_quant_int4_g64(None, 0, 64, None, None, None, None) == coli.COLI_OK
    assert L.coli_quant_int4_g64(a, -1, 64, a, a, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_int4_g64(a, 1, 0, a, a, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_int4_g64(P(4098), 1, 64, a, a, None, None) == coli.COLI_EALIGN
    assert L.coli_quant_int4_g64(a, 1, 64, P(4100), a, None, None) == coli.COLI_EALIGN
    assert L.coli_quant_int4_g64(a, 0, 64, a, a, None, None) == coli.COLI_OK  # no-op


def test_router_rejects_before_launch():
    L = coli.lib
    a = P(4096)
    ok = dict(T=1, H=64, E=16, K=4)

    def call(T=1, H=64, E=16, K=4, x=a, xd=0, wd=0, idx=a):
        return L.coli_router_topk(x, xd, T, H, a, wd, E, None, K, idx, a, a, None)
    assert call(x=None) == coli.COLI_EINVAL
    assert call(idx=None) == coli.COLI_EINVAL
    assert call(K=17) == coli.COLI_ESHAPE
    assert call(K=0) == coli.COLI_ESHAPE
    assert call(E=1025, K=4) == coli.COLI_ESHAPE
    assert call(H=0) == coli.COLI_ESHAPE
    assert call(T=-1) == coli.COLI_ESHAPE
    assert call(xd=7) == coli.COLI_EDTYPE
    assert call(x=P(4098)) == coli.COLI_EALIGN  # fp32 x: 4-byte aligned
    assert call(x=P(4098), xd=1, T=0) == coli.COLI_OK  # bf16 x: 2-byte aligned
    assert call(T=0) == coli.COLI_OK
    # scoring: unknown values are rejected
    assert L.coli_router_topk_scored(a, 0, 1, 64, a, 0, 16, None, 4, 7, a, a, a, None) == \
        coli.COLI_EINVAL
    assert L.coli_router_topk_scored(a, 0, 0, 64, a, 0, 16, None, 4, 1, a, a, None, None) == \
        coli.COLI_OK
    del ok


def test_permute_rejects_before_launch():
    L = coli.lib
    a = P(4096)
    assert L.coli_expert_permute(None, 1, 2, 8, a, a, a, a, a, None, 0, None) == coli.COLI_EINVAL
    assert L.coli_expert_permute(a, 1, 9, 8, a, a, a, a, a, None, 0, None) == coli.COLI_ESHAPE
    need = coli.coli_expert_permute_workspace_bytes(2048, 8, 256)
    assert need == 64 * 256 * 4  # one count per (256-pair chunk, expert)
    assert coli.coli_expert_permute_workspace_bytes(32, 8, 256) == 0
    assert coli.coli_expert_permute_workspace_bytes(32, 9, 8) == 0  # K > E: invalid
    assert (L.coli_expert_permute(a, 2048, 8, 256, a, a, a, a, a, None, 0, None)
            == coli.COLI_EWORKSPACE)
    assert (L.coli_expert_permute(a, 2048, 8, 256, a, a, a, a, a, a, need - 4, None)
            == coli.COLI_EWORKSPACE)


def test_forward_rejects_before_launch():
    L = coli.lib
    a = P(1 << 20)
    lay = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22)
    need = L.coli_moe_workspace_bytes(ctypes.byref(lay), 1, coli.COLI_DECODE)

    def call(layer=lay, mode=coli.COLI_DECODE, x=a, T=1, y=a, ws=a, nb=need, st=None):
        return L.coli_moe_forward(ctypes.byref(layer), mode, x, T, y, None, None, st, ws, nb,
                                  None)
    assert call(x=None) == coli.COLI_EINVAL
    assert call(mode=5) == coli.COLI_EINVAL
    assert call(T=65537) == coli.COLI_ESHAPE
    assert call(st=P((1 << 20) + 2)) == coli.COLI_EALIGN
    assert call(ws=None) == coli.COLI_EWORKSPACE
    assert call(nb=need - 1) == coli.COLI_EWORKSPACE
    assert call(x=P((1 << 20) + 8)) == coli.COLI_EALIGN
    assert call(ws=P((1 << 20) + 128)) == coli.COLI_EALIGN
    assert call(T=0) == coli.COLI_OK
    assert call(T=0, x=None, y=None) == coli.COLI_OK
    for H, I, E, K in [(0, 128, 16, 4), (256, 0, 16, 4), (256, 128, 0, 1), (256, 128, 16, 17),
                       (256, 128, 2000, 4), (70000, 128, 16, 4)]:
        bad = coli.coli_moe_layer(H, I, E, K, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22)
        assert call(layer=bad) == coli.COLI_ESHAPE
    badsc = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22, 5)
    assert call(layer=badsc) == coli.COLI_EINVAL
    unal = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, coli.COLI_F32, None, (1 << 21) + 64,
                               1 << 22)
    assert call(layer=unal) == coli.COLI_EALIGN
    badt = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, 3, None, 1 << 21, 1 << 22)
    assert call(layer=badt) == coli.COLI_EDTYPE
    badu = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22,
                               0, None, (1 << 23) + 4)
    assert call(layer=badu) == coli.COLI_EALIGN  # routing-history counters: 8-byte aligned


def test_two_phase_rejects_before_launch():
    L = coli.lib
    a = P(1 << 20)
    lay = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22)
    need = L.coli_moe_workspace_bytes(ctypes.byref(lay), 8, coli.COLI_DECODE)

    def route(layer=lay, mode=coli.COLI_DECODE, x=a, T=8, ws=a, nb=need, u=None):
        return L.coli_moe_route(ctypes.byref(layer), mode, x, T, None, None, u, None, ws, nb,
                                None)

    def experts(layer=lay, mode=coli.COLI_DECODE, x=a, T=8, y=a, ws=a, nb=need):
        return L.coli_moe_experts(ctypes.byref(layer), mode, x, T, y, None, None, None, ws, nb,
                                  None)
    for f in (route, experts):
        assert f(x=None) == coli.COLI_EINVAL
        assert f(mode=7) == coli.COLI_EINVAL
        assert f(ws=None) == coli.COLI_EWORKSPACE
        assert f(nb=need - 1) == coli.COLI_EWORKSPACE
        assert f(T=257) == coli.COLI_ESHAPE  # decode: one chunk of at most 256 tokens
        assert f(T=0) == coli.COLI_OK
    assert experts(y=None) == coli.COLI_EINVAL
    assert route(u=P((1 << 20) + 2)) == coli.COLI_EALIGN
    sm = coli.coli_moe_layer(256, 128, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22,
                             0, (1 << 23) + 2)
    assert route(layer=sm) == coli.COLI_EALIGN
    assert experts(layer=sm) == coli.COLI_EALIGN


def test_format_bytes_and_inference_match_the_oracle():
    """The registry's byte arithmetic and inference from byte counts are host code:
    they must agree with the oracle on every shape, including the ambiguous ones."""
    from oracle import formats as F
    rng = __import__("numpy").random.default_rng(11)
    shapes = [(2048, 6144), (6144, 2048), (1, 1), (1, 100), (10, 64), (3, 128), (72, 200),
              (129, 257), (1000, 330), (65536, 128)]
    shapes += [(int(rng.integers(1, 5000)), int(rng.integers(1, 9000))) for _ in range(200)]
    for O, I in shapes:
        for fmt in range(9):
            want = F.sizes(fmt, O, I)
            if want is None:
                with pytest.raises(coli.ColiError):
                    coli.coli_fmt_bytes(fmt, O, I)
                continue
            assert coli.coli_fmt_bytes(fmt, O, I) == want
            assert coli.coli_resolve_fmt(O, I, *want) == F.resolve(O, I, *want)
        assert coli.coli_resolve_fmt(O, I, 7, 3) == (None, [])
    assert coli.lib.coli_resolve_fmt(0, 5, 0, 0, None) == coli.COLI_ESHAPE
    assert coli.coli_resolve_fmt(10, 64, 320, 40) == (None, [2, 4])


def test_format_calls_reject_before_launch():
    L = coli.lib
    a = P(1 << 20)
    assert L.coli_quant_fmt(5, None, 4, 64, a, a, None, None) == coli.COLI_EINVAL
    assert L.coli_quant_fmt(6, a, 4, 64, a, a, None, None) == coli.COLI_EINVAL
    assert L.coli_quant_fmt(1, a, 4, 64, a, a, None, None) == coli.COLI_EINVAL
    assert L.coli_quant_fmt(5, a, 0, 64, a, a, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_fmt(5, a, 4, 65537, a, a, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_fmt(5, a, 4, 64, P((1 << 20) + 4), a, None, None) == coli.COLI_EALIGN
    assert L.coli_quant_fmt(7, P((1 << 20) + 2), 4, 64, a, a, None, None) == coli.COLI_EALIGN

    def mv(fmt=7, O=16, I=6144, x=a, T=1, y=a, pk=a):
        return L.coli_matvec_fmt(fmt, pk, a, O, I, x, T, y, None)
    assert mv(x=None) == coli.COLI_EINVAL
    assert mv(fmt=6) == coli.COLI_EINVAL and mv(fmt=0) == coli.COLI_EINVAL
    assert mv(T=9) == coli.COLI_ESHAPE and mv(T=-1) == coli.COLI_ESHAPE
    assert mv(T=5) == coli.COLI_ESHAPE  # 5 x 6144 floats exceed the x stage
    assert mv(fmt=8, I=100) == coli.COLI_ESHAPE  # fp8 rows must be 16-byte multiples
    assert mv(pk=P((1 << 20) + 8)) == coli.COLI_EALIGN
    assert mv(T=0, x=None, y=None) == coli.COLI_OK


def test_format_layer_rejects_before_launch():
    L = coli.lib
    a = P(1 << 20)
    lay = coli.coli_moe_layer(512, 512, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22)
    need = L.coli_moe_fmt_workspace_bytes(ctypes.byref(lay), 7, 2)
    assert need > 0
    assert L.coli_moe_fmt_workspace_bytes(ctypes.byref(lay), 6, 2) == 0
    assert L.coli_moe_fmt_workspace_bytes(ctypes.byref(lay), 7, 5) == 0  # T <= 4

    def fwd(layer=lay, fmt=7, x=a, T=2, y=a, ws=a, nb=need):
        return L.coli_moe_forward_fmt(ctypes.byref(layer), fmt, x, T, y, None, None, None, ws, nb,
                                      None)
    assert fwd(fmt=1) == coli.COLI_EINVAL and fwd(fmt=6) == coli.COLI_EINVAL
    assert fwd(x=None) == coli.COLI_EINVAL
    assert fwd(T=5) == coli.COLI_ESHAPE
    assert fwd(nb=need - 1) == coli.COLI_EWORKSPACE
    assert fwd(T=0) == coli.COLI_OK
    sm = coli.coli_moe_layer(512, 512, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22,
                             0, 1 << 23)
    assert fwd(layer=sm) == coli.COLI_EINVAL  # no slot map on this path
    big = coli.coli_moe_layer(6144, 2048, 256, 8, 1 << 20, coli.COLI_BF16, None, 1 << 21, 1 << 22)
    assert L.coli_moe_fmt_workspace_bytes(ctypes.byref(big), 8, 4) > 0
    assert L.coli_moe_forward_fmt(ctypes.byref(big), 8, a, 5, a, None, None, None, a, 1 << 30,
                                  None) == coli.COLI_ESHAPE
    ragged = coli.coli_moe_layer(200, 72, 16, 4, 1 << 20, coli.COLI_F32, None, 1 << 21, 1 << 22)
    assert L.coli_moe_fmt_workspace_bytes(ctypes.byref(ragged), 8, 1) == 0  # fp8: 16-byte rows
    assert L.coli_moe_fmt_workspace_bytes(ctypes.byref(ragged), 5, 1) > 0
    assert coli.coli_fmt_blob_bytes(6, 512, 512) == 0
    from oracle import formats as F
    for fmt in (4, 5, 7, 8):
        H, I = 6144, 2048
        parts = [F.sizes(fmt, I, H)] * 2 + [F.sizes(fmt, H, I)]
        a256 = lambda n: (n + 255) // 256 * 256
        want = sum(a256(w) for w, _ in parts) + sum(a256(max(s, 1)) for _, s in parts)
        assert coli.coli_fmt_blob_bytes(fmt, H, I) == want


def test_quant_many_rejects_before_launch():
    L = coli.lib
    a = P(1 << 20)
    assert L.coli_quant_int4_g64_many(None, a, a, 3, 64, 64, None, None) == coli.COLI_EINVAL
    assert L.coli_quant_int4_g64_many(a, a, a, -1, 64, 64, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_int4_g64_many(a, a, a, 70000, 64, 64, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_int4_g64_many(a, a, a, 3, 64, 0, None, None) == coli.COLI_ESHAPE
    assert L.coli_quant_int4_g64_many(P((1 << 20) + 4), a, a, 3, 64, 64, None, None) == \
        coli.COLI_EALIGN
    assert L.coli_quant_int4_g64_many(a, a, a, 0, 64, 64, None, None) == coli.COLI_OK
    assert L.coli_quant_int4_g64_many(a, a, a, 3, 0, 64, None, None) == coli.COLI_OK


def test_rmsnorm_rejects():
    L = coli.lib
    a = P(4096)
    assert L.coli_rmsnorm_f32(None, a, 1, 8, 1e-6, None) == coli.COLI_EINVAL
    assert L.coli_rmsnorm_f32(a, a, 1, 8, -1.0, None) == coli.COLI_EINVAL
    assert L.coli_rmsnorm_f32(a, a, 1, 8, float("nan"), None) == coli.COLI_EINVAL
    assert L.coli_rmsnorm_f32(a, a, 1, 0, 1e-6, None) == coli.COLI_ESHAPE
    assert L.coli_rmsnorm_f32(a, a, 0, 8, 1e-6, None) == coli.COLI_OK


def test_product_does_not_import_oracle():
    import sys
    pkg = os.path.join(ROOT, "int4_grouped_expert_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.replace("oracle is", ""), f
    assert "int4_grouped_expert_amd" in sys.modules


def test_noalloc_rejects_before_launch():
    """The no-alloc forward reports argument errors as coli_moe_forward does, and a
    call whose workspace exceeds the static scratch with ESCRATCH, before any HIP
    call (the pointers here are not device memory)."""
    L = coli.lib
    a = P(1 << 20)
    lay = coli.coli_moe_layer(6144, 2048, 256, 8, 1 << 20, coli.COLI_BF16, None, 1 << 30, 1 << 31)
    assert L.coli_moe_forward_noalloc(None, 0, a, 1, a, None, None, None, None) == coli.COLI_EINVAL
    assert L.coli_moe_forward_noalloc(ctypes.byref(lay), 0, None, 1, a, None, None, None,
                                      None) == coli.COLI_EINVAL
    # T = 2048 prefill of the decode-shaped layer needs far more than 32 MiB
    assert L.coli_moe_workspace_bytes(ctypes.byref(lay), 2048, coli.COLI_PREFILL) > \
        coli.COLI_NOALLOC_SCRATCH_BYTES
    assert L.coli_moe_forward_noalloc(ctypes.byref(lay), coli.COLI_PREFILL, a, 2048, a, None,
                                      None, None, None) == coli.COLI_ESCRATCH
    # the documented limits: this layer fits decode up to T = 74, prefill up to 206
    for mode, tmax in ((coli.COLI_DECODE, 74), (coli.COLI_PREFILL, 206)):
        assert L.coli_moe_workspace_bytes(ctypes.byref(lay), tmax, mode) <= \
            coli.COLI_NOALLOC_SCRATCH_BYTES
        assert L.coli_moe_workspace_bytes(ctypes.byref(lay), tmax + 1, mode) > \
            coli.COLI_NOALLOC_SCRATCH_BYTES
    assert L.coli_moe_forward_noalloc(ctypes.byref(lay), coli.COLI_DECODE, a, 75, a, None,
                                      None, None, None) == coli.COLI_ESCRATCH
    assert L.coli_moe_forward_noalloc(ctypes.byref(lay), coli.COLI_DECODE, a, 0, a, None,
                                      None, None, None) == coli.COLI_OK
    assert L.coli_strerror(coli.COLI_ESCRATCH) != b"unknown status"
