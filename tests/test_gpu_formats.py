"""GPU parity of the sibling weight formats against the oracle (oracle/formats.py):

* coli_quant_fmt bit-exact (packed bytes and scale bits) for int3-g64, MXFP4 and
  fp8-e4m3-b128: N(0, 0.02) weights of the decode layer's shapes and ragged ones,
  rows scaled over many binades, exact ties, all-zero groups, and non-finite
  inputs (NaN scale, neutral codes, status bit 1);
* coli_matvec_fmt against the oracle's fp64 product on the ORACLE's packed bytes
  (never the kernel's own), for T = 1..8, including every code of each element
  format (checks the hardware conversions the kernels use), with the per-token bar
  max|gpu - oracle| <= 2e-5 * rms(oracle y[t]) for the float element formats and
  1e-4 for the offset-integer ones (their kernels take sum u x - 8 sum x (4 for
  int3) per group: fp32 cancellation of about one decimal digit), next to the
  decode tolerance 2e-3 * max(1, rms);
* the layer with its experts in each format against the oracle's fp64 layer, with
  the same bars, except the MXFP4 and fp8-e4m3-b128 layers on the scaled matrix
  cores (gate/up for T <= 2, down for T = 1, H a multiple of 256): 2e-4 and 5e-4,
  as those sum each 128-term block product with about 2^-15 of its largest term
  (measured against a host product; worst seen over the two matrix-core products
  7.4e-5 for MXFP4 and 1.8e-4 for E4M3 weights, whose wider range leaves fewer
  bits to the smaller terms), four to ten times inside the decode tolerance.
Page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战", section 权重转换 (the
registry); OCP MX v1.0 and OCP FP8 for the element formats.
"""
import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.harness import log

pytestmark = pytest.mark.gpu

FMTS = (5, 7, 8)
NAMES = {4: "int4-g64", 5: "int3-g64", 7: "mxfp4", 8: "fp8-e4m3-b128"}
TIGHT = {4: 1e-4, 5: 1e-4, 7: 2e-5, 8: 2e-5}
MX_MFMA_TIGHT = {7: 2e-4, 8: 5e-4}  # the MXFP4 and fp8 layers on the scaled matrix cores


def weights(O, I, seed, spread=False):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((O, I)) * 0.02).astype(np.float32)
    if spread:  # rows over many binades
        w *= (2.0 ** rng.integers(-30, 30, size=(O, 1))).astype(np.float32)
    return w


def gpu_quant(fmt, w, status=None):
    import int4_grouped_expert_amd as coli
    O, I = w.shape
    nw, ns = coli.coli_fmt_bytes(fmt, O, I)
    pk = torch.zeros(max(nw, 16), dtype=torch.uint8, device="cuda")
    sc = torch.zeros(max(ns, 16), dtype=torch.uint8, device="cuda")
    coli.coli_quant_fmt(fmt, torch.from_numpy(w).cuda(), pk, sc, status=status)
    torch.cuda.synchronize()
    return pk[:nw].cpu().numpy(), sc[:ns].cpu().numpy()


def oracle_bytes(fmt, w):
    pk, sc = F.quant(fmt, w)
    return np.ascontiguousarray(pk).reshape(-1).view(np.uint8), \
        np.ascontiguousarray(sc).reshape(-1).view(np.uint8)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("O,I,spread", [(2048, 6144, False), (6144, 2048, False),
                                        (72, 200, True), (130, 1000, True), (3, 17, False)])
def test_quant_bit_exact(fmt, O, I, spread):
    if fmt == 8 and O * I > 4_000_000:
        O = 512  # the fp8 tiles of a 2048-row matrix are 128 rows apart: a slab is enough
    log(f"quant {NAMES[fmt]} O {O} I {I} spread {spread}")
    w = weights(O, I, 1000 * fmt + O + I, spread)
    g_pk, g_sc = gpu_quant(fmt, w)
    o_pk, o_sc = oracle_bytes(fmt, w)
    assert np.array_equal(g_sc, o_sc), "scales differ"
    bad = np.nonzero(g_pk != o_pk)[0]
    assert bad.size == 0, f"{bad.size} packed bytes differ, first at {bad[:5]}"


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_special_values(fmt):
    # ties of each rounding, exact grid values, zero groups, tiny and huge rows
    O, I = 256, 256
    w = weights(O, I, 7 + fmt)
    w[0, :] = 0.0
    if fmt == 5:  # s = 1: quotients on the half-integers
        w[1, :64] = np.tile(np.array([3.0, -3.0, 0.5, 1.5, 2.5, -2.5, -3.5, -0.5],
                                     np.float32), 8)
    if fmt == 7:  # X = 1: the E2M1 midpoints
        w[1, :32] = np.tile(np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0],
                                     np.float32), 4)
    if fmt == 8:  # s = 1: every E4M3 value and midpoint of the first tile's row 1
        vals = np.concatenate([F.E4M3, (F.E4M3[1:] + F.E4M3[:-1]) / 2])
        w[1, :128] = vals[:128].astype(np.float32)
        w[1, 127] = 448.0
        w[2:128, :128] = 0.0
    w[3, :] *= np.float32(2.0 ** -100)
    w[4, :] *= np.float32(2.0 ** 100)
    g_pk, g_sc = gpu_quant(fmt, w)
    o_pk, o_sc = oracle_bytes(fmt, w)
    assert np.array_equal(g_sc, o_sc)
    assert np.array_equal(g_pk, o_pk)


@pytest.mark.parametrize("fmt", FMTS)
def test_quant_non_finite(fmt):
    import int4_grouped_expert_amd as coli
    w = weights(200, 300, 9)
    w[5, 70] = np.nan
    w[150, 299] = -np.inf
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    g_pk, g_sc = gpu_quant(fmt, w, status=st)
    assert int(st.item()) & coli.COLI_STATUS_NONFINITE
    o_pk, o_sc = oracle_bytes(fmt, w)
    if fmt == 7:
        assert np.array_equal(g_sc, o_sc)
    else:  # NaN scales: compare the bit patterns' NaN-ness and the rest exactly
        gs, os_ = g_sc.view(np.float32), o_sc.view(np.float32)
        assert np.array_equal(np.isnan(gs), np.isnan(os_)) and np.isnan(os_).any()
        assert np.array_equal(gs[~np.isnan(os_)], os_[~np.isnan(os_)])
    assert np.array_equal(g_pk, o_pk)
    st.zero_()
    gpu_quant(fmt, weights(64, 64, 10), status=st)
    assert int(st.item()) == 0


def gpu_matvec(fmt, pk, sc, O, I, x):
    import int4_grouped_expert_amd as coli
    pk_d = torch.from_numpy(np.ascontiguousarray(pk).reshape(-1).view(np.uint8).copy()).cuda()
    sc_d = torch.from_numpy(np.ascontiguousarray(sc).reshape(-1).view(np.uint8).copy()).cuda()
    x_d = torch.from_numpy(x).cuda()
    y = torch.full((x.shape[0], O), float("nan"), dtype=torch.float32, device="cuda")
    coli.coli_matvec_fmt(fmt, pk_d, sc_d, O, I, x_d, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def check(yg, yr, what, tight):
    rms = np.sqrt(np.mean(yr * yr, axis=1, keepdims=True))
    err = np.abs(yg - yr).max(axis=1, keepdims=True)
    worst = float((err / np.maximum(rms, 1e-300)).max())
    log(f"[parity] matvec {what}: worst token err/rms {worst:.3e}; bar/rms {tight}")
    assert worst <= tight, what
    assert float((err / np.maximum(1.0, rms)).max()) <= 2e-3


@pytest.mark.parametrize("fmt", (4,) + FMTS)
@pytest.mark.parametrize("O,I,T", [(2048, 6144, 1), (6144, 2048, 1), (2048, 6144, 4),
                                   (300, 2048, 8), (70, 200, 3), (129, 1000, 2),
                                   (5, 64, 1)])
def test_matvec_parity(fmt, O, I, T):
    if fmt == 8 and I % 16:
        I = (I + 15) // 16 * 16
    log(f"matvec {NAMES[fmt]} O {O} I {I} T {T}")
    w = weights(O, I, 31 * O + I + fmt, spread=O < 200)
    if fmt == 4:
        import oracle
        pk, sc, _ = oracle.quant_int4_g64(w)
        W = oracle.dequant_int4_g64(pk, sc, I)
    else:
        pk, sc = F.quant(fmt, w)
        W = F.dequant(fmt, pk, sc, O, I)
    x = np.random.default_rng(O + T).standard_normal((T, I)).astype(np.float32)
    yr = F.matvec(W, x)
    yg = gpu_matvec(fmt, pk, sc, O, I, x)
    check(yg, yr, f"{NAMES[fmt]} O {O} I {I} T {T}", TIGHT[fmt])


@pytest.mark.parametrize("fmt", (7, 8))
def test_matvec_every_code(fmt):
    """One-hot x reads single weights back: every code of the element format,
    both signs, decodes as the oracle says (the kernels use the gfx950
    conversion instructions)."""
    O, I = 16, 256
    if fmt == 8:
        codes = np.arange(256, dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0  # the NaN codes are never produced
        pk = np.zeros((O, I), np.uint8)
        pk[0, :] = codes
        pk[1, :] = codes[::-1]
        sc = np.full((1, 2), 0.5, np.float32)
    else:
        nib = np.arange(16, dtype=np.uint8)
        row = np.tile(nib, I // 16)
        pk = np.zeros((O, I // 2), np.uint8)
        pk[0, :] = (row[0::2] | (row[1::2] << 4)).astype(np.uint8)
        pk[1, :] = (row[1::2] | (row[0::2] << 4)).astype(np.uint8)
        sc = np.full((O, I // 32), 127, np.uint8)
        sc[:, 3] = 120
    W = F.dequant(fmt, pk, sc, O, I)
    for start in range(0, I, 8):
        xs = np.eye(I, dtype=np.float32)[start:start + 8]
        yg = gpu_matvec(fmt, pk, sc, O, I, xs)
        assert np.array_equal(yg, F.matvec(W, xs)), f"codes {start}..{start + 7}"


@pytest.mark.parametrize("fmt", (4,) + FMTS)
def test_matvec_non_finite_group_poisons_its_rows(fmt):
    """A group, block or tile stored with the NaN scale (non-finite weights) makes
    exactly the outputs it feeds NaN, as the oracle's fp64 product says; every
    other output stays within the bar."""
    O, I, T = 260, 512, 2
    w = weights(O, I, 77 + fmt)
    w[3, 100] = np.nan
    w[200, 511] = np.inf
    if fmt == 4:
        import oracle
        pk, sc, _ = oracle.quant_int4_g64(w)
        W = oracle.dequant_int4_g64(pk, sc, I)
    else:
        pk, sc = F.quant(fmt, w)
        W = F.dequant(fmt, pk, sc, O, I)
    x = np.random.default_rng(5).standard_normal((T, I)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        yr = F.matvec(W, x)
    yg = gpu_matvec(fmt, pk, sc, O, I, x)
    bad = np.isnan(yr)
    assert bad.any() and np.array_equal(np.isnan(yg), bad)
    keep = ~bad.any(axis=0)
    check(yg[:, keep], yr[:, keep], f"{NAMES[fmt]} finite rows", TIGHT[fmt])


# ---------------------------------------------------------------- the layer in a format

class FmtLayer:
    """A layer of a workload with its experts quantised by the library into fmt."""

    def __init__(self, cfg_id, fmt):
        import int4_grouped_expert_amd as coli
        import workloads as W
        c = W.CONFIGS[cfg_id]
        self.cfg_id, self.fmt = cfg_id, fmt
        self.H, self.I, self.E, self.K = H, I, E, K = c["H"], c["I"], c["E"], c["K"]
        self.w_router = W.router_weights(cfg_id, "cuda").contiguous()
        b = W.router_bias(cfg_id)
        self.bias_np = b
        self.bias = None if b is None else torch.from_numpy(b).cuda()
        self.scoring = W.scoring(cfg_id)
        self.nb = nb = coli.coli_fmt_blob_bytes(fmt, H, I)
        self.experts = torch.empty(E * nb, dtype=torch.uint8, device="cuda")
        self.shared = torch.empty(nb, dtype=torch.uint8, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        for e in range(E + 1):
            wg, wu, wd = W.expert_weights(cfg_id, e, "cuda")
            ptr = self.shared.data_ptr() if e == E else self.experts.data_ptr() + e * nb
            coli.coli_quant_expert_fmt(fmt, ptr, H, I, wg, wu, wd, st)
            del wg, wu, wd
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        self.layer_c = coli.MoELayer(H, I, E, K, self.w_router, self.experts, self.shared,
                                     self.bias, self.scoring)

    def forward(self, x):
        import int4_grouped_expert_amd as coli
        T = x.shape[0]
        ws = torch.empty(coli.coli_moe_fmt_workspace_bytes(self.layer_c, self.fmt, T),
                         dtype=torch.uint8, device="cuda")
        y = torch.full((T, self.H), float("nan"), device="cuda")
        idx = torch.empty((T, self.K), dtype=torch.int32, device="cuda")
        gates = torch.empty((T, self.K), dtype=torch.float32, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        coli.coli_moe_forward_fmt(self.layer_c, self.fmt, x, y, ws, idx, gates, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        return y, idx, gates

    def blob_sections(self, e):
        """Host copies of expert e's six sections (e == E: the shared expert)."""
        blob = (self.shared if e == self.E else
                self.experts[e * self.nb:(e + 1) * self.nb]).cpu().numpy()
        parts = [F.sizes(self.fmt, self.I, self.H)] * 2 + [F.sizes(self.fmt, self.H, self.I)]
        a256 = lambda n: (n + 255) // 256 * 256
        o, q, s = 0, [], []
        for w, _ in parts:
            q.append(blob[o:o + w])
            o += a256(w)
        for _, sc in parts:
            s.append(blob[o:o + sc])
            o += a256(max(sc, 1))
        return q, s


def oracle_fmt_check(L, x, y, idx, gates):
    import workloads as W
    from tests.harness import host_array
    xh = host_array(x)
    wr = host_array(L.w_router)
    c = W.CONFIGS[L.cfg_id]
    ids = sorted(set(idx.cpu().numpy().reshape(-1).tolist()))
    experts = [None] * L.E
    for e in ids + [L.E]:
        wg, wu, wd = (t.cpu().numpy() for t in W.expert_weights(L.cfg_id, e, "cuda"))
        ex = F.quant_expert(L.fmt, wg, wu, wd)
        q, s = L.blob_sections(e)
        for m in range(3):  # the library's bytes are the oracle's
            assert np.array_equal(q[m], np.ascontiguousarray(ex[m][0]).reshape(-1).view(np.uint8))
            assert np.array_equal(s[m], np.ascontiguousarray(ex[m][1]).reshape(-1).view(np.uint8))
        if e == L.E:
            shared = ex
        else:
            experts[e] = ex
    yr, ridx, rg = F.moe_forward_fmt(L.fmt, xh, wr, L.bias_np, experts, shared, L.H, L.I,
                                      c["K"], L.scoring)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.abs(gates.cpu().numpy() - rg).max() <= 2e-3
    mfma = L.fmt in (7, 8) and x.shape[0] <= 2 and L.H % 256 == 0
    check(y.cpu().numpy().astype(np.float64), yr, f"layer {NAMES[L.fmt]} cfg {L.cfg_id} "
          f"T {x.shape[0]}", MX_MFMA_TIGHT[L.fmt] if mfma else TIGHT[L.fmt])


_fmt_layers = {}


def fmt_layer(cfg_id, fmt):
    key = (cfg_id, fmt)
    if key not in _fmt_layers:
        if cfg_id == 1:  # keep one full-size layer resident at a time
            for k in [k for k in _fmt_layers if k[0] == 1]:
                del _fmt_layers[k]
            torch.cuda.empty_cache()
        _fmt_layers[key] = FmtLayer(cfg_id, fmt)
    return _fmt_layers[key]


def _layer_cases():
    """(fmt, cfg, T) of the format-layer parity cases.  fp8-e4m3-b128 rows must be
    whole 16-byte multiples: its layer is not built for the ragged shape (119), whose
    rejection (COLI_ESHAPE, no workspace) test_abi_cpu.py checks."""
    import workloads as W
    out = []
    for cfg_id, T in [(107, 1), (107, 3), (116, 2), (119, 4), (1, 1), (1, 2), (1, 4)]:
        c = W.CONFIGS[cfg_id]
        for fmt in (4,) + FMTS:
            if (cfg_id, T) == (1, 2) and fmt not in (7, 8):
                continue  # the full-size matrix-core gate/up with the generic down
            if fmt == 8 and (c["H"] % 16 or c["I"] % 16):
                continue
            out.append((fmt, cfg_id, T))
    return out


@pytest.mark.parametrize("fmt,cfg_id,T", _layer_cases())
def test_layer_in_format(fmt, cfg_id, T):
    import workloads as W
    from tests.harness import host_array, margin_tokens
    c = W.CONFIGS[cfg_id]
    log(f"layer {NAMES[fmt]} cfg {cfg_id} T {T}")
    L = fmt_layer(cfg_id, fmt)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, c["K"])
    y, idx, gates = L.forward(x)
    oracle_fmt_check(L, x, y, idx, gates)


def _forward_status(L, x):
    """The format layer's forward with its status word returned (not asserted)."""
    import int4_grouped_expert_amd as coli
    T = x.shape[0]
    ws = torch.empty(coli.coli_moe_fmt_workspace_bytes(L.layer_c, L.fmt, T),
                     dtype=torch.uint8, device="cuda")
    y = torch.full((T, L.H), float("nan"), device="cuda")
    idx = torch.empty((T, L.K), dtype=torch.int32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    coli.coli_moe_forward_fmt(L.layer_c, L.fmt, x, y, ws, idx, status=st)
    torch.cuda.synchronize()
    return y.cpu().numpy(), idx.cpu().numpy(), int(st.item())


@pytest.mark.parametrize("fmt", (7, 8))
def test_matrix_core_layer_nan_block(fmt):
    """The matrix-core format layer (one token, H a multiple of 256) with one
    gate block of an expert stored with the NaN scale (E8M0 255 for MXFP4, a NaN
    tile scale for fp8): a token routed to that expert gets an all-NaN y and the
    status bit COLI_STATUS_NONFINITE, as the oracle's fp64 layer says (the NaN
    reaches every h' of that unit through its gate row, then every output through
    the down); the same block in an expert the token did not pick changes nothing,
    bit for bit.  The scale is restored afterwards."""
    import workloads as W
    from tests.harness import host_array, margin_tokens
    c = W.CONFIGS[107]
    log(f"matrix-core layer NaN block {NAMES[fmt]}")
    L = fmt_layer(107, fmt)
    x = margin_tokens(107, 1, host_array(L.w_router), L.bias_np, c["K"])
    y0, idx, st0 = _forward_status(L, x)
    assert st0 == 0 and np.isfinite(y0).all()
    picked = int(idx[0, 0])
    other = next(e for e in range(L.E) if e not in set(idx[0].tolist()))
    a256 = lambda n: (n + 255) // 256 * 256
    qbytes = [F.sizes(fmt, L.I, L.H)[0]] * 2 + [F.sizes(fmt, L.H, L.I)[0]]
    gate_scales = sum(a256(n) for n in qbytes)  # the gate scale section of a blob
    for e, expect_nan in ((other, False), (picked, True)):
        base = e * L.nb + gate_scales
        view = L.experts[base:base + 4]
        keep = view.clone()
        if fmt == 7:
            view[0] = 255
        else:
            view.copy_(torch.tensor([0, 0, 0xC0, 0x7F], dtype=torch.uint8))  # NaN f32
        try:
            y, _, st = _forward_status(L, x)
        finally:
            view.copy_(keep)
        if expect_nan:
            assert np.isnan(y).all() and st & 1, (NAMES[fmt], st)
        else:
            assert st == 0 and np.array_equal(y, y0)
    y1, _, st1 = _forward_status(L, x)
    assert st1 == 0 and np.array_equal(y1, y0)
