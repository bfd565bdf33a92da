"""GPU parity of the whole layer (coli_moe_forward), decode and prefill, and of the
RMSNorm between stacked layers.

Layer: route (page "Colibrì 深度解析", section 十一) -> batch union (section 四) ->
int4-g64 planar expert FFN (page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
section 权重转换) -> gate-weighted combine with the normalised gates (page "colibri 路由
遥测全解析", section 追踪流ROUTE_TRACE) + the shared expert.

Every expert the oracle uses is quantised by the oracle itself from the same seeded
fp32 draws; on the way its bytes are compared with the device blob (bit-exact).
Bars: idx bit-exact; gates within the spec's 2e-3; y under the spec bars (decode
max|d| <= 2e-3 * max(1, rms), prefill max|d| <= 2e-2 * rms) and, row by row, under
bars relative to each row's own rms (tests/harness.py: check_rows), so that layers
whose outputs are far below 1 are checked as strictly as the full-size ones.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.harness import (DEC_TOL, TIGHT_DEC, DeviceLayer, Timer, assert_close, check_rows,
                           host_array, log, margin_tokens, oracle_expert, oracle_topk, topk_gap,
                           MARGIN)

pytestmark = pytest.mark.gpu

DECODE, PREFILL = 0, 1

_layers = {}


def layer(cfg_id, l=0):
    key = (cfg_id, l)
    if key not in _layers:
        if W.CONFIGS[cfg_id]["H"] >= 4096:  # keep one full-size layer resident at a time
            for k in [k for k in _layers if W.CONFIGS[k[0]]["H"] >= 4096]:
                del _layers[k]
            torch.cuda.empty_cache()
        with Timer(f"build layer cfg {cfg_id} l {l}"):
            _layers[key] = DeviceLayer(cfg_id, l)
    return _layers[key]


def oracle_check(cfg_id, L, x, y, idx, gates, mode, rows=None, check_bytes=True, l=0,
                 what=""):
    """Compare (sampled rows of) a forward with the oracle: ids bit-exact, gates under
    the spec bar, y row by row (check_rows).  Returns the worst row err/rms."""
    c = W.CONFIGS[cfg_id]
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    xh = host_array(x[torch.from_numpy(rows).to(x.device)])
    wr = host_array(L.w_router)
    ridx, rg, _ = oracle_topk(cfg_id, xh, wr, L.bias_np, c["K"])
    need = sorted(set(ridx.reshape(-1).tolist()))
    experts = [None] * c["E"]
    with Timer(f"oracle experts {len(need)}"):
        for e in need:
            experts[e] = oracle_expert(cfg_id, e, l, "cuda", L if check_bytes else None)
        shared = oracle_expert(cfg_id, c["E"], l, "cuda", L if check_bytes else None)
    with Timer(f"oracle forward {len(rows)} rows"):
        yr, ridx2, rg2 = oracle.moe_forward(xh, wr, L.bias_np, experts, shared, c["H"], c["I"],
                                            c["K"], scoring=W.scoring(cfg_id))
    assert np.array_equal(ridx, ridx2)
    gi = idx.cpu().numpy()[rows]
    assert np.array_equal(gi, ridx), "top-K ids differ from the oracle"
    gerr = assert_close(gates.cpu().numpy()[rows], rg, DEC_TOL, what="gates")
    log(f"[parity] gates max err {gerr:.3e}")
    yg = y.float().cpu().numpy()[rows]
    tag = what or f"cfg {cfg_id} T {x.shape[0]} {'decode' if mode == DECODE else 'prefill'}"
    return check_rows(yg, yr, mode == PREFILL, what=tag,
                      tight=TIGHT_DEC if mode == DECODE else None)


# T <= 64 takes the one-chunk decode route (T = 64 sets bit 63 of its token
# bitmaps), T = 65 and 256 the chunked one
@pytest.mark.parametrize("cfg_id,T", [(0, 1), (0, 7), (101, 40), (102, 5), (103, 3), (106, 3),
                                      (0, 256), (101, 1), (101, 64), (101, 65)])
def test_decode_small(cfg_id, T):
    log(f"decode small cfg {cfg_id} T {T}")
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, c["K"])
    y, idx, gates = L.forward(x, DECODE)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, DECODE)


def test_decode_batch_row_scales():
    """Decode batch rows spanning 2^-8 .. 2^12 and an all-zero row: each row's x and h
    get their own power-of-two scale before the fp16 hi/lo split.  Power-of-two
    factors scale the logits exactly, so every row keeps its routing margin (the
    zero row's logits are exact ties or the bias, resolved the same way on both
    sides).  Each row is held to a bar relative to its own rms (check_rows), and the
    zero row must come out exactly zero."""
    cfg_id = 0
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    x = margin_tokens(cfg_id, 5, host_array(L.w_router), L.bias_np, c["K"])
    f = torch.tensor([1.0, 2.0 ** 4, 2.0 ** 12, 2.0 ** -8, 0.0], device=x.device)
    x = (x * f[:, None]).contiguous()
    y, idx, gates = L.forward(x, DECODE)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    for row in range(5):
        log(f"row scale {float(f[row])}")
        oracle_check(cfg_id, L, x, y, idx, gates, DECODE, rows=[row], check_bytes=(row == 0),
                     what=f"batch row scale {float(f[row]):g}")
    assert float(y[4].abs().max()) == 0.0


def test_decode_one_token_scales():
    """Single-token decode (int8 digit planes under one power-of-two scale per vector)
    with the token scaled by 2^12, 2^-8 and 0, each held to a bar relative to its own
    output rms (the zero token must give exactly zero)."""
    cfg_id = 107
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    x0 = margin_tokens(cfg_id, 1, host_array(L.w_router), L.bias_np, c["K"])
    for f in (2.0 ** 12, 2.0 ** -8, 0.0):
        log(f"one token scale {f}")
        x = (x0 * f).contiguous()
        y, idx, gates = L.forward(x, DECODE)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        oracle_check(cfg_id, L, x, y, idx, gates, DECODE, check_bytes=(f == 2.0 ** 12),
                     what=f"one token scale {f:g}")
        if f == 0.0:
            assert float(y.abs().max()) == 0.0


@pytest.mark.parametrize("cfg_id", [107, 108, 109, 110, 111, 112, 113, 114])
def test_decode_one_token(cfg_id):
    """Single-token decode on the int8 matrix-core path, several tokens per layer."""
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    xs = margin_tokens(cfg_id, 3, host_array(L.w_router), L.bias_np, c["K"])
    for t in range(3):
        log(f"one token cfg {cfg_id} token {t}")
        x = xs[t:t + 1].contiguous()
        y, idx, gates = L.forward(x, DECODE)
        torch.cuda.synchronize()
        oracle_check(cfg_id, L, x, y, idx, gates, DECODE, check_bytes=(t == 0))
    a = L.forward(xs[:1].contiguous(), DECODE)[0].cpu()
    b = L.forward(xs[:1].contiguous(), DECODE)[0].cpu()
    assert torch.equal(a, b), "repeated forward differs"


@pytest.mark.parametrize("cfg_id,T", [(100, 333), (104, 200), (100, 1), (100, 64), (100, 65)])
def test_prefill_small(cfg_id, T):
    log(f"prefill small cfg {cfg_id} T {T}")
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, c["K"])
    y, idx, gates = L.forward(x, PREFILL)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, PREFILL)


def test_prefill_row_scales():
    """Prefill rows scaled by 2^4 .. 2^-8 (bf16 x; power-of-two factors scale the
    logits exactly, so the routing margin holds): each row under its own rms bar."""
    cfg_id = 100
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    x = margin_tokens(cfg_id, 6, host_array(L.w_router), L.bias_np, c["K"])
    f = torch.tensor([2.0 ** 4, 1.0, 2.0 ** -2, 2.0 ** -4, 2.0 ** -6, 2.0 ** -8], device=x.device)
    # each token's x is scaled by its own power of two before the fp16 conversion
    # (and its h by the square), so every row keeps the same relative accuracy
    x = (x.float() * f[:, None]).to(torch.bfloat16).contiguous()
    y, idx, gates = L.forward(x, PREFILL)
    torch.cuda.synchronize()
    for row in range(6):
        oracle_check(cfg_id, L, x, y, idx, gates, PREFILL, rows=[row], check_bytes=(row == 0),
                     what=f"prefill row scale {float(f[row]):g}")


def test_decode_full_size_t1():
    """The decode workload: H=6144, I=2048, E=256, K=8, T=1, several tokens."""
    L = layer(1)
    c = W.CONFIGS[1]
    xs = margin_tokens(1, 3, host_array(L.w_router), None, c["K"])
    for t in range(3):
        log(f"decode full T=1 token {t}")
        x = xs[t:t + 1].contiguous()
        y, idx, gates = L.forward(x, DECODE)
        torch.cuda.synchronize()
        oracle_check(1, L, x, y, idx, gates, DECODE, check_bytes=(t == 0))


def test_decode_full_size_t32_zipf():
    """The Zipf decode batch: T=32; every token's ids and outputs."""
    L = layer(2)
    c = W.CONFIGS[2]
    x = margin_tokens(2, 32, host_array(L.w_router), L.bias_np, c["K"])
    y, idx, gates = L.forward(x, DECODE)
    torch.cuda.synchronize()
    # every token's routing
    logits = oracle.router_logits(host_array(x), host_array(L.w_router), L.bias_np)
    ridx, _, _ = oracle.topk(logits, c["K"])
    assert np.array_equal(idx.cpu().numpy(), ridx)
    U = len(set(ridx.reshape(-1).tolist()))
    log(f"zipf T=32 unique experts U={U}")
    assert U < 32 * 8
    oracle_check(2, L, x, y, idx, gates, DECODE)


def cover_rows(ridx: np.ndarray, T: int, chunk: int) -> list:
    """Rows of a prefill batch such that every routed expert with a token and every
    chunk-row block of the shared expert's tokens appears at least once: one row per
    shared block (the one adding the most new experts), then a greedy cover of the
    experts left."""
    left = set(ridx.reshape(-1).tolist())
    rows = []
    for b0 in range(0, T, chunk):
        blk = range(b0, min(T, b0 + chunk))
        best = max(blk, key=lambda t: len(left & set(ridx[t].tolist())))
        rows.append(best)
        left -= set(ridx[best].tolist())
    while left:
        best = max(range(T), key=lambda t: len(left & set(ridx[t].tolist())))
        rows.append(best)
        left -= set(ridx[best].tolist())
    return sorted(set(rows))


def test_prefill_full_size_sampled():
    """The prefill workload: T=2048 bf16; all ids and gates, and the outputs of rows
    that cover every routed expert with a token and every 128-token block of the
    shared expert's tokens (the grouped GEMM's M-chunks)."""
    L = layer(3)
    c = W.CONFIGS[3]
    with Timer("margin tokens T=2048"):
        x = margin_tokens(3, 2048, host_array(L.w_router), None, c["K"])
    y, idx, gates = L.forward(x, PREFILL)
    torch.cuda.synchronize()
    with Timer("oracle routing T=2048"):
        logits = oracle.router_logits(host_array(x), host_array(L.w_router), None)
        ridx, rg, _ = oracle.topk(logits, c["K"])
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert_close(gates.cpu().numpy(), rg, DEC_TOL, what="gates")
    counts = np.bincount(ridx.reshape(-1), minlength=c["E"])
    log(f"prefill tokens per expert min {counts.min()} max {counts.max()}")
    rows = cover_rows(ridx, 2048, 128)
    log(f"prefill rows checked: {len(rows)}")
    assert set(ridx[rows].reshape(-1).tolist()) == set(ridx.reshape(-1).tolist())
    oracle_check(3, L, x, y, idx, gates, PREFILL, rows=rows, check_bytes=False)


def test_forward_deterministic_and_t0():
    L = layer(0)
    x = margin_tokens(0, 4, host_array(L.w_router), None, 4)
    a = L.forward(x, DECODE)[0].cpu()
    b = L.forward(x, DECODE)[0].cpu()
    assert torch.equal(a, b)
    Lp = layer(100)
    xp = margin_tokens(100, 100, host_array(Lp.w_router), None, 6)
    a = Lp.forward(xp, PREFILL)[0].cpu()
    b = Lp.forward(xp, PREFILL)[0].cpu()
    assert torch.equal(a, b)
    y, _, _ = L.forward(x[:0], DECODE)  # T = 0: no-op, no error
    assert y.shape == (0, 256)


# H = 6144 (8 float4 per thread), 256/1000 (1, ragged), 2048 (2), 4000 (4), 8192 (8,
# full); 8196 (beyond the register rows), 6 (H % 4 != 0): the strided kernel
@pytest.mark.parametrize("H", [6144, 256, 1000, 2048, 4000, 8192, 8196, 6])
def test_rmsnorm_parity(H):
    import int4_grouped_expert_amd as coli
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((9, H), generator=g, device="cuda") * 3.0
    y = torch.empty_like(x)
    coli.coli_rmsnorm_f32(x, y, 1e-6)
    ref = oracle.rmsnorm(x.cpu().double().numpy(), 1e-6)
    assert_close(y.cpu().numpy(), ref, 1e-5, what="rmsnorm")
    coli.coli_rmsnorm_f32(x, x, 1e-6)  # in place
    assert torch.equal(x, y)


def test_rmsnorm_unaligned_rows():
    """Rows that are not 16-byte aligned take the strided kernel."""
    import int4_grouped_expert_amd as coli
    g = torch.Generator(device="cuda").manual_seed(4)
    buf = torch.randn(5 * 512 + 1, generator=g, device="cuda")
    x = buf[1:].view(5, 512)  # 4-byte offset
    y = torch.empty((5, 512), device="cuda")
    coli.coli_rmsnorm_f32(x, y, 1e-6)
    ref = oracle.rmsnorm(x.cpu().double().numpy(), 1e-6)
    assert_close(y.cpu().numpy(), ref, 1e-5, what="rmsnorm unaligned")


def stack_check(cfg_id, nlayers, T, e2e_layers):
    """A stack of MoE layers with RMSNorm between them (no attention, no residual).

    The layer-to-layer map amplifies perturbations (~1.4x per layer for these random
    layers: a 1e-7 relative change of x_0 reaches O(1) after ~36 layers even in
    fp64), so fp32 and fp64 chains cannot agree after 40 layers.  Checked instead:
      * per layer: the GPU layer l on the oracle chain's own input x_l (rounded to
        fp32) matches the oracle's y_l;
      * end to end: the GPU chain matches the oracle chain for the first e2e_layers;
      * the full GPU chain is finite, every normalised x has RMS sqrt(m/(m+eps))
        (m the mean square before the norm), and two runs are bitwise identical.
    Tokens whose top-K gap is under the margin at any layer are redrawn."""
    import int4_grouped_expert_amd as coli
    c = W.CONFIGS[cfg_id]
    Ls = [DeviceLayer(cfg_id, l) for l in range(nlayers)]
    ex = [[None] * c["E"] for _ in range(nlayers)]
    sh = [None] * nlayers

    def oexpert(l, e):
        if e == c["E"]:
            if sh[l] is None:
                sh[l] = oracle_expert(cfg_id, e, l, "cuda")
            return sh[l]
        if ex[l][e] is None:
            ex[l][e] = oracle_expert(cfg_id, e, l, "cuda")
        return ex[l][e]

    def ochain(xh):
        cur = xh
        gaps, xs, ys = [], [], []
        for l in range(nlayers):
            logits = oracle.router_logits(cur, host_array(Ls[l].w_router), Ls[l].bias_np)
            gaps.append(topk_gap(logits, c["K"]))
            ridx, _, _ = oracle.topk(logits, c["K"])
            for e in set(ridx.reshape(-1).tolist()):
                oexpert(l, e)
            y, _, _ = oracle.moe_forward(cur, host_array(Ls[l].w_router), Ls[l].bias_np, ex[l],
                                         oexpert(l, c["E"]), c["H"], c["I"], c["K"])
            xs.append(cur)
            ys.append(y)
            cur = oracle.rmsnorm(y, 1e-6)
        return xs, ys, np.min(np.stack(gaps), axis=0)

    x = W.tokens(cfg_id, T, "cuda", 0)
    draw = 1
    while True:
        xs, ys, gap = ochain(host_array(x))
        bad = np.nonzero(gap < MARGIN)[0]
        if bad.size == 0:
            break
        assert draw < 30
        fresh = W.tokens(cfg_id, T, "cuda", draw)
        x[torch.from_numpy(bad).cuda()] = fresh[: bad.size]
        draw += 1
    worst = 0.0
    for l in range(nlayers):
        xl = torch.from_numpy(np.asarray(xs[l], dtype=np.float32)).cuda()
        y, _, _ = Ls[l].forward(xl, DECODE)
        torch.cuda.synchronize()
        worst = max(worst, check_rows(y.cpu().numpy(), ys[l], False, what=f"stack layer {l}",
                                      tight=TIGHT_DEC))
    log(f"stack per-layer worst rel err {worst:.2e}")

    def gpu_chain(n):
        cur = x.clone()
        for l in range(n):
            y, _, _ = Ls[l].forward(cur, DECODE)
            if l + 1 < n:
                m = y.double().pow(2).mean(1)
                coli.coli_rmsnorm_f32(y, y, 1e-6)
                rms = y.double().pow(2).mean(1).sqrt()
                want = (m / (m + 1e-6)).sqrt()  # unit RMS up to the eps term
                assert torch.all((rms - want).abs() < 1e-5), f"layer {l} rms {rms}"
            cur = y
        torch.cuda.synchronize()
        return cur
    e2e = gpu_chain(e2e_layers)
    err = check_rows(e2e.cpu().numpy(), ys[e2e_layers - 1], False,
                     what=f"stack out after {e2e_layers} layers")
    log(f"stack end-to-end {e2e_layers} layers rel err {err:.2e}")
    full = gpu_chain(nlayers)
    assert torch.all(torch.isfinite(full))
    assert torch.equal(full, gpu_chain(nlayers))


def test_stack_small_40_layers():
    log("stack small 40 layers")
    stack_check(105, 40, 8, e2e_layers=8)


def test_stack_full_size_two_layers():
    log("stack full size, 2 layers")
    for k in list(_layers):
        del _layers[k]
    torch.cuda.empty_cache()
    stack_check(4, 2, 8, e2e_layers=2)
