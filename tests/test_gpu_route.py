"""GPU parity of the route stage: router logits, top-K with renormalised gates
(page "Colibrì 深度解析", section 十一; gates normalised as applied, page "colibri 路由
遥测全解析", section 分离计数与追踪; NaN guard, same page, section 测试与 CI 保障) and the
batch-union permute (page "Colibrì 深度解析", section 四).

Indices, counts, offsets, perm and the unique list are bit-exact; gates and logits
within the fp32 tolerance.  Inputs pass the oracle's top-K margin filter (>= 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.harness import DEC_TOL, assert_close, host_array, log, margin_tokens

pytestmark = pytest.mark.gpu


def run_router(x, wr, bias, K):
    import int4_grouped_expert_amd as coli
    T, E = x.shape[0], wr.shape[0]
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    coli.coli_router_topk(x, wr, bias, K, idx, gates, logits)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gates.cpu().numpy(), logits.cpu().numpy()


@pytest.mark.parametrize("cfg_id,T", [(0, 1), (0, 9), (1, 1), (1, 3), (2, 32), (102, 5),
                                      (103, 3), (104, 200)])
def test_router_topk_parity(cfg_id, T):
    log(f"router cfg {cfg_id} T {T}")
    c = W.CONFIGS[cfg_id]
    wr = W.router_weights(cfg_id, "cuda").contiguous()
    b = W.router_bias(cfg_id)
    bias = None if b is None else torch.from_numpy(b).cuda()
    wr_h = host_array(wr)
    x = margin_tokens(cfg_id, T, wr_h, b, c["K"])
    idx, gates, logits = run_router(x, wr, bias, c["K"])
    ref_logits = oracle.router_logits(host_array(x), wr_h, b)
    ridx, rg, fb = oracle.topk(ref_logits, c["K"])
    assert fb == 0
    assert np.array_equal(idx, ridx)
    assert_close(gates, rg, DEC_TOL, what="gates")
    assert np.all(np.abs(gates.astype(np.float64).sum(1) - 1) <= c["K"] * 2.0 ** -22)
    assert_close(logits, ref_logits, 1e-4, what="logits")


def test_router_ties_lower_id_wins():
    """Rows 5, 9, 12 of the router are identical and give the top logit of every
    token; equal logits are bit-identical on the GPU, so with K = 2 the two lower
    ids must be taken."""
    H, E = 128, 16
    g = torch.Generator(device="cuda").manual_seed(11)
    wr = torch.randn((E, H), generator=g, device="cuda") * 0.02
    x = torch.randn((4, H), generator=g, device="cuda")
    v = x.sum(0)
    v = 0.5 * v / v.norm()
    for e in (5, 9, 12):
        wr[e] = v
    idx, _, logits = run_router(x, wr.contiguous(), None, 2)
    for t in range(4):
        assert logits[t, 5] == logits[t, 9] == logits[t, 12]
        assert logits[t, 5] == logits[t].max()
    assert np.array_equal(idx, np.tile(np.array([5, 9], dtype=np.int32), (4, 1)))


def test_router_nan_fallback():
    """All-NaN logits: slot k takes id k (page "colibrì 路由遥测全解析", 测试与 CI 保障)."""
    H, E, K = 64, 12, 4
    wr = torch.ones((E, H), device="cuda") * 0.01
    x = torch.full((2, H), float("nan"), device="cuda")
    idx, _, _ = run_router(x, wr, None, K)
    assert np.array_equal(idx, np.tile(np.arange(K, dtype=np.int32), (2, 1)))


def run_permute(idx_np, E):
    import int4_grouped_expert_amd as coli
    T, K = idx_np.shape
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    perm = torch.full((max(T * K, 1),), -1, dtype=torch.int32, device="cuda")
    unique = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    nu = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    nb = coli.coli_expert_permute_workspace_bytes(T, K, E)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda") if nb else None
    coli.coli_expert_permute(idx, E, counts, offsets, perm, unique, nu, ws)
    torch.cuda.synchronize()
    n = int(nu.item())
    return (counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()[:T * K],
            unique.cpu().numpy()[:n])


@pytest.mark.parametrize("T,K,E", [(1, 8, 256), (32, 8, 256), (64, 8, 256), (128, 8, 256),
                                   (129, 8, 256), (333, 6, 24), (2048, 8, 256), (5, 8, 8),
                                   (40, 1, 1024), (700, 16, 1024), (0, 4, 16)])
def test_permute_parity(T, K, E):
    log(f"permute T {T} K {K} E {E}")
    rng = np.random.default_rng(T * 31 + K * 7 + E)
    if T:
        # Zipf-like skew so some experts are hot and many are absent
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        idx = np.stack([np.sort(rng.choice(E, K, replace=False, p=p)) for _ in range(T)])
    else:
        idx = np.zeros((0, K), dtype=np.int32)
    idx = idx.astype(np.int32)
    got = run_permute(idx, E)
    ref = oracle.permute(idx, E)
    for g, r, name in zip(got, ref, ("counts", "offsets", "perm", "unique")):
        assert np.array_equal(g, r), name


def test_permute_skips_out_of_range_ids():
    idx = np.array([[0, 3, 9], [1, 3, -2], [2, 7, 3]], dtype=np.int32)  # E = 8: 9, -2 invalid
    counts, offsets, perm, unique = run_permute(idx, 8)
    assert list(counts) == [1, 1, 1, 3, 0, 0, 0, 1]
    assert list(offsets) == [0, 1, 2, 3, 6, 6, 6, 6, 7]
    assert list(perm[:7]) == [0, 3, 6, 1, 4, 8, 7]
    assert list(unique) == [0, 1, 2, 3, 7]


def crafted_logits(E, K, seed):
    """Logit vectors whose top-K is decided by the tie and NaN rules (page "Colibrì
    深度解析", section 十一, lower id on equal values; page "colibrì 路由遥测全解析",
    section 测试与 CI 保障, NaN never selected, fallback ids): integers from a few
    values; all equal; the K-th largest repeated at ids on both sides of it and
    across 64-id slots; integers with infinities; NaN everywhere but K + 1 ids; NaN
    everywhere but K - 2 ids (the fallback).  Every value is exact in fp32, so the
    logits are the same on both sides."""
    rng = np.random.default_rng(seed)
    out = [("ints", rng.integers(-2, 3, E).astype(np.float32)),
           ("equal", np.full(E, 0.25, np.float32))]
    v = np.round(rng.standard_normal(E) * 64).astype(np.float32) / 64
    kth = np.sort(v)[::-1][K - 1]
    v[rng.choice(E, min(E, 3 * K + 2), replace=False)] = kth
    out.append(("kth_ties", v))
    w = rng.integers(-3, 4, E).astype(np.float32)
    w[rng.choice(E, max(1, E // 5), replace=False)] = np.inf
    w[rng.choice(E, max(1, E // 5), replace=False)] = -np.inf
    out.append(("inf", w))
    n = np.full(E, np.nan, np.float32)
    keep = rng.choice(E, min(E, K + 1), replace=False)
    n[keep] = rng.integers(-4, 5, keep.size).astype(np.float32)
    out.append(("nan_some", n))
    if K >= 2:
        f = np.full(E, np.nan, np.float32)
        keep = rng.choice(E, K - 2, replace=False)
        f[keep] = rng.integers(-4, 5, keep.size).astype(np.float32)
        out.append(("nan_fallback", f))
    return out


def check_crafted(name, col, idx, gates, K):
    ref = col[None, :].astype(np.float64)
    ridx, rg, fb = oracle.topk(ref, K)
    assert (fb > 0) == (name == "nan_fallback"), name
    assert np.array_equal(idx.reshape(-1), ridx.reshape(-1)), (name, idx, ridx)
    if np.isfinite(col[ridx[0]]).all():
        assert np.allclose(gates.reshape(-1), rg.reshape(-1), rtol=1e-6, atol=1e-7), name


@pytest.mark.parametrize("E,K", [(12, 4), (100, 7), (256, 8), (256, 1), (256, 16), (200, 13), (300, 16), (1024, 8),
                                 (1024, 16), (16, 16)])
def test_router_topk_crafted(E, K):
    """coli_router_topk on crafted logits: the router reads one-hot tokens, so each
    token's logits are exactly one column of the router matrix."""
    H = 64
    for name, col in crafted_logits(E, K, E * 131 + K):
        log(f"router crafted {name} E {E} K {K}")
        wr = torch.zeros((E, H), dtype=torch.float32, device="cuda")
        wr[:, 0] = torch.from_numpy(col).cuda()
        x = torch.zeros((1, H), dtype=torch.float32, device="cuda")
        x[0, 0] = 1.0
        idx, gates, logits = run_router(x, wr, None, K)
        assert np.array_equal(logits[0], col, equal_nan=True), name
        check_crafted(name, col, idx, gates, K)


def small_layer(H, I, E, K, wr, seed=5):
    """A layer of E random experts (N(0, 0.02), quantised by the library) under the
    router matrix wr."""
    import int4_grouped_expert_amd as coli
    experts, shared, nb = coli.alloc_layer_blobs(H, I, E)
    g = torch.Generator(device="cuda").manual_seed(seed)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    for e in range(E + 1):
        wg = torch.randn((I, H), generator=g, device="cuda") * 0.02
        wu = torch.randn((I, H), generator=g, device="cuda") * 0.02
        wd = torch.randn((H, I), generator=g, device="cuda") * 0.02
        coli.coli_quant_expert(shared.data_ptr() if e == E else experts.data_ptr() + e * nb,
                               H, I, wg, wu, wd, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return coli.MoELayer(H, I, E, K, wr, experts, shared), (experts, shared)


@pytest.mark.parametrize("T", [1, 3])
def test_forward_topk_crafted(T):
    """The decode forward's own top-K on crafted logits: at T = 1 the selection fused
    into the single-token gate/up kernel (E = 256, K = 8), at T = 3 the batch route
    kernel.  Token t is one-hot at feature t, so its logits are column t of the
    router matrix; columns with infinities or NaN go one at a time (0 times them is
    NaN for the other tokens)."""
    import int4_grouped_expert_amd as coli
    H, I, E, K = 256, 256, 256, 8
    cases = crafted_logits(E, K, 77 + T)
    finite = [c for c in cases if np.isfinite(c[1]).all()]
    groups = [finite[i:i + T] for i in range(0, len(finite), T)]
    groups += [[c] for c in cases if not np.isfinite(c[1]).all()]
    wr = torch.zeros((E, H), dtype=torch.float32, device="cuda")
    layer, keep = small_layer(H, I, E, K, wr)
    for grp in groups:
        n = len(grp)
        log(f"forward crafted T {n}: {[c[0] for c in grp]}")
        wr.zero_()
        x = torch.zeros((n, H), dtype=torch.float32, device="cuda")
        for t, (_, col) in enumerate(grp):
            wr[:, t] = torch.from_numpy(col).cuda()
            x[t, t] = 1.0
        y = torch.empty((n, H), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(layer.workspace_bytes(n, coli.COLI_DECODE), 256), dtype=torch.uint8,
                         device="cuda")
        idx = torch.full((n, K), -7, dtype=torch.int32, device="cuda")
        gates = torch.empty((n, K), dtype=torch.float32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        coli.coli_moe_forward(layer, coli.COLI_DECODE, x, y, ws, idx, gates, status=status)
        torch.cuda.synchronize()
        idx_h, g_h = idx.cpu().numpy(), gates.cpu().numpy()
        for t, (name, col) in enumerate(grp):
            check_crafted(name, col, idx_h[t], g_h[t], K)
