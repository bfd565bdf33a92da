"""GPU checks of the boundary's contracts beyond the headline workloads, each against
the oracle: the permute with repeated ids, the router without a logits array, the
sigmoid router ("n_group=1 sigmoid + noaux_tc", page "Colibrì 深度解析", section 十一),
ragged H and I (zero-padded last groups, page "从源码开始colibri纯C引擎的编译、权重转换
与.bin直映射实战", section 权重转换: ngroups = ceil(I / 64)), the largest expert count and dimensions,
decode batches longer than 256 tokens, and the device status flag (fail closed: page "colibrì 路由遥测全解析",
section 测试与 CI 保障).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.harness import (DEC_TOL, TIGHT_DEC, DeviceLayer, Timer, assert_close, check_rows,
                           host_array, log, margin_tokens, oracle_expert, oracle_topk)
from tests.test_gpu_forward import DECODE, PREFILL, oracle_check
from tests.test_gpu_route import run_permute

pytestmark = pytest.mark.gpu

_layers = {}


def layer(cfg_id):
    if cfg_id not in _layers:
        if W.CONFIGS[cfg_id]["H"] >= 4096:
            for k in [k for k in _layers if W.CONFIGS[k]["H"] >= 4096]:
                del _layers[k]
            torch.cuda.empty_cache()
        with Timer(f"build layer cfg {cfg_id}"):
            _layers[cfg_id] = DeviceLayer(cfg_id)
    return _layers[cfg_id]


# ---------------------------------------------------------------- permute


@pytest.mark.parametrize("T,K,E", [(5, 4, 8), (100, 8, 16), (700, 8, 64), (300, 16, 1024)])
def test_permute_repeated_ids(T, K, E):
    """Rows that name one expert several times: every (token, slot) pair is counted
    and placed, in the order of a stable sort (T * K <= 2048 takes the one-block
    path, larger the chunked one)."""
    log(f"permute repeated ids T {T} K {K} E {E}")
    rng = np.random.default_rng(T + 17 * K + E)
    idx = rng.integers(0, min(E, 6), size=(T, K)).astype(np.int32)  # many repeats per row
    got = run_permute(idx, E)
    ref = oracle.permute(idx, E)
    for g, r, name in zip(got, ref, ("counts", "offsets", "perm", "unique")):
        assert np.array_equal(g, r), name
    flat = idx.reshape(-1)
    assert np.array_equal(got[2], np.argsort(flat, kind="stable"))


# ---------------------------------------------------------------- router


def run_router(x, wr, bias, K, scoring, with_logits=True):
    import int4_grouped_expert_amd as coli
    T, E = x.shape[0], wr.shape[0]
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
    coli.coli_router_topk(x, wr, bias, K, idx, gates, logits, scoring=scoring)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), gates.cpu().numpy(), (logits.cpu().numpy() if with_logits else None)


@pytest.mark.parametrize("cfg_id,T", [(0, 9), (104, 200), (115, 40), (116, 1), (118, 32),
                                      (119, 5), (120, 77), (121, 33)])
@pytest.mark.parametrize("with_logits", [True, False])
def test_router_scored_parity(cfg_id, T, with_logits):
    """Ids bit-exact and gates within the spec bar, softmax and sigmoid scoring, any
    H (vector kernels, element-load kernel, logits kept on chip)."""
    log(f"router cfg {cfg_id} T {T} logits {with_logits}")
    c = W.CONFIGS[cfg_id]
    sc = W.scoring(cfg_id)
    wr = W.router_weights(cfg_id, "cuda").contiguous()
    b = W.router_bias(cfg_id)
    bias = None if b is None else torch.from_numpy(b).cuda()
    wr_h = host_array(wr)
    x = margin_tokens(cfg_id, T, wr_h, b, c["K"])
    idx, gates, logits = run_router(x, wr, bias, c["K"], sc, with_logits)
    ridx, rg, fb = oracle_topk(cfg_id, host_array(x), wr_h, b, c["K"])
    assert fb == 0
    assert np.array_equal(idx, ridx)
    assert_close(gates, rg, DEC_TOL, what="gates")
    assert np.all(np.abs(gates.astype(np.float64).sum(1) - 1) <= c["K"] * 2.0 ** -22)
    if with_logits:
        # softmax: the bias is in the logits; sigmoid: the logits are raw
        ref = oracle.router_logits(host_array(x), wr_h, b if sc == 0 else None)
        assert_close(logits, ref, 1e-4, what="logits")


# ---------------------------------------------------------------- forward


@pytest.mark.parametrize("cfg_id,T,mode", [(115, 40, DECODE), (115, 1, DECODE),
                                           (116, 1, DECODE), (116, 3, DECODE),
                                           (117, 200, PREFILL), (117, 1, PREFILL)])
def test_forward_sigmoid(cfg_id, T, mode):
    """The whole layer under the sigmoid router, decode (single-token int8 path and
    batch path) and prefill."""
    log(f"sigmoid forward cfg {cfg_id} T {T} mode {mode}")
    L = layer(cfg_id)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    if mode == PREFILL:
        x = x.to(torch.bfloat16) if x.dtype != torch.bfloat16 else x
    y, idx, gates = L.forward(x, mode)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, mode)


def test_forward_sigmoid_full_size():
    """The decode-shaped layer under the sigmoid router: T = 32 and T = 1."""
    L = layer(118)
    for T in (32, 1):
        log(f"sigmoid full size T {T}")
        x = margin_tokens(118, T, host_array(L.w_router), L.bias_np, L.K)
        y, idx, gates = L.forward(x, DECODE)
        torch.cuda.synchronize()
        oracle_check(118, L, x, y, idx, gates, DECODE, check_bytes=(T == 32))


@pytest.mark.parametrize("cfg_id,T,mode", [(119, 5, DECODE), (119, 1, DECODE),
                                           (121, 33, DECODE), (120, 77, PREFILL),
                                           (120, 1, PREFILL), (122, 150, PREFILL),
                                           (122, 3, DECODE)])
def test_forward_ragged(cfg_id, T, mode):
    """H and I that are not multiples of 64 (and rows that are not 16-byte aligned):
    the last group of every row is zero padded by the quantiser and the kernels."""
    log(f"ragged forward cfg {cfg_id} T {T} mode {mode}")
    L = layer(cfg_id)
    c = W.CONFIGS[cfg_id]
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    # a bf16 draw passed as fp32 keeps its values (and its routing margin)
    assert c["x"] == "bf16" or mode == DECODE
    x = x.to(torch.bfloat16 if mode == PREFILL else torch.float32).contiguous()
    y, idx, gates = L.forward(x, mode)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, mode)


@pytest.mark.parametrize("cfg_id,T,mode", [(123, 1, DECODE), (123, 5, DECODE),
                                           (124, 1, DECODE), (124, 2, DECODE),
                                           (125, 300, PREFILL), (125, 1, PREFILL)])
def test_forward_max_experts(cfg_id, T, mode):
    """E = 1024, the largest expert count the boundary accepts, with top-8 and with
    K = E (every expert selected: the gates are the softmax over all 1024 logits)."""
    log(f"max experts forward cfg {cfg_id} T {T} mode {mode}")
    L = layer(cfg_id)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    y, idx, gates = L.forward(x, mode)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, mode)


@pytest.mark.parametrize("cfg_id,T,mode", [(126, 3, DECODE), (126, 1, DECODE),
                                           (127, 3, DECODE), (128, 40, PREFILL),
                                           (129, 40, PREFILL)])
def test_forward_max_dims(cfg_id, T, mode):
    """H = 65536 or I = 65536, the largest dimension the boundary accepts."""
    log(f"max dims forward cfg {cfg_id} T {T} mode {mode}")
    L = layer(cfg_id)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    y, idx, gates = L.forward(x, mode)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, mode)


@pytest.mark.parametrize("cfg_id,T,mode", [(130, 1024, PREFILL), (131, 256, DECODE),
                                           (131, 100, DECODE)])
def test_forward_many_chunks(cfg_id, T, mode):
    """Four experts, top-2, hundreds of tokens: each routed expert spans several
    M-chunks of the grouped GEMMs (and the shared expert many more)."""
    log(f"many chunks forward cfg {cfg_id} T {T} mode {mode}")
    L = layer(cfg_id)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    y, idx, gates = L.forward(x, mode)
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=L.E)
    log(f"tokens per expert {counts.tolist()}")
    assert counts.min() > (128 if mode == PREFILL else 32)
    oracle_check(cfg_id, L, x, y, idx, gates, mode)


@pytest.mark.parametrize("cfg_id,T", [(0, 300), (101, 600)])
def test_decode_longer_than_256(cfg_id, T):
    """Decode batches beyond 256 tokens run as consecutive 256-token batches."""
    log(f"decode long cfg {cfg_id} T {T}")
    L = layer(cfg_id)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    y, idx, gates = L.forward(x, DECODE)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, DECODE)


# ---------------------------------------------------------------- status flag


def run_with_status(L, x, mode):
    import int4_grouped_expert_amd as coli
    T = x.shape[0]
    dtype = torch.float32 if mode == DECODE else torch.bfloat16
    y = torch.empty((T, L.H), dtype=dtype, device="cuda")
    ws = torch.empty(max(L.layer_c.workspace_bytes(T, mode), 256), dtype=torch.uint8,
                     device="cuda")
    idx = torch.empty((T, L.K), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, L.K), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    coli.coli_moe_forward(L.layer_c, mode, x, y, ws, idx, gates, status=st)
    torch.cuda.synchronize()
    return y, idx, gates, int(st.item())


def test_unfinished_blob_fails_closed():
    """Experts quantised into their blobs with coli_quant_int4_g64 alone (no
    coli_expert_finish): a decode forward gives NaN outputs and raises
    COLI_STATUS_UNFINISHED, on the batch path and the single-token path; prefill,
    which reads the format's own row-major scales, is unaffected.  After
    coli_expert_finish the decode forward matches the oracle."""
    import int4_grouped_expert_amd as coli
    for cfg_id, T in ((0, 3), (107, 1)):
        c = W.CONFIGS[cfg_id]
        H, I, E, K = c["H"], c["I"], c["E"], c["K"]
        L = DeviceLayer(cfg_id)
        # a fresh set of blobs holding the same experts, never finished
        experts, shared, nb = coli.alloc_layer_blobs(H, I, E)
        experts.fill_(0x5A)
        shared.fill_(0x5A)
        for e in range(E + 1):
            wg, wu, wd = W.expert_weights(cfg_id, e, "cuda")
            ptr = shared.data_ptr() if e == E else experts.data_ptr() + e * nb
            coli.coli_quant_expert(ptr, H, I, wg, wu, wd, finish=False)
        L.experts, L.shared = experts, shared
        L.layer_c = coli.MoELayer(H, I, E, K, L.w_router, experts, shared, L.bias, L.scoring)
        x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, K)
        y, idx, gates, st = run_with_status(L, x, DECODE)
        log(f"unfinished cfg {cfg_id} T {T}: status {st}")
        assert st & coli.COLI_STATUS_UNFINISHED
        assert torch.isnan(y).all(), "every token reads the unfinished shared expert"
        # prefill reads only the row-major scales: correct, no flag
        xp = x.to(torch.bfloat16).contiguous()
        yp, ip, gp, stp = run_with_status(L, xp, PREFILL)
        assert stp == 0
        oracle_check(cfg_id, L, xp, yp, ip, gp, PREFILL, check_bytes=False)
        # finished: decode parity
        for e in range(E + 1):
            coli.coli_expert_finish(shared.data_ptr() if e == E else experts.data_ptr() + e * nb,
                                    H, I)
        y2, idx2, gates2, st2 = run_with_status(L, x, DECODE)
        assert st2 == 0
        oracle_check(cfg_id, L, x, y2, idx2, gates2, DECODE)


def test_prefill_range_flag():
    """A layer whose weights are large (group scales around 20) drives h past the
    fp16 range even after the per-token scaling: COLI_STATUS_RANGE is raised."""
    import int4_grouped_expert_amd as coli
    H, I, E, K = 256, 128, 8, 2
    g = torch.Generator(device="cuda").manual_seed(5)
    wr = (torch.randn((E, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    experts, shared, nb = coli.alloc_layer_blobs(H, I, E)
    for e in range(E + 1):
        ws = [torch.randn(s, generator=g, device="cuda") * 40.0 for s in ((I, H), (I, H), (H, I))]
        ptr = shared.data_ptr() if e == E else experts.data_ptr() + e * nb
        coli.coli_quant_expert(ptr, H, I, *ws)
    lay = coli.MoELayer(H, I, E, K, wr, experts, shared)
    x = torch.randn((4, H), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty((4, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(lay.workspace_bytes(4, PREFILL), dtype=torch.uint8, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    coli.coli_moe_forward(lay, PREFILL, x, y, ws, status=st)
    torch.cuda.synchronize()
    log(f"range flag status {int(st.item())}")
    assert int(st.item()) & coli.COLI_STATUS_RANGE


@pytest.mark.parametrize("cfg_id,T,mode", [(0, 3, DECODE), (107, 1, DECODE), (100, 5, PREFILL)])
def test_nonfinite_input_flag(cfg_id, T, mode):
    """A token holding Inf or NaN: its y is non-finite and COLI_STATUS_NONFINITE is
    raised; the other tokens are unaffected."""
    import int4_grouped_expert_amd as coli
    L = layer(cfg_id)
    x = margin_tokens(cfg_id, T, host_array(L.w_router), L.bias_np, L.K)
    if mode == PREFILL:
        x = x.to(torch.bfloat16)
    x = x.clone()
    x[T - 1, 7] = float("inf")
    y, idx, gates, st = run_with_status(L, x, mode)
    log(f"nonfinite cfg {cfg_id}: status {st}")
    assert st & coli.COLI_STATUS_NONFINITE
    assert not torch.isfinite(y[T - 1].float()).all()
    if T > 1:
        oracle_check(cfg_id, L, x[:T - 1].contiguous(), y[:T - 1], idx[:T - 1], gates[:T - 1],
                     mode, check_bytes=False)
