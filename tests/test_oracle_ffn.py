"""Pins for the oracle's expert FFN, whole-layer forward and RMSNorm.

Expert matmul on int4-g64 planar weights: page "从源码开始colibri纯C引擎的编译、权重转换与
.bin直映射实战", section 权重转换 (the expert FFN consumes the converter's bytes
directly; dequantised weight = s * (u - 8)).  SiLU(gate)*up then down, the
gate-weighted combine and the shared expert with weight 1 are this build's reading
of the stages the pages name without formulas.
Each test reduces the oracle to library routines (torch fp64) or to closed forms.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rand_expert(rng, H, I, sd=0.02):
    wg = (rng.standard_normal((I, H)) * sd).astype(np.float32)
    wu = (rng.standard_normal((I, H)) * sd).astype(np.float32)
    wd = (rng.standard_normal((H, I)) * sd).astype(np.float32)
    return oracle.Expert.quantise(wg, wu, wd)


def torch_ffn(ex, x, H, I):
    """Dense SwiGLU with torch fp64 library routines on the dequantised weights."""
    wg = torch.from_numpy(oracle.dequant_int4_g64(ex.gq, ex.gs, H))
    wu = torch.from_numpy(oracle.dequant_int4_g64(ex.uq, ex.us, H))
    wd = torch.from_numpy(oracle.dequant_int4_g64(ex.dq, ex.ds, I))
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    h = F.silu(xt @ wg.T) * (xt @ wu.T)
    return (h @ wd.T).numpy(), h.numpy()


@pytest.mark.parametrize("H,I", [(256, 128), (192, 320), (100, 70)])
def test_ffn_is_dense_swiglu(H, I):
    rng = np.random.default_rng(H + I)
    ex = rand_expert(rng, H, I)
    x = rng.standard_normal((3, H))
    out, h = oracle.expert_ffn(ex, x, H, I, want_h=True)
    ref, href = torch_ffn(ex, x, H, I)
    assert np.allclose(h, href, rtol=1e-12, atol=1e-14)
    assert np.allclose(out, ref, rtol=1e-11, atol=1e-13)


def test_ffn_all_nibbles_eight_gives_zero():
    H, I = 128, 64
    z = np.zeros((I, H), dtype=np.float32)
    ex = oracle.Expert.quantise(z, z, np.zeros((H, I), dtype=np.float32))
    out = oracle.expert_ffn(ex, np.random.default_rng(0).standard_normal((2, H)), H, I)
    assert np.all(out == 0)


def test_ffn_one_hot_picks_column():
    """x = e_j: gate[o] = s[o, j//64] (u[o,j] - 8); checked through the planar bytes."""
    H, I = 192, 64
    rng = np.random.default_rng(9)
    ex = rand_expert(rng, H, I, sd=0.5)
    j = 133
    x = np.zeros((1, H))
    x[0, j] = 1.0
    _, h = oracle.expert_ffn(ex, x, H, I, want_h=True)
    g, b = j // 64, j % 64
    lo = b < 32
    ug = (ex.gq[:, g * 32 + b % 32] & 0xF) if lo else (ex.gq[:, g * 32 + b % 32] >> 4)
    uu = (ex.uq[:, g * 32 + b % 32] & 0xF) if lo else (ex.uq[:, g * 32 + b % 32] >> 4)
    gate = ex.gs[:, g].astype(np.float64) * (ug.astype(np.float64) - 8)
    up = ex.us[:, g].astype(np.float64) * (uu.astype(np.float64) - 8)
    assert np.allclose(h[0], gate / (1 + np.exp(-gate)) * up, rtol=1e-14, atol=0)


def torch_layer(x, wr, bias, experts, shared, H, I, K):
    """Whole layer via library routines: matmul, topk, softmax, dense SwiGLU."""
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    logits = xt @ torch.from_numpy(wr.astype(np.float64)).T
    if bias is not None:
        logits = logits + torch.from_numpy(bias.astype(np.float64))
    top = torch.topk(logits, K, dim=1)
    order = torch.argsort(top.indices, dim=1)
    idx = torch.gather(top.indices, 1, order)
    gates = torch.softmax(torch.gather(logits, 1, idx), dim=1)
    y = np.zeros((x.shape[0], H))
    for t in range(x.shape[0]):
        for k in range(K):
            o, _ = torch_ffn(experts[int(idx[t, k])], x[t:t + 1], H, I)
            y[t] += float(gates[t, k]) * o[0]
        o, _ = torch_ffn(shared, x[t:t + 1], H, I)
        y[t] += o[0]
    return y, idx.numpy().astype(np.int32), gates.numpy()


@pytest.mark.parametrize("bias", [False, True])
def test_moe_forward_matches_library_composition(bias):
    H, I, E, K, T = 128, 64, 8, 3, 4
    rng = np.random.default_rng(17 + bias)
    experts = [rand_expert(rng, H, I) for _ in range(E)]
    shared = rand_expert(rng, H, I)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32) if bias else None
    x = rng.standard_normal((T, H)).astype(np.float32)
    y, idx, gates = oracle.moe_forward(x, wr, b, experts, shared, H, I, K)
    yr, idxr, gr = torch_layer(x, wr, b, experts, shared, H, I, K)
    assert np.array_equal(idx, idxr)
    assert np.allclose(gates, gr, rtol=1e-13)
    assert np.allclose(y, yr, rtol=1e-10, atol=1e-12)


def test_moe_forward_unselected_experts_may_be_absent():
    H, I, E, K = 64, 64, 6, 2
    rng = np.random.default_rng(23)
    full = [rand_expert(rng, H, I) for _ in range(E)]
    shared = rand_expert(rng, H, I)
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    x = rng.standard_normal((1, H)).astype(np.float32)
    y, idx, _ = oracle.moe_forward(x, wr, None, full, shared, H, I, K)
    sparse = [full[e] if e in set(idx[0]) else None for e in range(E)]
    y2, _, _ = oracle.moe_forward(x, wr, None, sparse, shared, H, I, K)
    assert np.array_equal(y, y2)
    with pytest.raises(ValueError):
        oracle.moe_forward(x, wr, None, [None] * E, shared, H, I, K)


def test_moe_single_expert_gate_one_is_dense():
    """K = 1 with a zero shared expert is exactly that expert's dense SwiGLU."""
    H, I, E = 64, 64, 4
    rng = np.random.default_rng(29)
    experts = [rand_expert(rng, H, I) for _ in range(E)]
    z = np.zeros((I, H), dtype=np.float32)
    shared = oracle.Expert.quantise(z, z, np.zeros((H, I), dtype=np.float32))
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    x = rng.standard_normal((2, H)).astype(np.float32)
    y, idx, g = oracle.moe_forward(x, wr, None, experts, shared, H, I, 1)
    assert np.all(g == 1.0)
    for t in range(2):
        ref, _ = torch_ffn(experts[idx[t, 0]], x[t:t + 1], H, I)
        assert np.allclose(y[t], ref[0], rtol=1e-12, atol=1e-14)


def test_rmsnorm_closed_forms():
    c = np.array([[3.0] * 16, [-0.25] * 16])
    out = oracle.rmsnorm(c, 1e-6)
    assert np.allclose(out[0], 1 / np.sqrt(1 + 1e-6 / 9.0), rtol=1e-15)
    assert np.allclose(out[1], -1 / np.sqrt(1 + 1e-6 / 0.0625), rtol=1e-15)
    rng = np.random.default_rng(31)
    y = rng.standard_normal((4, 100))
    assert np.allclose(oracle.rmsnorm(y * 7.5, 0.0), oracle.rmsnorm(y, 0.0), rtol=1e-14)
    ref = F.rms_norm(torch.from_numpy(y), (100,), eps=1e-6).numpy()
    assert np.allclose(oracle.rmsnorm(y, 1e-6), ref, rtol=1e-13)
