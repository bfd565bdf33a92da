"""Pins for the oracle's router logits, top-K with renormalised gates, and permute.

Route step: page "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
section 十一 (the router selects the top-k experts of a token); the gates applied are
the normalised ones (page "colibrì 路由遥测全解析", section 分离计数与追踪); a NaN
router falls back to deterministic ids (same page, section 测试与 CI 保障).
Batch union: page "Colibrì 深度解析", section 四 (positions routed to the same expert
are grouped so the expert is read once).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle


def brute_topk(l, K):
    """The unique K-subset whose smallest logit beats every unselected one."""
    E = len(l)
    found = []
    for S in itertools.combinations(range(E), K):
        rest = [l[e] for e in range(E) if e not in S]
        if not rest or min(l[e] for e in S) > max(rest):
            found.append(S)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("E,K", [(4, 1), (5, 2), (8, 3), (10, 4), (12, 6), (12, 12),
                                 (9, 8)])
def test_topk_brute_force(E, K):
    rng = np.random.default_rng(E * 100 + K)
    for _ in range(20):
        l = rng.standard_normal((1, E))
        idx, g, fb = oracle.topk(l, K)
        assert fb == 0
        assert list(idx[0]) == brute_topk(list(l[0]), K)
        assert list(idx[0]) == sorted(idx[0])  # ascending expert id


def test_gates_sum_and_softmax_restriction():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((50, 64)) * 3
    K = 8
    idx, g, _ = oracle.topk(l, K)
    assert np.all(np.abs(g.sum(1) - 1) <= K * 2.0 ** -52)
    # softmax over all E (library), restricted to the selected K and renormalised
    full = torch.softmax(torch.from_numpy(l), dim=1).numpy()
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    ref = sel / sel.sum(1, keepdims=True)
    assert np.allclose(g, ref, rtol=1e-13, atol=0)
    # and equal to the softmax over the K selected logits
    ref2 = torch.softmax(torch.from_numpy(np.take_along_axis(l, idx.astype(np.int64), 1)),
                         dim=1).numpy()
    assert np.allclose(g, ref2, rtol=1e-13, atol=0)


def test_k_equals_e_is_library_softmax():
    rng = np.random.default_rng(2)
    l = rng.standard_normal((7, 16))
    idx, g, _ = oracle.topk(l, 16)
    assert np.array_equal(idx, np.tile(np.arange(16, dtype=np.int32), (7, 1)))
    assert np.allclose(g, torch.softmax(torch.from_numpy(l), 1).numpy(), rtol=1e-14, atol=0)


def test_k_one_gate_is_exactly_one():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((9, 32))
    idx, g, _ = oracle.topk(l, 1)
    assert np.array_equal(idx[:, 0], np.argmax(l, axis=1))
    assert np.all(g == 1.0)


def test_ties_go_to_lower_id():
    l = np.array([[0.5, 2.0, 1.0, 2.0, 1.0, 1.0, -3.0]])
    idx, _, _ = oracle.topk(l, 3)
    assert list(idx[0]) == [1, 2, 3]  # 2.0, 2.0 then the lowest-id 1.0
    idx, _, _ = oracle.topk(l, 5)
    assert list(idx[0]) == [1, 2, 3, 4, 5]  # all three 1.0s before 0.5


def test_nan_never_wins_and_fallback():
    l = np.array([[np.nan, 0.1, np.nan, -0.2, np.nan, np.nan]])
    idx, _, fb = oracle.topk(l, 2)
    assert fb == 0 and list(idx[0]) == [1, 3]
    # three rounds: two real picks, then a fallback round (round 2 -> id 2 is free)
    idx, _, fb = oracle.topk(l, 3)
    assert fb == 1 and list(idx[0]) == [1, 2, 3]
    # all NaN: round k takes id k
    idx, g, fb = oracle.topk(np.full((1, 6), np.nan), 4)
    assert fb == 4 and list(idx[0]) == [0, 1, 2, 3]
    assert np.all(np.isnan(g))
    # round k's own id already taken -> lowest free id
    l = np.array([[np.nan, np.nan, 5.0, np.nan]])
    idx, _, fb = oracle.topk(l, 3)  # round0 -> 2, round1 -> id 1, round2 -> id 2 taken -> 0
    assert fb == 2 and list(idx[0]) == [0, 1, 2]


def test_router_logits_library_matmul():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 96)).astype(np.float32)
    wr = (rng.standard_normal((12, 96)) * 0.02).astype(np.float32)
    b = rng.standard_normal(12).astype(np.float32)
    got = oracle.router_logits(x, wr, b)
    ref = (torch.from_numpy(x).double() @ torch.from_numpy(wr).double().T
           + torch.from_numpy(b).double()).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_router_logits_bf16_inputs():
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((3, 64)).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((8, 64)) * 0.02).astype(np.float32)).to(
        torch.bfloat16)
    got = oracle.router_logits(x.view(torch.int16).numpy().view(np.uint16),
                               wr.view(torch.int16).numpy().view(np.uint16))
    ref = (x.double() @ wr.double().T).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("T,K,E", [(1, 8, 256), (32, 8, 256), (7, 3, 10), (0, 4, 16),
                                   (64, 16, 16)])
def test_permute_matches_stable_argsort(T, K, E):
    rng = np.random.default_rng(T * 7 + K)
    rows = [np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]
    idx = (np.stack(rows) if rows else np.zeros((0, K))).astype(np.int32).reshape(T, K)
    counts, offsets, perm, unique = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(unique, np.unique(flat))


# ---------------------------------------------------------------- sigmoid router
# Page "Colibrì 深度解析", section 十一: the router of the GLM-class engine scores
# experts with a sigmoid, uses one expert group (n_group = 1) and the "noaux_tc"
# selection (no auxiliary loss: a per-expert bias shifts which experts are picked
# and nothing else); the gates are the selected scores normalised to sum 1.

def expit(z):
    from scipy.special import expit as sp_expit
    return sp_expit(np.asarray(z, dtype=np.float64))


def brute_keys(keys, K):
    return brute_topk(list(keys), K)


@pytest.mark.parametrize("E,K", [(4, 1), (6, 2), (8, 3), (10, 4), (12, 6), (12, 12), (9, 8)])
def test_sigmoid_brute_force(E, K):
    rng = np.random.default_rng(E * 131 + K)
    for _ in range(20):
        l = rng.standard_normal((1, E)) * 2
        b = (rng.standard_normal(E) * 0.3).astype(np.float32)
        idx, g, fb = oracle.topk_sigmoid(l, K, b)
        assert fb == 0
        keys = expit(l[0]) + b.astype(np.float64)
        assert list(idx[0]) == brute_keys(keys, K)
        s = expit(l[0][idx[0]])
        assert np.allclose(g[0], s / s.sum(), rtol=1e-14, atol=0)


def test_sigmoid_hand_worked():
    """l = (0, ln 3, -ln 3, 2), b = (0, 0, 0.6, -0.5), K = 2.  Scores (1/2, 3/4, 1/4,
    0.8808); keys (0.5, 0.75, 0.85, 0.3808): the bias brings expert 2 in and pushes
    expert 3 out; the gates use the scores alone: 3/4 / (3/4 + 1/4) and 1/4 / 1."""
    l = np.array([[0.0, np.log(3.0), -np.log(3.0), 2.0]])
    b = np.array([0.0, 0.0, 0.6, -0.5], dtype=np.float32)
    idx, g, fb = oracle.topk_sigmoid(l, 2, b)
    assert fb == 0 and list(idx[0]) == [1, 2]
    assert abs(g[0, 0] - 0.75) < 1e-15 and abs(g[0, 1] - 0.25) < 1e-15
    # without the bias the two largest scores win: experts 1 and 3
    idx, g, _ = oracle.topk_sigmoid(l, 2, None)
    assert list(idx[0]) == [1, 3]
    s3 = 1.0 / (1.0 + np.exp(-2.0))
    assert abs(g[0, 1] - s3 / (0.75 + s3)) < 1e-15


def test_sigmoid_without_bias_selects_like_softmax():
    """The sigmoid is increasing, so with no bias the selected set is the K largest
    logits (numpy argsort), as for the softmax router."""
    rng = np.random.default_rng(21)
    l = rng.standard_normal((40, 64)) * 3
    idx, g, _ = oracle.topk_sigmoid(l, 8, None)
    ref = np.sort(np.argsort(-l, axis=1, kind="stable")[:, :8], axis=1)
    assert np.array_equal(idx, ref)
    assert np.all(np.abs(g.sum(1) - 1) <= 8 * 2.0 ** -52)


def test_sigmoid_bias_is_selection_only():
    """A large bias forces expert 5 into every selection; its gate is still its own
    score over the selected scores, and shifting the bias without changing the
    selection leaves the gates bit-identical."""
    rng = np.random.default_rng(22)
    l = rng.standard_normal((16, 12))
    b = np.zeros(12, dtype=np.float32)
    b[5] = 10.0
    idx, g, _ = oracle.topk_sigmoid(l, 3, b)
    assert np.all(np.any(idx == 5, axis=1))
    s = expit(np.take_along_axis(l, idx.astype(np.int64), 1))
    assert np.allclose(g, s / s.sum(1, keepdims=True), rtol=1e-14, atol=0)
    idx2, g2, _ = oracle.topk_sigmoid(l, 3, b * 2)
    assert np.array_equal(idx, idx2) and np.array_equal(g, g2)


def test_sigmoid_k_one_and_k_equals_e():
    rng = np.random.default_rng(23)
    l = rng.standard_normal((9, 16))
    b = (rng.standard_normal(16) * 0.1).astype(np.float32)
    idx, g, _ = oracle.topk_sigmoid(l, 1, b)
    assert np.array_equal(idx[:, 0], np.argmax(expit(l) + b.astype(np.float64), axis=1))
    assert np.all(g == 1.0)
    idx, g, _ = oracle.topk_sigmoid(l, 16, b)
    assert np.array_equal(idx, np.tile(np.arange(16, dtype=np.int32), (9, 1)))
    s = expit(l)
    assert np.allclose(g, s / s.sum(1, keepdims=True), rtol=1e-14, atol=0)


def test_sigmoid_nan_fallback():
    l = np.array([[np.nan, 0.3, np.nan, -0.2]])
    idx, _, fb = oracle.topk_sigmoid(l, 3, None)
    assert fb == 1 and list(idx[0]) == [1, 2, 3]  # two picks, then round 2 -> id 2
    idx, g, fb = oracle.topk_sigmoid(np.full((1, 5), np.nan), 2, None)
    assert fb == 2 and list(idx[0]) == [0, 1] and np.all(np.isnan(g))


def test_sigmoid_layer_reduces_to_dense_swiglu_sum():
    """The whole layer under the sigmoid router equals the gate-weighted sum of the
    selected experts' outputs (each expert run alone through the oracle's pinned
    expert FFN) plus the shared expert, with the gates of topk_sigmoid."""
    rng = np.random.default_rng(24)
    H, I, E, K = 128, 64, 8, 3
    exps = [oracle.Expert.quantise(*(rng.standard_normal(s).astype(np.float32) * 0.05
                                     for s in ((I, H), (I, H), (H, I)))) for _ in range(E + 1)]
    wr = (rng.standard_normal((E, H)) * 0.1).astype(np.float32)
    b = (rng.standard_normal(E) * 0.2).astype(np.float32)
    x = rng.standard_normal((4, H)).astype(np.float32)
    y, idx, g = oracle.moe_forward(x, wr, b, exps[:E], exps[E], H, I, K, scoring=oracle.SIGMOID)
    l = x.astype(np.float64) @ wr.astype(np.float64).T
    ridx, rg, _ = oracle.topk_sigmoid(l, K, b)
    assert np.array_equal(idx, ridx) and np.allclose(g, rg, rtol=1e-12, atol=0)
    for t in range(4):
        ref = oracle.expert_ffn(exps[E], x[t:t + 1].astype(np.float64), H, I)[0]
        for k in range(K):
            ref = ref + g[t, k] * oracle.expert_ffn(exps[idx[t, k]],
                                                    x[t:t + 1].astype(np.float64), H, I)[0]
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-15)
