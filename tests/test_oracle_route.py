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
