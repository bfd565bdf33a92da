"""Seeded random layer shapes through coli_moe_forward, each against the oracle:
H in [1, 700], I in [1, 320], E in [1, 40], K in [1, min(E, 8)], decode T in [1, 70]
and prefill T in [1, 150], fp32 or bf16 routers, no bias, a Zipf bias or a sigmoid
router's selection bias; a second set with E in [41, 300] and K up to 16 (the
top-K's 2, 4 and 8 logits per lane).  A few draws put H and I on multiples of 256 at T = 1 (the
single-token int8 path); the rest take the batch and prefill paths with ragged
groups and rows of any alignment.  Every case checks ids bit-exact, gates and y row
by row (the same bars as the named workloads)."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.harness import DeviceLayer, host_array, log, margin_tokens
from tests.test_gpu_forward import DECODE, PREFILL, oracle_check

pytestmark = pytest.mark.gpu

N_CASES = 24
N_WIDE = 12
BASE_ID = 300


def draw_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(N_CASES):
        mode = "prefill" if i % 3 == 2 else "decode"
        if i % 8 == 1:  # single-token int8 path
            H, I = 256 * int(rng.integers(1, 4)), 256 * int(rng.integers(1, 3))
            T = 1
        else:
            H, I = int(rng.integers(1, 701)), int(rng.integers(1, 321))
            T = int(rng.integers(1, 71 if mode == "decode" else 151))
        E = int(rng.integers(1, 41))
        K = int(rng.integers(1, min(E, 8) + 1))
        kind = ("none", "zipf", "sel")[i % 3]
        cfg = dict(name=f"random_{i}", H=H, I=I, E=E, K=K, T=T,
                   router="bf16" if rng.integers(0, 2) else "f32",
                   x="bf16" if mode == "prefill" else "f32",
                   bias=None if kind == "none" else kind, mode=mode, layers=1)
        if kind == "sel":
            cfg["scoring"] = "sigmoid"
        cases.append((BASE_ID + i, cfg))
    # wider routers: E in [41, 300], K up to 16
    rng = np.random.default_rng(20261203)
    for i in range(N_WIDE):
        mode = "prefill" if i % 4 == 3 else "decode"
        E = int(rng.integers(41, 301))
        K = int(rng.integers(1, min(E, 16) + 1))
        if i % 4 == 1 and E <= 256:  # single-token int8 path
            H, I = 256 * int(rng.integers(1, 3)), 256 * int(rng.integers(1, 3))
            T = 1
        else:
            H, I = int(rng.integers(64, 513)), int(rng.integers(1, 257))
            T = int(rng.integers(1, 49 if mode == "decode" else 121))
        kind = ("none", "zipf", "sel")[i % 3]
        cfg = dict(name=f"random_wide_{i}", H=H, I=I, E=E, K=K, T=T,
                   router="bf16" if rng.integers(0, 2) else "f32",
                   x="bf16" if mode == "prefill" else "f32",
                   bias=None if kind == "none" else kind, mode=mode, layers=1)
        if kind == "sel":
            cfg["scoring"] = "sigmoid"
        cases.append((BASE_ID + N_CASES + i, cfg))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("cfg_id,cfg", CASES, ids=[c[1]["name"] for c in CASES])
def test_random_shape(cfg_id, cfg):
    W.CONFIGS[cfg_id] = cfg
    c = cfg
    log(f"random shape {c['name']}: H {c['H']} I {c['I']} E {c['E']} K {c['K']} T {c['T']} "
        f"{c['mode']} router {c['router']} bias {c['bias']}")
    L = DeviceLayer(cfg_id)
    x = margin_tokens(cfg_id, c["T"], host_array(L.w_router), L.bias_np, c["K"])
    mode = PREFILL if c["mode"] == "prefill" else DECODE
    y, idx, gates = L.forward(x, mode)
    torch.cuda.synchronize()
    oracle_check(cfg_id, L, x, y, idx, gates, mode)


CACHE_CASES = [c for c in CASES if c[1]["T"] * c[1]["K"] < c[1]["E"] or c[1]["T"] <= 3][:8]


@pytest.mark.parametrize("cfg_id,cfg", CACHE_CASES, ids=[c[1]["name"] for c in CACHE_CASES])
def test_random_shape_through_cache(cfg_id, cfg):
    """The same shapes through the two-phase forward and an expert cache of fewer
    slots than experts where the batch allows: bit-identical to the resident
    forward over a few batches."""
    import int4_grouped_expert_amd as coli
    from tests.test_gpu_cache import CachedLayer, same
    W.CONFIGS[cfg_id] = cfg
    c = cfg
    mode = PREFILL if c["mode"] == "prefill" else DECODE
    S = min(c["E"], max(1, c["T"] * c["K"]) + 1)
    log(f"random shape through cache {c['name']}: E {c['E']} S {S} T {c['T']} {c['mode']}")
    L = DeviceLayer(cfg_id)
    cl = CachedLayer(coli, L, S)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    for b in range(4):
        x = W.tokens(cfg_id, c["T"], "cuda", draw=40 + b)
        y_ref, idx_ref, _ = L.forward(x, mode)
        y, idx, _ = cl.forward(x, mode, st, repin=(b == 2))
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(idx, idx_ref)
        assert same(y, y_ref), f"batch {b}"
