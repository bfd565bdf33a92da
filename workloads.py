"""Seeded synthetic inputs for the MoE-layer workloads (no method arithmetic here).

Both the HIP path and the oracle consume the tensors drawn here; neither side draws
its own.  Every tensor has its own 63-bit seed derived with numpy's SeedSequence from
(base seed + workload id, tensor tag, layer, index), and is drawn with torch's
generator on the requested device (Philox on the GPU, mt19937 on the CPU), so a
tensor is reproducible per device type.  Tests copy device draws to the host for the
oracle; they never mix a CPU draw with a GPU draw of the same tensor.

Workloads (shapes of the pages' 256-expert, top-8, ~19 MB-per-expert layers; the
values are synthetic since no trained checkpoint is used):
  tiny        H=256,  I=128,  E=16,  K=4, T=1,    router fp32, x fp32 (decode)
  decode      H=6144, I=2048, E=256, K=8, T=1,    router bf16, x fp32 (decode)
  decode_zipf same layer, T=32, router bias for Zipf(1.1) selections (decode)
  prefill     same layer, T=2048, x bf16 (prefill)
  stack       40 layers of the decode shape, T=8, Zipf bias per layer with its own
              expert permutation, RMSNorm between layers
Weights are N(0, 0.02) fp32 (quantised by the caller), router N(0, 0.02), x N(0, 1).
"""
from __future__ import annotations

import numpy as np
import torch

SEED_BASE = 20261202

CONFIGS = {
    0: dict(name="tiny", H=256, I=128, E=16, K=4, T=1, router="f32", x="f32", bias=None,
            mode="decode", layers=1),
    1: dict(name="decode", H=6144, I=2048, E=256, K=8, T=1, router="bf16", x="f32", bias=None,
            mode="decode", layers=1),
    2: dict(name="decode_zipf", H=6144, I=2048, E=256, K=8, T=32, router="bf16", x="f32",
            bias="zipf", mode="decode", layers=1),
    3: dict(name="prefill", H=6144, I=2048, E=256, K=8, T=2048, router="bf16", x="bf16",
            bias=None, mode="prefill", layers=1),
    4: dict(name="stack", H=6144, I=2048, E=256, K=8, T=8, router="bf16", x="f32", bias="zipf",
            mode="decode", layers=40),
}

# Smaller shapes used only as parity cases (ragged tiles, edge cases); same recipe.
CONFIGS.update({
    100: dict(name="small_prefill", H=384, I=192, E=24, K=6, T=333, router="bf16", x="bf16",
              bias=None, mode="prefill", layers=1),
    101: dict(name="small_decode_zipf", H=384, I=192, E=24, K=6, T=40, router="bf16", x="f32",
              bias="zipf", mode="decode", layers=1),
    102: dict(name="k_equals_e", H=128, I=64, E=8, K=8, T=5, router="f32", x="f32", bias=None,
              mode="decode", layers=1),
    103: dict(name="k_one", H=128, I=64, E=8, K=1, T=3, router="f32", x="f32", bias=None,
              mode="decode", layers=1),
    104: dict(name="small_prefill_f32_router", H=256, I=128, E=16, K=4, T=200, router="f32",
              x="bf16", bias="zipf", mode="prefill", layers=1),
    105: dict(name="small_stack", H=256, I=128, E=16, K=4, T=8, router="bf16", x="f32",
              bias="zipf", mode="decode", layers=40),
    106: dict(name="wide_decode", H=10240, I=320, E=12, K=3, T=3, router="bf16", x="f32",
              bias=None, mode="decode", layers=1),
    # single-token shapes with H, I multiples of 256 (the int8 matrix-core decode path):
    # K slices of 1..6 chunks per wave, 1..8 down waves, 2..17 units
    107: dict(name="one_token_small", H=512, I=512, E=16, K=4, T=1, router="f32", x="f32",
              bias=None, mode="decode", layers=1),
    108: dict(name="one_token_mid", H=1536, I=768, E=40, K=6, T=1, router="bf16", x="f32",
              bias="zipf", mode="decode", layers=1),
    109: dict(name="one_token_k16", H=1024, I=256, E=64, K=16, T=1, router="bf16", x="f32",
              bias=None, mode="decode", layers=1),
    110: dict(name="one_token_wide", H=10240, I=512, E=12, K=3, T=1, router="bf16", x="f32",
              bias=None, mode="decode", layers=1),
    111: dict(name="one_token_h2048", H=2048, I=1024, E=32, K=8, T=1, router="f32", x="f32",
              bias="zipf", mode="decode", layers=1),
    112: dict(name="one_token_h4096", H=4096, I=2048, E=20, K=5, T=1, router="bf16", x="f32",
              bias=None, mode="decode", layers=1),
    # single-token top-8 shapes whose gate/up and down kernels run the same block shape
    # (I/8 blocks of I/256 waves): one wave per block, four waves per block
    113: dict(name="one_token_fused_small", H=768, I=256, E=32, K=8, T=1, router="bf16",
              x="f32", bias=None, mode="decode", layers=1),
    114: dict(name="one_token_fused_h3072", H=3072, I=1024, E=64, K=8, T=1, router="f32",
              x="f32", bias="zipf", mode="decode", layers=1),
    # the sigmoid router ("n_group=1 sigmoid + noaux_tc"): raw logits, a selection bias
    115: dict(name="sigmoid_decode", H=384, I=192, E=24, K=6, T=40, router="bf16", x="f32",
              bias="sel", mode="decode", layers=1, scoring="sigmoid"),
    116: dict(name="sigmoid_one_token", H=512, I=512, E=16, K=4, T=1, router="f32", x="f32",
              bias="sel", mode="decode", layers=1, scoring="sigmoid"),
    117: dict(name="sigmoid_prefill", H=256, I=128, E=16, K=4, T=200, router="bf16", x="bf16",
              bias="sel", mode="prefill", layers=1, scoring="sigmoid"),
    118: dict(name="sigmoid_full", H=6144, I=2048, E=256, K=8, T=32, router="bf16", x="f32",
              bias="sel", mode="decode", layers=1, scoring="sigmoid"),
    # ragged shapes: H and I not multiples of 64 (zero-padded last groups), rows of
    # any alignment
    119: dict(name="ragged_decode", H=200, I=72, E=12, K=3, T=5, router="f32", x="f32",
              bias=None, mode="decode", layers=1),
    120: dict(name="ragged_prefill", H=100, I=70, E=10, K=2, T=77, router="bf16", x="bf16",
              bias=None, mode="prefill", layers=1),
    121: dict(name="ragged_decode_bf16", H=130, I=200, E=16, K=4, T=33, router="bf16", x="f32",
              bias="zipf", mode="decode", layers=1),
    122: dict(name="ragged_prefill_wide", H=1000, I=330, E=20, K=5, T=150, router="bf16",
              x="bf16", bias="zipf", mode="prefill", layers=1),
    # the largest expert count the boundary accepts (E = 1024), with top-8 and with
    # every expert selected (K = E)
    123: dict(name="max_experts", H=256, I=128, E=1024, K=8, T=5, router="bf16", x="f32",
              bias=None, mode="decode", layers=1),
    124: dict(name="max_experts_all_selected", H=128, I=64, E=1024, K=1024, T=2, router="f32",
              x="f32", bias=None, mode="decode", layers=1),
    125: dict(name="max_experts_prefill", H=256, I=128, E=1024, K=8, T=300, router="bf16",
              x="bf16", bias=None, mode="prefill", layers=1),
    # the largest H and I the boundary accepts (65536), each beside a small other side
    126: dict(name="max_hidden", H=65536, I=128, E=8, K=2, T=3, router="bf16", x="f32",
              bias=None, mode="decode", layers=1),
    127: dict(name="max_intermediate", H=128, I=65536, E=4, K=2, T=3, router="f32", x="f32",
              bias=None, mode="decode", layers=1),
    128: dict(name="max_hidden_prefill", H=65536, I=64, E=4, K=2, T=40, router="bf16",
              x="bf16", bias=None, mode="prefill", layers=1),
    129: dict(name="max_intermediate_prefill", H=64, I=65536, E=4, K=2, T=40, router="bf16",
              x="bf16", bias=None, mode="prefill", layers=1),
    # few experts, many tokens: every routed expert spans several M-chunks (128 tokens
    # in prefill, 32 in a decode batch)
    130: dict(name="many_chunks_prefill", H=256, I=128, E=4, K=2, T=1024, router="bf16",
              x="bf16", bias=None, mode="prefill", layers=1),
    131: dict(name="many_chunks_decode", H=256, I=128, E=4, K=2, T=256, router="f32",
              x="f32", bias=None, mode="decode", layers=1),
})

WEIGHT_STD = 0.02
ROUTER_STD = 0.02
ZIPF_S = 1.1
ZIPF_TAU = 0.8  # logit temperature of the bias: about 95 unique experts for 32 tokens x top-8

_TAGS = {"router": 1, "bias_perm": 2, "expert": 3, "x": 4}


# "Same layer as the decode workload": these draw their router and experts from it.
CONFIGS[2]["weights_from"] = 1
CONFIGS[3]["weights_from"] = 1
CONFIGS[118]["weights_from"] = 1

SEL_BIAS_STD = 0.1  # the sigmoid router's selection bias: N(0, 0.1) per expert


def seed_for(cfg_id: int, tag: str, layer: int = 0, index: int = 0) -> int:
    if tag in ("router", "expert"):
        cfg_id = CONFIGS[cfg_id].get("weights_from", cfg_id)
    ss = np.random.SeedSequence([SEED_BASE + cfg_id, _TAGS[tag], layer, index])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64((1 << 63) - 1))


def _randn(shape, seed: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def router_weights(cfg_id: int, device="cpu", layer: int = 0) -> torch.Tensor:
    c = CONFIGS[cfg_id]
    w = _randn((c["E"], c["H"]), seed_for(cfg_id, "router", layer), device) * ROUTER_STD
    return w.to(torch.bfloat16) if c["router"] == "bf16" else w


def expert_weights(cfg_id: int, e: int, device="cpu", layer: int = 0, shape=None):
    """fp32 (gate [I,H], up [I,H], down [H,I]) of expert e; e == E is the shared one."""
    c = CONFIGS[cfg_id]
    H, I = (c["H"], c["I"]) if shape is None else shape
    base = seed_for(cfg_id, "expert", layer, e)
    wg = _randn((I, H), base, device) * WEIGHT_STD
    wu = _randn((I, H), base ^ 0x5555, device) * WEIGHT_STD
    wd = _randn((H, I), base ^ 0xAAAA, device) * WEIGHT_STD
    return wg, wu, wd


def scoring(cfg_id: int) -> int:
    """0: softmax router (bias added to the logits), 1: sigmoid router (bias steers
    the selection only)."""
    return 1 if CONFIGS[cfg_id].get("scoring") == "sigmoid" else 0


def router_bias(cfg_id: int, layer: int = 0):
    """fp32 [E] router bias, or None.

    "zipf": b_e = tau * ln p_{pi(e)}, p_r proportional to r^-s over ranks r = 1..E, pi
    a seeded permutation of the experts (one per layer): selections follow Zipf(1.1).
    "sel": the sigmoid router's selection bias, N(0, SEL_BIAS_STD) per expert.
    """
    c = CONFIGS[cfg_id]
    if c["bias"] is None:
        return None
    E = c["E"]
    if c["bias"] == "sel":
        rng = np.random.default_rng(seed_for(cfg_id, "bias_perm", layer))
        return (rng.standard_normal(E) * SEL_BIAS_STD).astype(np.float32)
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** -ZIPF_S
    p /= p.sum()
    perm = np.random.default_rng(seed_for(cfg_id, "bias_perm", layer)).permutation(E)
    return (ZIPF_TAU * np.log(p[perm])).astype(np.float32)


def tokens(cfg_id: int, T: int, device="cpu", draw: int = 0) -> torch.Tensor:
    """x [T, H] N(0, 1) in the workload's activation dtype (draw = redraw counter)."""
    c = CONFIGS[cfg_id]
    x = _randn((T, c["H"]), seed_for(cfg_id, "x", 0, draw), device)
    return x.to(torch.bfloat16) if c["x"] == "bf16" else x


def token_pool(cfg_id: int, n: int, device="cpu", draw: int = 0) -> torch.Tensor:
    """n independent N(0,1) token rows (a pool to rotate over in timing loops)."""
    c = CONFIGS[cfg_id]
    x = _randn((n, c["H"]), seed_for(cfg_id, "x", 1, draw), device)
    return x.to(torch.bfloat16) if c["x"] == "bf16" else x
