"""GPU routing counters (coli_usage_count) against the oracle's count: bit-exact, over
the routing of real forwards and over large random id arrays; then the counters go
through the library's history writer and the oracle's reader (page "colibrì 路由遥测
全解析：.coli_usage专家历史、ROUTE_TRACE追踪流与route_trace.h统一格式", section 历史文件)."""
import numpy as np
import pytest
import torch

import int4_grouped_expert_amd as coli
import workloads as W
from oracle import usage as U
from tests.harness import DeviceLayer, host_array, log, margin_tokens

pytestmark = pytest.mark.gpu


def test_usage_counts_of_stacked_forwards(tmp_path):
    cfg_id, NL, T = 105, 3, 8
    c = W.CONFIGS[cfg_id]
    E = c["E"]
    counts = torch.zeros((NL, E), dtype=torch.int64, device="cuda")
    ref = [[0] * E for _ in range(NL)]
    x = W.tokens(cfg_id, T, "cuda", 0)
    for l in range(NL):
        L = DeviceLayer(cfg_id, l)
        y, idx, _ = L.forward(x.contiguous(), 0)
        coli.coli_usage_count(idx, E, l, counts)
        coli.coli_usage_count(idx, E, l, counts)  # a second call adds again
        U.count_routes(idx.cpu().numpy(), NL, E, l, ref)
        U.count_routes(idx.cpu().numpy(), NL, E, l, ref)
        coli.coli_rmsnorm_f32(y, y, 1e-6)
        x = y
    torch.cuda.synchronize()
    got = counts.cpu().numpy().astype(np.uint64)
    assert got.tolist() == ref
    path = tmp_path / ".coli_usage"
    coli.coli_usage_save(str(path), got, coli.coli_usage_engine_hash("glm_moe_dsa"))
    back, total = U.read(path.read_bytes(), NL, E, "glm_moe_dsa")
    assert back == ref and total == 2 * NL * T * c["K"]


@pytest.mark.parametrize("T,K,E", [(65536, 8, 256), (333, 6, 24), (1, 1, 1024)])
def test_usage_count_random_ids(T, K, E):
    log(f"usage count T {T} K {K} E {E}")
    rng = np.random.default_rng(T + K + E)
    idx = rng.integers(-3, E + 3, size=(T, K)).astype(np.int32)  # some out of range
    counts = torch.zeros((2, E), dtype=torch.int64, device="cuda")
    coli.coli_usage_count(torch.from_numpy(idx).cuda(), E, 1, counts)
    torch.cuda.synchronize()
    ref = U.count_routes(idx, 2, E, 1)
    assert counts.cpu().numpy().tolist() == ref


@pytest.mark.parametrize("cfg_id,T,mode,path", [
    (107, 1, 0, "forward"),       # single-token int8 path: the fused top-K counts
    (114, 1, 0, "forward"),
    (101, 40, 0, "forward"),      # decode batch route
    (0, 300, 0, "forward"),       # decode over 256 tokens: two route calls
    (100, 333, 1, "forward"),     # prefill route
    (115, 40, 0, "forward"),      # sigmoid router
    (107, 1, 0, "two_phase"),     # the route part counts, the experts part does not
    (101, 40, 0, "two_phase"),
    (107, 2, 0, "format"),        # the sibling-format layer's route
])
def test_forward_counts_routing_history(cfg_id, T, mode, path):
    """coli_moe_layer.usage: each forward adds its (token, slot) decisions to the
    layer's counters inside its routing kernels; three calls must equal three times
    the oracle's count of the returned ids, on every routing path."""
    log(f"fused usage cfg {cfg_id} T {T} mode {mode} path {path}")
    c = W.CONFIGS[cfg_id]
    E, K = c["E"], c["K"]
    L = DeviceLayer(cfg_id)
    usage = torch.zeros(E, dtype=torch.int64, device="cuda")
    ref = [[0] * E]
    for call in range(3):
        x = W.tokens(cfg_id, T, "cuda", draw=50 + call)
        if path == "format":
            from tests.test_gpu_formats import fmt_layer
            F = fmt_layer(cfg_id, 7)
            lay = coli.MoELayer(F.H, F.I, F.E, F.K, F.w_router, F.experts, F.shared, F.bias,
                                F.scoring, usage=usage)
            ws = torch.empty(coli.coli_moe_fmt_workspace_bytes(lay, 7, T), dtype=torch.uint8,
                             device="cuda")
            y = torch.empty((T, F.H), device="cuda")
            idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
            coli.coli_moe_forward_fmt(lay, 7, x, y, ws, idx)
        else:
            lay = coli.MoELayer(L.H, L.I, L.E, L.K, L.w_router, L.experts, L.shared, L.bias,
                                L.scoring, usage=usage)
            ws = torch.empty(max(lay.workspace_bytes(T, mode), 256), dtype=torch.uint8,
                             device="cuda")
            y = torch.empty((T, L.H), dtype=torch.float32 if mode == 0 else torch.bfloat16,
                            device="cuda")
            idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
            gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
            if path == "forward":
                coli.coli_moe_forward(lay, mode, x, y, ws, idx, gates)
            else:
                coli.coli_moe_route(lay, mode, x, ws, idx, gates)
                coli.coli_moe_experts(lay, mode, x, y, ws, idx, gates)
        torch.cuda.synchronize()
        U.count_routes(idx.cpu().numpy(), 1, E, 0, ref)
    assert usage.cpu().numpy().astype(np.uint64).tolist() == ref[0]
    assert sum(ref[0]) == 3 * T * K
