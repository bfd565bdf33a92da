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
