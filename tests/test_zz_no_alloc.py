"""coli_moe_forward_noalloc (workspace in the library's static device scratch)
against coli_moe_forward (caller's workspace) through the C ABI: two calls in a row
on one layer, the second with fewer tokens, each output identical to the existing
entry point's and within the oracle bars; decode on the batch and single-token
paths and prefill."""
import numpy as np
import pytest
import torch

import workloads as W
from tests.harness import DeviceLayer, check_rows, host_array, log, margin_tokens, oracle_topk

pytestmark = pytest.mark.gpu

DECODE, PREFILL = 0, 1


def both(L, x, mode):
    import int4_grouped_expert_amd as coli
    T = x.shape[0]
    dtype = torch.float32 if mode == DECODE else torch.bfloat16
    outs = []
    for noalloc in (False, True):
        y = torch.full((T, L.H), float("nan"), dtype=dtype, device="cuda")
        idx = torch.full((T, L.K), -1, dtype=torch.int32, device="cuda")
        gates = torch.full((T, L.K), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.zeros(1, dtype=torch.int32, device="cuda")
        if noalloc:
            coli.coli_moe_forward_noalloc(L.layer_c, mode, x, y, idx, gates, status=st)
        else:
            ws = torch.empty(L.layer_c.workspace_bytes(T, mode), dtype=torch.uint8, device="cuda")
            coli.coli_moe_forward(L.layer_c, mode, x, y, ws, idx, gates, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        outs.append((y, idx, gates))
    return outs


@pytest.mark.parametrize("cfg_id,mode,Ts", [(0, DECODE, (9, 4)), (107, DECODE, (1, 1)),
                                            (100, PREFILL, (65, 20))])
def test_noalloc_matches_forward(cfg_id, mode, Ts):
    import oracle
    L = DeviceLayer(cfg_id)
    c = W.CONFIGS[cfg_id]
    xs = margin_tokens(cfg_id, Ts[0], host_array(L.w_router), L.bias_np, L.K)
    for call, T in enumerate(Ts):
        log(f"noalloc cfg {cfg_id} mode {mode} call {call} T {T}")
        x = xs[call:call + T].contiguous() if T < Ts[0] else xs
        (y0, i0, g0), (y1, i1, g1) = both(L, x, mode)
        assert torch.equal(i0, i1) and torch.equal(g0, g1)
        assert torch.equal(y0, y1), "no-alloc output differs from coli_moe_forward"
        # and the oracle's bars, on the routing and the output
        from tests.test_gpu_forward import oracle_check
        oracle_check(cfg_id, L, x, y1, i1, g1, mode, check_bytes=(call == 0))
