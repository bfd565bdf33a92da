"""GPU checks of the two-phase forward and the HBM expert cache (page "Colibrì 深度解析",
section 三: experts live in a slow tier and are brought into a small fast tier on
demand, placed by the heat / LFRU rules; page "为什么Colibrì越用越快", section 实时重固定
REPIN).

* coli_moe_route + coli_moe_experts give bit-identical results to coli_moe_forward on
  the single-token, batch-decode and prefill paths, and the union they report is the
  set of routed ids;
* a layer whose experts live in S < E cache slots (host blobs in pinned memory, the
  loads planned by coli_cache_admit / coli_cache_repin, staged by coli_cache_stage,
  mapped by coli_cache_slot_map) gives bit-identical results to the resident layer
  over a sequence of batches that evicts and re-admits experts, and the oracle
  agrees with it;
* an expert routed while unmapped poisons only its tokens (NaN) and raises
  COLI_STATUS_NOT_RESIDENT: a cache miss never reads another expert's weights.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests.harness import DeviceLayer, Timer, host_array, log, margin_tokens
from tests.test_gpu_forward import DECODE, PREFILL, oracle_check

pytestmark = pytest.mark.gpu

_layers = {}


def layer(cfg_id):
    if cfg_id not in _layers:
        with Timer(f"build layer cfg {cfg_id}"):
            _layers[cfg_id] = DeviceLayer(cfg_id)
    return _layers[cfg_id]


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality (NaN payloads included)."""
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def two_phase(coli, L, mode, x):
    """coli_moe_route on the MoELayer L: (workspace, ids, gates, union, union size)."""
    T = x.shape[0]
    ws = torch.empty(max(L.workspace_bytes(T, mode), 256), dtype=torch.uint8, device="cuda")
    idx = torch.empty((T, L.K), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, L.K), dtype=torch.float32, device="cuda")
    uniq = torch.empty(L.E, dtype=torch.int32, device="cuda")
    nu = torch.empty(1, dtype=torch.int32, device="cuda")
    coli.coli_moe_route(L, mode, x, ws, idx, gates, uniq, nu)
    return ws, idx, gates, uniq, nu


CASES = [(107, DECODE, 1), (114, DECODE, 1), (101, DECODE, 40), (115, DECODE, 40),
         (100, PREFILL, 333), (117, PREFILL, 200)]


@pytest.mark.parametrize("cfg_id,mode,T", CASES)
def test_two_phase_matches_forward(cfg_id, mode, T):
    import int4_grouped_expert_amd as coli
    log(f"two-phase cfg {cfg_id} mode {mode} T {T}")
    dl = layer(cfg_id)
    x = W.tokens(cfg_id, T, "cuda", draw=3)
    y_ref, idx_ref, g_ref = dl.forward(x, mode)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws, idx, gates, uniq, nu = two_phase(coli, dl.layer_c, mode, x)
    torch.cuda.synchronize()
    n = int(nu.item())
    want = sorted(set(idx_ref.cpu().numpy().reshape(-1).tolist()))
    assert uniq.cpu().numpy()[:n].tolist() == want
    assert (uniq.cpu().numpy()[n:] == -1).all()
    y = torch.empty_like(y_ref)
    coli.coli_moe_experts(dl.layer_c, mode, x, y, ws, idx, gates, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(idx, idx_ref) and same(gates, g_ref)
    assert same(y, y_ref), "two-phase forward differs from coli_moe_forward"


class CachedLayer:
    """The layer of `dl` with its routed experts in S HBM slots over pinned host blobs."""

    def __init__(self, coli, dl, S):
        self.coli, self.dl, self.S = coli, dl, S
        self.blob = dl.blob
        self.host = torch.empty(dl.E * dl.blob, dtype=torch.uint8, pin_memory=True)
        self.host.copy_(dl.experts)
        self.slots = torch.empty(S * dl.blob, dtype=torch.uint8, device="cuda")
        self.slots.fill_(0)  # no finish tag: an unstaged slot reads as unfinished
        self.slot_map = torch.full((dl.E,), -1, dtype=torch.int32, device="cuda")
        self.cache = coli.Cache(dl.E, S)
        self.layer_c = coli.MoELayer(dl.H, dl.I, dl.E, dl.K, dl.w_router, self.slots, dl.shared,
                                     dl.bias, dl.scoring, slot_map=self.slot_map)
        self.loads = 0

    def forward(self, x, mode, status, repin=False):
        coli = self.coli
        ws, idx, gates, uniq, nu = two_phase(coli, self.layer_c, mode, x)
        torch.cuda.synchronize()
        needed = uniq.cpu().numpy()[:int(nu.item())]
        loads = self.cache.admit(needed)
        if repin:
            loads += [(h, s) for h, s, _ in self.cache.repin(4)]
        self.loads += len(loads)
        coli.coli_cache_stage(self.host, self.slots, self.blob, loads)
        self.cache.slot_map(self.slot_map)
        y = torch.empty((x.shape[0], self.dl.H),
                        dtype=torch.float32 if mode == DECODE else torch.bfloat16, device="cuda")
        coli.coli_moe_experts(self.layer_c, mode, x, y, ws, idx, gates, status=status)
        return y, idx, gates


@pytest.mark.parametrize("cfg_id,mode,T,S", [(107, DECODE, 1, 6), (101, DECODE, 2, 14),
                                             (100, PREFILL, 3, 18), (115, DECODE, 2, 13)])
def test_cache_matches_resident(cfg_id, mode, T, S):
    import int4_grouped_expert_amd as coli
    log(f"cache cfg {cfg_id} mode {mode} T {T} S {S}")
    dl = layer(cfg_id)
    cl = CachedLayer(coli, dl, S)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    nb = 16
    for b in range(nb):
        # the last batch: tokens clear of top-K near-ties, for the oracle check
        x = (W.tokens(cfg_id, T, "cuda", draw=100 + b) if b < nb - 1 else
             margin_tokens(cfg_id, T, host_array(dl.w_router), dl.bias_np, dl.K))
        y_ref, idx_ref, _ = dl.forward(x, mode)
        y, idx, gates = cl.forward(x, mode, st, repin=(b % 4 == 3))
        torch.cuda.synchronize()
        assert int(st.item()) == 0, f"batch {b}: status {int(st.item())}"
        assert torch.equal(idx, idx_ref)
        assert same(y, y_ref), f"batch {b}: cached forward differs from the resident one"
        # the map and the slots agree with the cache's plan
        sm = cl.slot_map.cpu().numpy()
        assert sm.tolist() == cl.cache.slot_of.tolist()
        if cl.cache.expert_of.min() >= 0 and b == nb - 1:
            for s, e in enumerate(cl.cache.expert_of.tolist()):
                assert torch.equal(cl.slots[s * cl.blob:(s + 1) * cl.blob],
                                   dl.experts[e * cl.blob:(e + 1) * cl.blob])
    log(f"[cache] {nb} batches, {cl.loads} blob loads into {S} slots of {dl.E}")
    assert cl.loads > S, "the trace never evicted"
    # the last batch against the oracle, read from the slots
    oracle_check(cfg_id, dl, x, y, idx, gates, mode)


@pytest.mark.parametrize("cfg_id,mode,T", [(107, DECODE, 1), (101, DECODE, 6),
                                           (100, PREFILL, 40)])
def test_unmapped_expert_poisons_its_tokens(cfg_id, mode, T):
    import int4_grouped_expert_amd as coli
    log(f"not resident cfg {cfg_id} mode {mode} T {T}")
    dl = layer(cfg_id)
    x = W.tokens(cfg_id, T, "cuda", draw=7)
    y_ref, idx_ref, _ = dl.forward(x, mode)
    torch.cuda.synchronize()
    ids = idx_ref.cpu().numpy()
    victim = int(ids[0, 0])
    sm = torch.arange(dl.E, dtype=torch.int32, device="cuda")
    sm[victim] = -1
    L = coli.MoELayer(dl.H, dl.I, dl.E, dl.K, dl.w_router, dl.experts, dl.shared, dl.bias,
                      dl.scoring, slot_map=sm)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.empty_like(y_ref)
    ws = torch.empty(max(L.workspace_bytes(T, mode), 256), dtype=torch.uint8, device="cuda")
    coli.coli_moe_forward(L, mode, x, y, ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & coli.COLI_STATUS_NOT_RESIDENT
    hit = (ids == victim).any(axis=1)
    yn = torch.isnan(y.float()).cpu().numpy()
    assert yn[hit].all(), "a token routed to the unmapped expert is not NaN"
    assert not yn[~hit].any()
    keep = torch.from_numpy(np.nonzero(~hit)[0]).to("cuda")
    if keep.numel():
        assert same(y[keep], y_ref[keep])
    # with the identity map the layer is the resident one
    sm[victim] = victim
    st.zero_()
    coli.coli_moe_forward(L, mode, x, y, ws, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and same(y, y_ref)
