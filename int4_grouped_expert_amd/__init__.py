"""Python binding of libcoli.so: the routed-expert MoE layer with int4-g64 planar
experts on one MI355X (gfx950).

Argument marshalling only.  Every step of the layer runs in the library's HIP
kernels; this module turns torch tensors into device pointers and sizes, passes
the current HIP stream, and raises on a non-zero status.  There is no fallback:
if ``libcoli.so`` is missing, importing this package fails.

The functions carry the C names (see ``include/coli.h`` for the contracts and the
citations of the passages each operation follows).
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libcoli.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")

# One HIP runtime per process.  A PyTorch wheel carries its own HIP and HSA
# runtimes and loads them into the global symbol scope; libcoli.so is linked
# against the system ROCm HIP runtime.  Loaded after torch, that runtime binds
# to torch's HSA runtime (the one that owns the device in this process);
# loaded first, it would bring up a second HSA runtime, which then finds no
# device once torch has opened it.  So torch, when installed, is imported first.
try:
    import torch as _torch  # noqa: F401
except ImportError:  # pure C-ABI use without PyTorch
    _torch = None

lib = ctypes.CDLL(_LIB_PATH)

COLI_OK, COLI_EINVAL, COLI_ESHAPE, COLI_EALIGN = 0, -1, -2, -3
COLI_EDTYPE, COLI_EWORKSPACE, COLI_EDEVICE, COLI_ESCRATCH = -4, -5, -6, -7
COLI_EUSAGE, COLI_EIO, COLI_EFORMAT = -8, -9, -10
COLI_USAGE_VERSION = 1
COLI_NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
COLI_F32, COLI_BF16 = 0, 1
COLI_DECODE, COLI_PREFILL = 0, 1
COLI_SCORE_SOFTMAX, COLI_SCORE_SIGMOID = 0, 1
COLI_STATUS_NONFINITE, COLI_STATUS_RANGE, COLI_STATUS_UNFINISHED = 1, 2, 4
COLI_STATUS_NOT_RESIDENT = 8
COLI_MAX_EXPERTS = 1024
COLI_MAX_DIM = 65536
COLI_MAX_TOKENS = 65536
COLI_MAX_DECODE_T = 256
(COLI_FMT_F32, COLI_FMT_INT8_ROW, COLI_FMT_INT4_ROW, COLI_FMT_INT2_ROW, COLI_FMT_INT4_G64,
 COLI_FMT_INT3_G64, COLI_FMT_E8_IQ3, COLI_FMT_MXFP4, COLI_FMT_FP8_E4M3_B128) = range(9)
COLI_FMT_MAX_ROWS = 1048576
COLI_MATVEC_MAX_T = 8

EXPORTS = [
    "coli_strerror", "coli_int4_g64_packed_bytes", "coli_int4_g64_scale_count",
    "coli_quant_int4_g64", "coli_router_topk", "coli_router_topk_scored",
    "coli_expert_permute_workspace_bytes", "coli_expert_permute", "coli_expert_blob_bytes",
    "coli_expert_views", "coli_expert_finish", "coli_quant_expert", "coli_moe_workspace_bytes",
    "coli_moe_forward", "coli_moe_forward_timed", "coli_moe_forward_noalloc",
    "coli_usage_count", "coli_usage_engine_hash", "coli_usage_save", "coli_usage_load",
    "coli_rmsnorm_f32", "coli_moe_route", "coli_moe_experts", "coli_tier_should_promote",
    "coli_tier_lfru_score", "coli_cache_init", "coli_cache_decay", "coli_cache_admit",
    "coli_cache_repin", "coli_cache_stage", "coli_cache_slot_map", "coli_fmt_bytes",
    "coli_resolve_fmt", "coli_quant_fmt", "coli_matvec_fmt", "coli_fmt_blob_bytes",
    "coli_quant_expert_fmt", "coli_moe_fmt_workspace_bytes", "coli_moe_forward_fmt",
    "coli_quant_int4_g64_many",
]

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class coli_q4(ctypes.Structure):
    _fields_ = [("q", _p), ("s", _p)]


class coli_moe_layer(ctypes.Structure):
    _fields_ = [("H", _i), ("I", _i), ("E", _i), ("K", _i), ("w_router", _p),
                ("router_dtype", _i), ("router_bias", _p), ("experts", _p), ("shared", _p),
                ("scoring", _i), ("slot_map", _p), ("usage", _p)]


class coli_cache(ctypes.Structure):
    _fields_ = [("E", _i), ("S", _i), ("clock", ctypes.c_uint32), ("heat", _p), ("last", _p),
                ("slot_of", _p), ("expert_of", _p)]


def _proto(name, res, args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = args
    return f


_proto("coli_strerror", ctypes.c_char_p, [_i])
_proto("coli_int4_g64_packed_bytes", _sz, [_i64, _i64])
_proto("coli_int4_g64_scale_count", _sz, [_i64, _i64])
_proto("coli_quant_int4_g64", _i, [_p, _i64, _i64, _p, _p, _p, _p])
_proto("coli_quant_int4_g64_many", _i, [_p, _p, _p, _i, _i64, _i64, _p, _p])
_proto("coli_router_topk", _i, [_p, _i, _i, _i, _p, _i, _i, _p, _i, _p, _p, _p, _p])
_proto("coli_router_topk_scored", _i, [_p, _i, _i, _i, _p, _i, _i, _p, _i, _i, _p, _p, _p, _p])
_proto("coli_expert_permute_workspace_bytes", _sz, [_i, _i, _i])
_proto("coli_expert_permute", _i, [_p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p])
_proto("coli_expert_blob_bytes", _sz, [_i, _i])
_proto("coli_expert_views", _i, [_p, _i, _i, ctypes.POINTER(coli_q4), ctypes.POINTER(coli_q4),
                                 ctypes.POINTER(coli_q4)])
_proto("coli_expert_finish", _i, [_p, _i, _i, _p])
_proto("coli_quant_expert", _i, [_p, _i, _i, _p, _p, _p, _p, _p])
_proto("coli_moe_workspace_bytes", _sz, [ctypes.POINTER(coli_moe_layer), _i, _i])
_proto("coli_moe_forward", _i, [ctypes.POINTER(coli_moe_layer), _i, _p, _i, _p, _p, _p, _p, _p,
                                _sz, _p])
_proto("coli_moe_forward_timed", _i, [ctypes.POINTER(coli_moe_layer), _i, _p, _i, _p, _p, _p,
                                      _p, _p, _sz, _p, ctypes.POINTER(_p), _i])
_proto("coli_moe_forward_noalloc", _i, [ctypes.POINTER(coli_moe_layer), _i, _p, _i, _p, _p, _p,
                                        _p, _p])
_proto("coli_rmsnorm_f32", _i, [_p, _p, _i, _i, ctypes.c_float, _p])
_proto("coli_moe_route", _i, [ctypes.POINTER(coli_moe_layer), _i, _p, _i, _p, _p, _p, _p, _p,
                              _sz, _p])
_proto("coli_moe_experts", _i, [ctypes.POINTER(coli_moe_layer), _i, _p, _i, _p, _p, _p, _p, _p,
                                _sz, _p])
_proto("coli_tier_should_promote", _i, [ctypes.c_uint32, ctypes.c_uint32])
_proto("coli_tier_lfru_score", ctypes.c_uint64, [ctypes.c_uint32, ctypes.c_uint32,
                                                 ctypes.c_uint32])
_proto("coli_cache_init", _i, [ctypes.POINTER(coli_cache)])
_proto("coli_cache_decay", _i, [ctypes.POINTER(coli_cache)])
_proto("coli_cache_admit", _i, [ctypes.POINTER(coli_cache), _p, _i, _p, _p,
                                ctypes.POINTER(_i)])
_proto("coli_cache_repin", _i, [ctypes.POINTER(coli_cache), _i, _p, _p, _p, ctypes.POINTER(_i)])
_proto("coli_cache_stage", _i, [_p, _p, _sz, _p, _p, _i, _p])
_proto("coli_cache_slot_map", _i, [ctypes.POINTER(coli_cache), _p, _p])
_proto("coli_fmt_bytes", _i, [_i, _i64, _i64, ctypes.POINTER(ctypes.c_uint64),
                              ctypes.POINTER(ctypes.c_uint64)])
_proto("coli_resolve_fmt", _i, [_i64, _i64, ctypes.c_uint64, ctypes.c_uint64,
                                ctypes.POINTER(ctypes.c_uint32)])
_proto("coli_quant_fmt", _i, [_i, _p, _i64, _i64, _p, _p, _p, _p])
_proto("coli_matvec_fmt", _i, [_i, _p, _p, _i64, _i64, _p, _i, _p, _p])
_proto("coli_fmt_blob_bytes", _sz, [_i, _i, _i])
_proto("coli_quant_expert_fmt", _i, [_i, _p, _i, _i, _p, _p, _p, _p, _p])
_proto("coli_moe_fmt_workspace_bytes", _sz, [ctypes.POINTER(coli_moe_layer), _i, _i])
_proto("coli_moe_forward_fmt", _i, [ctypes.POINTER(coli_moe_layer), _i, _p, _i, _p, _p, _p, _p,
                                    _p, _sz, _p])
_proto("coli_usage_count", _i, [_p, _i, _i, _i, _i, _i, _p, _p])
_proto("coli_usage_engine_hash", ctypes.c_uint32, [ctypes.c_char_p])
_proto("coli_usage_save", _i, [ctypes.c_char_p, _p, _i, _i, ctypes.c_uint32, ctypes.c_double, _p])
_proto("coli_usage_load", _i, [ctypes.c_char_p, _p, _i, _i, ctypes.c_uint32, _i, _p,
                               ctypes.POINTER(ctypes.c_uint64)])


class ColiError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {lib.coli_strerror(status).decode()} (status {status})")
        self.status = status


def _check(status: int, where: str) -> int:
    if status != COLI_OK:
        raise ColiError(status, where)
    return status


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return COLI_F32
    if t.dtype == torch.bfloat16:
        return COLI_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------- format helpers

def coli_int4_g64_packed_bytes(rows: int, cols: int) -> int:
    return int(lib.coli_int4_g64_packed_bytes(rows, cols))


def coli_int4_g64_scale_count(rows: int, cols: int) -> int:
    return int(lib.coli_int4_g64_scale_count(rows, cols))


def coli_expert_blob_bytes(H: int, I: int) -> int:
    return int(lib.coli_expert_blob_bytes(H, I))


def coli_expert_views(blob_ptr: int, H: int, I: int):
    """Device addresses of ((gate.q, gate.s), (up.q, up.s), (down.q, down.s))."""
    g, u, d = coli_q4(), coli_q4(), coli_q4()
    _check(lib.coli_expert_views(ctypes.c_void_p(blob_ptr), H, I, ctypes.byref(g),
                                 ctypes.byref(u), ctypes.byref(d)), "coli_expert_views")
    return (g.q, g.s), (u.q, u.s), (d.q, d.s)


# ---------------------------------------------------------------- entry points

def coli_quant_int4_g64(w, packed, scales, status=None, stream=None):
    """w fp32 [rows, cols] (device) -> packed u8 [rows, G*32], scales f32 [rows, G]."""
    rows, cols = w.shape
    return _check(lib.coli_quant_int4_g64(_ptr(w), rows, cols, _ptr(packed), _ptr(scales),
                                          _ptr(status), _stream(stream)), "coli_quant_int4_g64")


def coli_quant_int4_g64_many(w_ptrs, packed_ptrs, scale_ptrs, n: int, rows: int, cols: int,
                             status=None, stream=None):
    """n matrices of one shape in one launch: the three pointer arguments are int64
    device tensors [n] holding the matrices' device addresses."""
    return _check(lib.coli_quant_int4_g64_many(_ptr(w_ptrs), _ptr(packed_ptrs),
                                               _ptr(scale_ptrs), n, rows, cols, _ptr(status),
                                               _stream(stream)), "coli_quant_int4_g64_many")


def coli_router_topk(x, w_router, bias, K, topk_idx, topk_gate, logits=None, stream=None,
                     scoring=COLI_SCORE_SOFTMAX):
    """logits may be None (then kept on chip).  scoring: COLI_SCORE_SOFTMAX (the C
    coli_router_topk) or COLI_SCORE_SIGMOID (coli_router_topk_scored)."""
    T, H = x.shape
    E = w_router.shape[0]
    if scoring == COLI_SCORE_SOFTMAX:
        return _check(lib.coli_router_topk(_ptr(x), _dtype(x), T, H, _ptr(w_router),
                                           _dtype(w_router), E, _ptr(bias), K, _ptr(topk_idx),
                                           _ptr(topk_gate), _ptr(logits), _stream(stream)),
                      "coli_router_topk")
    return _check(lib.coli_router_topk_scored(_ptr(x), _dtype(x), T, H, _ptr(w_router),
                                              _dtype(w_router), E, _ptr(bias), K, scoring,
                                              _ptr(topk_idx), _ptr(topk_gate), _ptr(logits),
                                              _stream(stream)), "coli_router_topk_scored")


def coli_expert_permute_workspace_bytes(T: int, K: int, E: int) -> int:
    return int(lib.coli_expert_permute_workspace_bytes(T, K, E))


def coli_expert_permute(topk_idx, E, counts, offsets, perm, unique, n_unique, workspace=None,
                        stream=None):
    T, K = topk_idx.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return _check(lib.coli_expert_permute(_ptr(topk_idx), T, K, E, _ptr(counts), _ptr(offsets),
                                          _ptr(perm), _ptr(unique), _ptr(n_unique),
                                          _ptr(workspace), nbytes, _stream(stream)),
                  "coli_expert_permute")


class MoELayer:
    """A layer's device tensors and the C struct describing them.

    experts: uint8 tensor of E * coli_expert_blob_bytes(H, I) bytes (256-B aligned),
    shared:  uint8 tensor of one blob; w_router: [E, H] fp32 or bf16; bias: [E] fp32 or None;
    scoring: COLI_SCORE_SOFTMAX or COLI_SCORE_SIGMOID; slot_map: None, or an int32 device
    tensor [E] mapping each expert to its blob in `experts` (then the cache slots; -1:
    not resident); usage: None, or an int64 device tensor [E] (uint64 counters) that
    every forward adds its routing decisions to.
    """

    def __init__(self, H, I, E, K, w_router, experts, shared, bias=None,
                 scoring=COLI_SCORE_SOFTMAX, slot_map=None, usage=None):
        self.H, self.I, self.E, self.K = H, I, E, K
        self.w_router, self.experts, self.shared, self.bias = w_router, experts, shared, bias
        self.scoring, self.slot_map, self.usage = scoring, slot_map, usage
        self.c = coli_moe_layer(H, I, E, K, w_router.data_ptr(), _dtype(w_router),
                                None if bias is None else bias.data_ptr(), experts.data_ptr(),
                                shared.data_ptr(), scoring,
                                None if slot_map is None else slot_map.data_ptr(),
                                None if usage is None else usage.data_ptr())

    def workspace_bytes(self, T: int, mode: int) -> int:
        return int(lib.coli_moe_workspace_bytes(ctypes.byref(self.c), T, mode))


def coli_moe_workspace_bytes(layer: MoELayer, T: int, mode: int) -> int:
    return layer.workspace_bytes(T, mode)


def coli_moe_forward(layer: MoELayer, mode: int, x, y, workspace, topk_idx=None,
                     topk_gate=None, stream=None, status=None):
    """status: optional int32 device tensor; COLI_STATUS_* bits are OR-ed into it."""
    T = x.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    return _check(lib.coli_moe_forward(ctypes.byref(layer.c), mode, _ptr(x), T, _ptr(y),
                                       _ptr(topk_idx), _ptr(topk_gate), _ptr(status),
                                       _ptr(workspace), nbytes, _stream(stream)),
                  "coli_moe_forward")


def coli_moe_forward_timed(layer: MoELayer, mode: int, x, y, workspace, events, topk_idx=None,
                           topk_gate=None, stream=None, status=None):
    """events: torch.cuda.Event objects (timing enabled): a (start, stop) pair per stage,
    6 (decode) or 10 (prefill)."""
    T = x.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    arr = (_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    return _check(lib.coli_moe_forward_timed(ctypes.byref(layer.c), mode, _ptr(x), T, _ptr(y),
                                             _ptr(topk_idx), _ptr(topk_gate), _ptr(status),
                                             _ptr(workspace), nbytes, _stream(stream), arr,
                                             len(events)),
                  "coli_moe_forward_timed")


def coli_moe_forward_noalloc(layer: MoELayer, mode: int, x, y, topk_idx=None, topk_gate=None,
                             stream=None, status=None):
    """coli_moe_forward with the library's static scratch as workspace (no allocation)."""
    T = x.shape[0]
    return _check(lib.coli_moe_forward_noalloc(ctypes.byref(layer.c), mode, _ptr(x), T, _ptr(y),
                                               _ptr(topk_idx), _ptr(topk_gate), _ptr(status),
                                               _stream(stream)), "coli_moe_forward_noalloc")


def coli_moe_route(layer: MoELayer, mode: int, x, workspace, topk_idx=None, topk_gate=None,
                   unique=None, n_unique=None, stream=None):
    """First half of coli_moe_forward: the routing, left in `workspace`; unique / n_unique
    (int32 device [E] / [1], optional) receive the batch's experts in ascending order."""
    T = x.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    return _check(lib.coli_moe_route(ctypes.byref(layer.c), mode, _ptr(x), T, _ptr(topk_idx),
                                     _ptr(topk_gate), _ptr(unique), _ptr(n_unique),
                                     _ptr(workspace), nbytes, _stream(stream)), "coli_moe_route")


def coli_moe_experts(layer: MoELayer, mode: int, x, y, workspace, topk_idx=None,
                     topk_gate=None, stream=None, status=None):
    """Second half: the expert FFNs and the combine from the routing in `workspace`."""
    T = x.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    return _check(lib.coli_moe_experts(ctypes.byref(layer.c), mode, _ptr(x), T, _ptr(y),
                                       _ptr(topk_idx), _ptr(topk_gate), _ptr(status),
                                       _ptr(workspace), nbytes, _stream(stream)),
                  "coli_moe_experts")


def coli_rmsnorm_f32(x, y, eps=1e-6, stream=None):
    T, H = x.shape
    return _check(lib.coli_rmsnorm_f32(_ptr(x), _ptr(y), T, H, ctypes.c_float(eps),
                                       _stream(stream)), "coli_rmsnorm_f32")


# ---------------------------------------------------------------- routing history

def coli_usage_count(topk_idx, n_experts: int, layer: int, counts, stream=None):
    """counts: uint64-sized device tensor [n_layers, n_experts] (torch.int64)."""
    T, K = topk_idx.shape
    return _check(lib.coli_usage_count(_ptr(topk_idx), T, K, n_experts, layer, counts.shape[0],
                                       _ptr(counts), _stream(stream)), "coli_usage_count")


def coli_usage_engine_hash(name: str) -> int:
    return int(lib.coli_usage_engine_hash(name.encode()))


def coli_usage_save(path: str, counts, engine_hash: int, decay: float = 1.0, dropped=None):
    """counts: host numpy uint64 [n_layers, n_experts]; dropped: host uint8 [n_layers]."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    d = None if dropped is None else np.ascontiguousarray(dropped, dtype=np.uint8)
    return _check(lib.coli_usage_save(path.encode(), c.ctypes.data_as(_p), c.shape[0], c.shape[1],
                                      engine_hash, decay,
                                      None if d is None else d.ctypes.data_as(_p)),
                  "coli_usage_save")


def coli_usage_load(path: str, n_layers: int, n_experts: int, engine_hash: int, trusted=False,
                    dropped=None):
    """-> (counts numpy uint64 [n_layers, n_experts], accepted_total); raises ColiError."""
    import numpy as np
    c = np.zeros((n_layers, n_experts), dtype=np.uint64)
    d = None if dropped is None else np.ascontiguousarray(dropped, dtype=np.uint8)
    tot = ctypes.c_uint64(0)
    _check(lib.coli_usage_load(path.encode(), c.ctypes.data_as(_p), n_layers, n_experts,
                               engine_hash, int(bool(trusted)),
                               None if d is None else d.ctypes.data_as(_p), ctypes.byref(tot)),
           "coli_usage_load")
    return c, int(tot.value)


# ---------------------------------------------------------------- expert placement

def coli_tier_should_promote(hot: int, cold: int) -> bool:
    return bool(lib.coli_tier_should_promote(hot, cold))


def coli_tier_lfru_score(heat: int, last: int, clock: int) -> int:
    return int(lib.coli_tier_lfru_score(heat, last, clock))


class Cache:
    """The C coli_cache over numpy arrays it owns (E experts, S slots)."""

    def __init__(self, E: int, S: int):
        import numpy as np
        self.heat = np.zeros(E, dtype=np.uint32)
        self.last = np.zeros(E, dtype=np.uint32)
        self.slot_of = np.full(E, -1, dtype=np.int32)
        self.expert_of = np.full(max(S, 0), -1, dtype=np.int32)
        self.c = coli_cache(E, S, 0, self.heat.ctypes.data, self.last.ctypes.data,
                            self.slot_of.ctypes.data, self.expert_of.ctypes.data)
        self._buf = [np.zeros(max(S, 1), dtype=np.int32) for _ in range(3)]
        _check(lib.coli_cache_init(ctypes.byref(self.c)), "coli_cache_init")

    @property
    def clock(self) -> int:
        return int(self.c.clock)

    def decay(self):
        _check(lib.coli_cache_decay(ctypes.byref(self.c)), "coli_cache_decay")

    def admit(self, needed) -> list:
        """-> [(expert, slot)] loads (coli_cache_admit)."""
        import numpy as np
        nd = np.ascontiguousarray(needed, dtype=np.int32)
        le, ls = self._buf[0], self._buf[1]
        n = _i(0)
        _check(lib.coli_cache_admit(ctypes.byref(self.c), nd.ctypes.data if nd.size else None,
                                    int(nd.size), le.ctypes.data, ls.ctypes.data,
                                    ctypes.byref(n)), "coli_cache_admit")
        return [(int(le[i]), int(ls[i])) for i in range(n.value)]

    def repin(self, max_swaps: int = 4) -> list:
        """-> [(admitted expert, slot, evicted expert)] (coli_cache_repin)."""
        import numpy as np
        bufs = [np.zeros(max(max_swaps, 1), dtype=np.int32) for _ in range(3)]
        n = _i(0)
        _check(lib.coli_cache_repin(ctypes.byref(self.c), max_swaps, bufs[0].ctypes.data,
                                    bufs[1].ctypes.data, bufs[2].ctypes.data, ctypes.byref(n)),
               "coli_cache_repin")
        return [(int(bufs[0][i]), int(bufs[1][i]), int(bufs[2][i])) for i in range(n.value)]

    def slot_map(self, slot_map, stream=None):
        """Upload slot_of to an int32 device tensor [E] (coli_cache_slot_map)."""
        _check(lib.coli_cache_slot_map(ctypes.byref(self.c), _ptr(slot_map), _stream(stream)),
               "coli_cache_slot_map")


def coli_cache_stage(host_blobs, slots, blob_bytes: int, loads, stream=None):
    """Copy blobs of pinned host uint8 tensor host_blobs to device slots: loads =
    [(expert, slot), ...] (coli_cache_stage)."""
    import numpy as np
    le = np.ascontiguousarray([e for e, _ in loads] or [0], dtype=np.int32)
    ls = np.ascontiguousarray([s for _, s in loads] or [0], dtype=np.int32)
    return _check(lib.coli_cache_stage(_ptr(host_blobs), _ptr(slots), blob_bytes,
                                       le.ctypes.data, ls.ctypes.data, len(loads),
                                       _stream(stream)), "coli_cache_stage")


# ---------------------------------------------------------------- sibling formats

def coli_fmt_bytes(fmt: int, O: int, I: int):
    """-> (weight bytes, scale bytes) of an [O, I] tensor in `fmt`."""
    w, sc = ctypes.c_uint64(0), ctypes.c_uint64(0)
    _check(lib.coli_fmt_bytes(fmt, O, I, ctypes.byref(w), ctypes.byref(sc)), "coli_fmt_bytes")
    return int(w.value), int(sc.value)


def coli_resolve_fmt(O: int, I: int, weight_bytes: int, scale_bytes: int):
    """-> (fmt or None, sorted list of the matching ordinals)."""
    m = ctypes.c_uint32(0)
    r = lib.coli_resolve_fmt(O, I, weight_bytes, scale_bytes, ctypes.byref(m))
    if r not in (COLI_EFORMAT,) and r < 0:
        _check(r, "coli_resolve_fmt")
    cands = [f for f in range(9) if (m.value >> f) & 1]
    return (r if r >= 0 else None), cands


def coli_quant_fmt(fmt: int, w, packed, scales, status=None, stream=None):
    """Quantise fp32 w [O, I] (device) into packed / scales (device uint8 tensors)."""
    O, I = w.shape
    return _check(lib.coli_quant_fmt(fmt, _ptr(w), O, I, _ptr(packed), _ptr(scales),
                                     _ptr(status), _stream(stream)), "coli_quant_fmt")


def coli_matvec_fmt(fmt: int, packed, scales, O: int, I: int, x, y, stream=None):
    """y [T, O] = x [T, I] W^T with W the dequantised [O, I] tensor (device)."""
    T = x.shape[0]
    return _check(lib.coli_matvec_fmt(fmt, _ptr(packed), _ptr(scales), O, I, _ptr(x), T,
                                      _ptr(y), _stream(stream)), "coli_matvec_fmt")


def coli_fmt_blob_bytes(fmt: int, H: int, I: int) -> int:
    return int(lib.coli_fmt_blob_bytes(fmt, H, I))


def coli_quant_expert_fmt(fmt: int, blob_ptr: int, H: int, I: int, wg, wu, wd, status=None,
                          stream=None):
    """Quantise fp32 gate [I,H], up [I,H], down [H,I] (device) into a blob of fmt."""
    return _check(lib.coli_quant_expert_fmt(fmt, ctypes.c_void_p(blob_ptr), H, I, _ptr(wg),
                                            _ptr(wu), _ptr(wd), _ptr(status), _stream(stream)),
                  "coli_quant_expert_fmt")


def coli_moe_fmt_workspace_bytes(layer: "MoELayer", fmt: int, T: int) -> int:
    return int(lib.coli_moe_fmt_workspace_bytes(ctypes.byref(layer.c), fmt, T))


def coli_moe_forward_fmt(layer: "MoELayer", fmt: int, x, y, workspace, topk_idx=None,
                         topk_gate=None, stream=None, status=None):
    """The decode layer with experts in fmt (layer.experts: E blobs of coli_fmt_blob_bytes)."""
    T = x.shape[0]
    nbytes = workspace.numel() * workspace.element_size()
    return _check(lib.coli_moe_forward_fmt(ctypes.byref(layer.c), fmt, _ptr(x), T, _ptr(y),
                                           _ptr(topk_idx), _ptr(topk_gate), _ptr(status),
                                           _ptr(workspace), nbytes, _stream(stream)),
                  "coli_moe_forward_fmt")


# ---------------------------------------------------------------- layer assembly

def coli_expert_finish(blob_ptr: int, H: int, I: int, stream=None):
    """The blob's group-major and 8-row blocked scale copies from its row-major scales."""
    return _check(lib.coli_expert_finish(ctypes.c_void_p(blob_ptr), H, I, _stream(stream)),
                  "coli_expert_finish")


def coli_quant_expert(blob_ptr: int, H: int, I: int, wg, wu, wd, status=None, stream=None,
                      finish=True):
    """Quantise fp32 gate [I,H], up [I,H], down [H,I] (device) into the blob at blob_ptr and
    finish it (the C coli_quant_expert).  finish=False runs only the three
    coli_quant_int4_g64 calls into the coli_expert_views sections (no derived scale
    copies, no finish tag)."""
    st = _stream(stream)
    if finish:
        return _check(lib.coli_quant_expert(ctypes.c_void_p(blob_ptr), H, I, _ptr(wg), _ptr(wu),
                                            _ptr(wd), _ptr(status), st), "coli_quant_expert")
    views = coli_expert_views(blob_ptr, H, I)
    for (qp, sp), w in zip(views, (wg, wu, wd)):
        rows, cols = w.shape
        _check(lib.coli_quant_int4_g64(_ptr(w), rows, cols, ctypes.c_void_p(qp),
                                       ctypes.c_void_p(sp), _ptr(status), st),
               "coli_quant_int4_g64")
    return COLI_OK


def alloc_layer_blobs(H: int, I: int, E: int, device="cuda"):
    """Device storage for E routed expert blobs and one shared blob (uint8)."""
    import torch
    nb = coli_expert_blob_bytes(H, I)
    experts = torch.empty(E * nb, dtype=torch.uint8, device=device)
    shared = torch.empty(nb, dtype=torch.uint8, device=device)
    assert experts.data_ptr() % 256 == 0 and shared.data_ptr() % 256 == 0
    return experts, shared, nb
