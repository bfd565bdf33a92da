"""The oracle: a plain fp64 CPU statement of the routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (the HIP library and its binding) never imports, links or calls it, and
this package imports nothing from the product.

The arithmetic lives in ``coli_oracle.c`` (fp64, ``-ffp-contract=off``); this
module only builds it with gcc and marshals numpy arrays through ctypes.
Every function names the passage it follows in the C source's comments:

* quantiser and planar packer -- page "从源码开始colibri纯C引擎的编译、权重转换
  与.bin直映射实战", section 权重转换;
* router top-K with renormalised gates -- page "Colibrì 深度解析", section 十一,
  and page "colibrì 路由遥测全解析", sections 分离计数与追踪 and 测试与 CI 保障;
  the sigmoid router ("n_group=1 sigmoid + noaux_tc") of the same section 十一;
* batch-union permute -- page "Colibrì 深度解析", section 四;
* expert FFN, combine, RMSNorm -- read as: h = SiLU(gate) * up with
  SiLU(z) = z / (1 + e^-z), y = sum_k g_k * down_k(h_k) + the shared expert's
  down(h) with weight 1 (no routed scaling factor), RMSNorm with unit weight,
  eps 1e-6 and no residual (the pages name these stages without formulas).

Plain-Python modules beside it: ``tier.py`` (expert placement), ``usage.py`` (the
.coli_usage history) and ``formats.py`` (the sibling weight formats of the
registry: byte arithmetic, inference from byte counts, int3-g64, MXFP4 and
fp8-e4m3-b128).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
except the composition of a whole layer's float output, which the pages give
no numbers for ("parity unpinned" beyond its pinned parts and the reductions
to library routines tested there).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coli_oracle.c")
_LIB = os.path.join(_HERE, "libcoli_oracle.so")

F32, BF16, F64 = 0, 1, 2

_lib = None


def build() -> str:
    """Compile the oracle shared object with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        L.orc_groups.restype = i64
        L.orc_groups.argtypes = [i64]
        L.orc_quant_int4_g64.restype = i32
        L.orc_quant_int4_g64.argtypes = [p, i64, i64, p, p]
        L.orc_dequant_int4_g64.restype = None
        L.orc_dequant_int4_g64.argtypes = [p, p, i64, i64, p]
        L.orc_router_logits.restype = None
        L.orc_router_logits.argtypes = [p, i32, i32, i32, p, i32, i32, p, p]
        L.orc_topk.restype = i32
        L.orc_topk.argtypes = [p, i32, i32, i32, p, p]
        L.orc_topk_sigmoid.restype = i32
        L.orc_topk_sigmoid.argtypes = [p, i32, i32, i32, p, p, p]
        L.orc_permute.restype = i32
        L.orc_permute.argtypes = [p, i32, i32, i32, p, p, p, p]
        L.orc_expert_ffn.restype = None
        L.orc_expert_ffn.argtypes = [p, p, p, p, p, p, i32, i32, p, i32, p, p]
        L.orc_moe_forward.restype = i32
        L.orc_moe_forward.argtypes = [p, i32, i32, i32, i32, i32, i32, p, i32, p, i32,
                                      p, p, p, p, p]
        L.orc_rmsnorm.restype = None
        L.orc_rmsnorm.argtypes = [p, i32, i32, ctypes.c_double, p]
        L.orc_threads.restype = i32
        L.orc_threads.argtypes = []
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"oracle takes float32, float64 or bf16-as-uint16, got {a.dtype}")


def groups(cols: int) -> int:
    return int(lib().orc_groups(cols))


def threads() -> int:
    return int(lib().orc_threads())


def quant_int4_g64(w: np.ndarray):
    """fp32 [rows, cols] -> (packed u8 [rows, G*32], scales f32 [rows, G], status)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    G = groups(cols)
    packed = np.empty((rows, G * 32), dtype=np.uint8)
    scales = np.empty((rows, G), dtype=np.float32)
    st = lib().orc_quant_int4_g64(_ptr(w), rows, cols, _ptr(packed), _ptr(scales))
    return packed, scales, int(st)


def dequant_int4_g64(packed: np.ndarray, scales: np.ndarray, cols: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    rows = packed.shape[0]
    out = np.empty((rows, cols), dtype=np.float64)
    lib().orc_dequant_int4_g64(_ptr(packed), _ptr(scales), rows, cols, _ptr(out))
    return out


def router_logits(x: np.ndarray, wr: np.ndarray, bias: np.ndarray | None = None):
    x = np.ascontiguousarray(x)
    wr = np.ascontiguousarray(wr)
    T, H = x.shape
    E, H2 = wr.shape
    assert H == H2
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), dtype=np.float64)
    lib().orc_router_logits(_ptr(x), _dtype_code(x), T, H, _ptr(wr), _dtype_code(wr),
                            E, _ptr(b), _ptr(out))
    return out


def topk(logits: np.ndarray, K: int):
    """-> (idx int32 [T,K] ascending, gates fp64 [T,K], n_fallback_rounds)."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    idx = np.empty((T, K), dtype=np.int32)
    gates = np.empty((T, K), dtype=np.float64)
    fb = lib().orc_topk(_ptr(logits), T, E, K, _ptr(idx), _ptr(gates))
    return idx, gates, int(fb)


def topk_sigmoid(logits: np.ndarray, K: int, bias=None):
    """Sigmoid router on raw logits, bias for the selection only.
    -> (idx int32 [T,K] ascending, gates fp64 [T,K], n_fallback_rounds)."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    T, E = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((T, K), dtype=np.int32)
    gates = np.empty((T, K), dtype=np.float64)
    fb = lib().orc_topk_sigmoid(_ptr(logits), T, E, K, _ptr(b), _ptr(idx), _ptr(gates))
    return idx, gates, int(fb)


SOFTMAX, SIGMOID = 0, 1


def permute(idx: np.ndarray, E: int):
    """-> (counts [E], offsets [E+1], perm [T*K], unique [n])."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, K = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(max(T * K, 1), dtype=np.int32)
    unique = np.empty(max(E, 1), dtype=np.int32)
    n = lib().orc_permute(_ptr(idx), T, K, E, _ptr(counts), _ptr(offsets), _ptr(perm),
                          _ptr(unique))
    return counts, offsets, perm[: T * K].copy(), unique[:n].copy()


class Expert:
    """One quantised expert held by the oracle (its own packed arrays)."""

    def __init__(self, gq, gs, uq, us, dq, ds):
        c = np.ascontiguousarray
        self.gq, self.gs = c(gq, dtype=np.uint8), c(gs, dtype=np.float32)
        self.uq, self.us = c(uq, dtype=np.uint8), c(us, dtype=np.float32)
        self.dq, self.ds = c(dq, dtype=np.uint8), c(ds, dtype=np.float32)

    @classmethod
    def quantise(cls, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> "Expert":
        gq, gs, _ = quant_int4_g64(wg)
        uq, us, _ = quant_int4_g64(wu)
        dq, ds, _ = quant_int4_g64(wd)
        return cls(gq, gs, uq, us, dq, ds)

    def ptrs(self):
        return [_ptr(self.gq), _ptr(self.gs), _ptr(self.uq), _ptr(self.us),
                _ptr(self.dq), _ptr(self.ds)]


class _CExpert(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("gq", "gs", "uq", "us", "dq", "ds")]


def expert_ffn(ex: Expert, x: np.ndarray, H: int, I: int, want_h: bool = False):
    """x fp64 [n, H] -> out fp64 [n, H] (and h fp64 [n, I] if want_h)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    n = x.shape[0]
    out = np.empty((n, H), dtype=np.float64)
    h = np.empty((n, I), dtype=np.float64) if want_h else None
    lib().orc_expert_ffn(*ex.ptrs(), H, I, _ptr(x), n, _ptr(out), _ptr(h))
    return (out, h) if want_h else out


def moe_forward(x: np.ndarray, wr: np.ndarray, bias, experts: list, shared: Expert,
                H: int, I: int, K: int, scoring: int = SOFTMAX):
    """Whole layer.  experts: list of E entries (Expert or None if unused).
    scoring: SOFTMAX (bias added to the logits) or SIGMOID (bias steers the
    selection only).

    -> (y fp64 [T,H], idx int32 [T,K], gates fp64 [T,K]).
    """
    x = np.ascontiguousarray(x)
    wr = np.ascontiguousarray(wr)
    T = x.shape[0]
    E = wr.shape[0]
    arr = (_CExpert * max(E, 1))()
    for e, ex in enumerate(experts):
        if ex is not None:
            arr[e] = _CExpert(*ex.ptrs())
    sh = _CExpert(*shared.ptrs())
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    y = np.empty((T, H), dtype=np.float64)
    idx = np.empty((T, K), dtype=np.int32)
    gates = np.empty((T, K), dtype=np.float64)
    rc = lib().orc_moe_forward(_ptr(x), _dtype_code(x), T, H, I, E, K, _ptr(wr),
                               _dtype_code(wr), _ptr(b), int(scoring),
                               ctypes.cast(arr, ctypes.c_void_p),
                               ctypes.byref(sh), _ptr(y), _ptr(idx), _ptr(gates))
    if rc != 0:
        raise ValueError("oracle: a selected expert was not supplied")
    return y, idx, gates


def rmsnorm(y: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float64)
    T, H = y.shape
    out = np.empty_like(y)
    lib().orc_rmsnorm(_ptr(y), T, H, eps, _ptr(out))
    return out
