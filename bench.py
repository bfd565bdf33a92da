#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Metric: MoE-layer decode tokens/s + HBM GB/s (% of peak); prefill MFMA util.

Workload (the step): one decode forward of the layer H=6144, I=2048, E=256 routed
experts (top-8) + 1 shared expert, int4-g64 planar weights, T=1 fp32 token:
router logits -> top-K + renormalised gates -> gate/up + SiLU*up -> down +
gate-weighted combine + shared expert (three kernels on the int8 matrix cores).  Inputs are resident in HBM
before the timed region.  Steps rotate over 8 byte-identical replicas of the layer
(43.7 GB) and a pool of 64 tokens, so the 256 MB Infinity Cache cannot serve the
~191 MB a token touches.

Printed: one JSON line (rank 0).  Extra fields: per-stage times and the roofline
of the dominant kernel (the single-token gate/up kernel, timed with start/stop
events stamped by its own launch on the library's stream), the T=32 Zipf decode
batch, the T=2048 prefill (MFMA utilisation of the grouped GEMMs), and the fp64
CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 vector, TFLOP/s
METRIC = "MoE-layer decode tokens/s + HBM GB/s (% of peak); prefill MFMA util"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(coli, W, cfg_id, replicas):
    import torch
    c = W.CONFIGS[cfg_id]
    H, I, E, K = c["H"], c["I"], c["E"], c["K"]
    experts, shared, nb = coli.alloc_layer_blobs(H, I, E)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for e in range(E + 1):
        wg, wu, wd = W.expert_weights(cfg_id, e, "cuda")
        ptr = shared.data_ptr() if e == E else experts.data_ptr() + e * nb
        coli.coli_quant_expert(ptr, H, I, wg, wu, wd, status)
        del wg, wu, wd
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    wr = W.router_weights(cfg_id, "cuda").contiguous()
    b = W.router_bias(cfg_id)
    bias = None if b is None else torch.from_numpy(b).cuda()
    layers = [coli.MoELayer(H, I, E, K, wr, experts, shared, bias)]
    for _ in range(replicas - 1):
        layers.append(coli.MoELayer(H, I, E, K, wr.clone(), experts.clone(), shared.clone(),
                                    None if bias is None else bias.clone()))
    torch.cuda.synchronize()
    return layers, nb


class Caller:
    """Pre-marshalled coli_moe_forward(_timed) calls (keeps host overhead small)."""

    def __init__(self, coli, layer, mode, x, y, ws, idx, gates):
        import torch
        self.coli, self.layer, self.mode = coli, layer, mode
        self.args = [ctypes.byref(layer.c), mode, ctypes.c_void_p(x.data_ptr()), x.shape[0],
                     ctypes.c_void_p(y.data_ptr()), ctypes.c_void_p(idx.data_ptr()),
                     ctypes.c_void_p(gates.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()),
                     ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)]

    def __call__(self):
        st = self.coli.lib.coli_moe_forward(*self.args)
        if st:
            raise RuntimeError(f"coli_moe_forward: {st}")

    def timed(self, evarr, n):
        st = self.coli.lib.coli_moe_forward_timed(*self.args, evarr, n)
        if st:
            raise RuntimeError(f"coli_moe_forward_timed: {st}")


def make_events(n):
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()  # torch creates the HIP event on first record
    arr = (ctypes.c_void_p * n)(*[ctypes.c_void_p(e.cuda_event) for e in ev])
    return ev, arr


def run_decode(coli, W, layers, cfg_id, T, steps, warmup, pool_n=64):
    """Time `steps` decode forwards; returns dict with value and per-stage times."""
    import torch
    c = W.CONFIGS[cfg_id]
    H, K = c["H"], c["K"]
    pool = W.token_pool(cfg_id, pool_n * T, "cuda").reshape(pool_n, T, H).contiguous()
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(layers[0].workspace_bytes(T, coli.COLI_DECODE), dtype=torch.uint8,
                     device="cuda")
    R = len(layers)
    callers = [[Caller(coli, layers[r], coli.COLI_DECODE, pool[p], y, ws, idx, gates)
                for p in range(pool_n)] for r in range(R)]

    def call(i):
        callers[i % R][i % pool_n]()

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        call(warmup + i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end)
    # per-stage durations: the library brackets each stage with a (start, stop)
    # event pair on its stream; on the single-token path each stage is one
    # kernel and the pair is stamped by that kernel's launch
    nst = min(steps, 400)
    if nst < steps and steps < 400:
        nst = steps
    evs = [make_events(6) for _ in range(nst)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)  # let the host queue run ahead of the GPU
    for i in range(nst):
        callers[i % R][i % pool_n].timed(evs[i][1], 6)
    torch.cuda.synchronize()
    stage = [0.0, 0.0, 0.0]
    for ev, _ in evs:
        for s_ in range(3):
            stage[s_] += ev[2 * s_].elapsed_time(ev[2 * s_ + 1])
    stage = [s_ / nst for s_ in stage]
    # the distribution of the plain step: blocks of `blk` back-to-back steps with
    # an event between blocks (so the events barely touch the steps they time)
    blk = 10
    nblk = max(20, min(300, steps // blk))
    bev = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
    torch.cuda.synchronize()
    bev[0].record()
    for b in range(nblk):
        for j in range(blk):
            call(b * blk + j)
        bev[b + 1].record()
    torch.cuda.synchronize()
    per_step = [bev[b].elapsed_time(bev[b + 1]) / blk for b in range(nblk)]
    # unique experts of each pool batch (the timed loop cycles the pool): the
    # algorithmic bytes of a step depend on it
    uniq = []
    for p in range(pool_n):
        callers[0][p]()
        uniq.append(int(torch.unique(idx).numel()))
    u_mean = sum(uniq[i % pool_n] for i in range(warmup, warmup + steps)) / steps
    return dict(ms=ms, wall=wall, steps=steps, stage_ms=stage, T=T, u_mean=u_mean,
                step_ms=dist(per_step))


def dist(v):
    """Median, p10 and p90 of a list of times (ms), and how many (here: per-step
    times of blocks of 10 back-to-back steps)."""
    v = sorted(v)
    n = len(v)

    def q(f):
        return v[min(n - 1, int(round(f * (n - 1))))]
    return {"median": round(q(0.5), 5), "p10": round(q(0.1), 5), "p90": round(q(0.9), 5),
            "n": n}


def decode_bytes(c, U, T):
    """Algorithmic HBM bytes of one decode forward: router, unique experts + shared, x, y."""
    H, I, E = c["H"], c["I"], c["E"]
    blob = 3 * (I * (H // 64) * 32 + I * (H // 64) * 4)  # gate+up+down nibbles and scales
    router = E * H * (2 if c["router"] == "bf16" else 4)
    return int(router + (U + 1) * blob + 2 * T * H * 4)


def t32_compute_ceiling(c):
    """The batch's second roofline: its algorithmic multiply-adds (router + K routed +
    the shared expert's three matrices per token) at the fp32 vector peak.  The GEMMs
    run on the fp16 matrix cores (exact u - 8 weights, hi/lo activations), whose
    padded 32-row tiles do more work than this count; HBM is the bound that binds."""
    H, I, E, K, T = c["H"], c["I"], c["E"], c["K"], c["T"]
    fma = T * (H * E + (K + 1) * 3 * H * I)
    return {"fma": fma, "fp32_vector_peak_tflops": FP32_PEAK_TFLOPS,
            "us_at_peak": round(2 * fma / (FP32_PEAK_TFLOPS * 1e12) * 1e6, 1)}


def gateup_bytes(c, U, T):
    H, I = c["H"], c["I"]
    per = 2 * (I * (H // 64) * 32 + I * (H // 64) * 4)
    return (U + 1) * per + T * H * 4 + (T * c["K"] + T) * I * 4


def run_prefill(coli, W, layer, steps=10, warmup=2):
    import torch
    c = W.CONFIGS[3]
    T, H, K = c["T"], c["H"], c["K"]
    x = W.tokens(3, T, "cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(layer.workspace_bytes(T, coli.COLI_PREFILL), dtype=torch.uint8,
                     device="cuda")
    call = Caller(coli, layer, coli.COLI_PREFILL, x, y, ws, idx, gates)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    stage = [0.0] * 5
    for _ in range(steps):
        ev, arr = make_events(10)
        call.timed(arr, 10)
        torch.cuda.synchronize()
        for i in range(5):
            stage[i] += ev[2 * i].elapsed_time(ev[2 * i + 1])
    stage = [s_ / steps for s_ in stage]
    flops_routed = 2.0 * T * K * 3 * H * c["I"]
    flops_shared = 2.0 * T * 3 * H * c["I"]
    gemm_ms = stage[2] + stage[3]
    tflops = (flops_routed + flops_shared) / (gemm_ms * 1e-3) / 1e12
    return dict(ms_per_forward=round(ms, 4), tokens_per_s=round(T / (ms * 1e-3), 1),
                stage_ms=dict(route=round(stage[0], 4), prep=round(stage[1], 4),
                              gateup=round(stage[2], 4), down=round(stage[3], 4),
                              combine=round(stage[4], 4)),
                grouped_gemm_tflops=round(tflops, 1),
                mfma_frac=round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                whole_forward_mfma_frac=round(
                    (flops_routed + flops_shared + 2.0 * T * H * c["E"]) / (ms * 1e-3) / 1e12
                    / MFMA_F16_PEAK_TFLOPS, 4),
                flops=flops_routed + flops_shared, dtype="fp16 MFMA operands (bf16 I/O)")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_layer_experts(W, cfg_id, ids, layer=0):
    """The oracle's own quantisation of the listed experts (and the shared one)."""
    import oracle
    E = W.CONFIGS[cfg_id]["E"]
    experts = [None] * E
    for e in ids:
        experts[e] = oracle.Expert.quantise(
            *(w.cpu().numpy() for w in W.expert_weights(cfg_id, e, "cuda", layer)))
    shared = oracle.Expert.quantise(
        *(w.cpu().numpy() for w in W.expert_weights(cfg_id, E, "cuda", layer)))
    return experts, shared


def cpu_baseline(coli, W, budget_s=6.0, n_tok=6):
    """The oracle (fp64, as committed, OpenMP over the host cores) on bounded samples
    of each workload, its experts quantised by the oracle beforehand (untimed):
      decode T=1   -- n_tok tokens cycled for about budget_s seconds;
      decode T=32  -- one Zipf batch of 32 tokens;
      prefill      -- 64 of the 2048 tokens, scaled x 32 (the oracle's time per token
                      does not depend on the batch);
      stack step   -- layer 0 of the 40-layer stack on its 8 tokens, scaled x 40;
      quantiser    -- 16 of one layer's 256 experts, scaled x 16;
      tiny T=1     -- the tiny layer (all 16 experts), 8 tokens cycled for about 0.5 s.
    The headline fields are the T=1 leg's; `legs` holds every leg."""
    import numpy as np
    import oracle
    import torch
    c = W.CONFIGS[1]
    H, I, E, K = c["H"], c["I"], c["E"], c["K"]

    def bits(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.cpu().numpy()
    wr_h = bits(W.router_weights(1, "cuda"))
    pool = W.token_pool(1, 64, "cuda").cpu().numpy()
    x32 = W.tokens(2, 32, "cuda").cpu().numpy()
    b32 = W.router_bias(2)
    xp = bits(W.tokens(3, 2048, "cuda"))[:64].copy()
    need = set()
    for xs, b in ((pool[:n_tok], None), (x32, b32), (xp, None)):
        idx, _, _ = oracle.topk(oracle.router_logits(xs, wr_h, b), K)
        need |= set(idx.reshape(-1).tolist())
    t_prep = time.perf_counter()
    experts, shared = oracle_layer_experts(W, 1, sorted(need))
    log(f"[bench] cpu baseline: {len(need)} experts quantised by the oracle "
        f"({time.perf_counter() - t_prep:.1f} s, untimed)")
    legs = {}
    done = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) < budget_s:
        k = done % n_tok
        oracle.moe_forward(pool[k:k + 1], wr_h, None, experts, shared, H, I, K)
        done += 1
    el = time.perf_counter() - t0
    legs["decode_t1"] = {"value": round(done / el, 3), "unit": "tokens/s",
                         "sample": f"{done} single-token forwards, {n_tok} tokens cycled, "
                                   f"{el:.1f} s"}
    t0 = time.perf_counter()
    oracle.moe_forward(x32, wr_h, b32, experts, shared, H, I, K)
    el = time.perf_counter() - t0
    legs["decode_t32_zipf"] = {"value": round(32 / el, 3), "unit": "tokens/s",
                               "ms_per_step": round(el * 1e3, 1),
                               "sample": f"one batch of 32 tokens, {el:.1f} s"}
    t0 = time.perf_counter()
    oracle.moe_forward(xp, wr_h, None, experts, shared, H, I, K)
    el = time.perf_counter() - t0
    legs["prefill_t2048"] = {"value": round(64 / el, 3), "unit": "tokens/s",
                             "ms_per_forward": round(el * 1e3 * 2048 / 64, 1),
                             "sample": f"64 of the 2048 tokens in {el:.1f} s, scaled x 32"}
    # stack: layer 0 of the stack workload, its own experts and bias
    cs = W.CONFIGS[4]
    wr4 = bits(W.router_weights(4, "cuda", 0))
    b4 = W.router_bias(4, 0)
    x4 = W.tokens(4, cs["T"], "cuda").cpu().numpy()
    idx4, _, _ = oracle.topk(oracle.router_logits(x4, wr4, b4), K)
    ex4, sh4 = oracle_layer_experts(W, 4, sorted(set(idx4.reshape(-1).tolist())), 0)
    t0 = time.perf_counter()
    y4, _, _ = oracle.moe_forward(x4, wr4, b4, ex4, sh4, H, I, K)
    oracle.rmsnorm(y4, 1e-6)
    el = time.perf_counter() - t0
    legs["stack_t8_40_layers"] = {"value": round(cs["T"] / (el * 40), 3), "unit": "tokens/s",
                                  "ms_per_step": round(el * 1e3 * 40, 1),
                                  "sample": f"layer 0 of 40 on 8 tokens in {el:.2f} s, "
                                            f"scaled x 40"}
    draws = [[w.cpu().numpy() for w in W.expert_weights(4, e, "cuda", 0)] for e in range(16)]
    t0 = time.perf_counter()
    for ws in draws:
        for w in ws:
            oracle.quant_int4_g64(w)
    el = time.perf_counter() - t0
    legs["quantise_one_layer"] = {"value": round(el * 1e3 * 16, 1), "unit": "ms per layer",
                                  "sample": f"16 of 256 experts (48 matrices) in {el:.2f} s, "
                                            f"scaled x 16"}
    c0 = W.CONFIGS[0]
    wr0 = bits(W.router_weights(0, "cuda"))
    pool0 = W.token_pool(0, 8, "cuda").cpu().numpy()
    ex0, sh0 = oracle_layer_experts(W, 0, list(range(c0["E"])))
    done0 = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) < 0.5:
        k = done0 % 8
        oracle.moe_forward(pool0[k:k + 1], wr0, None, ex0, sh0, c0["H"], c0["I"], c0["K"])
        done0 += 1
    el = time.perf_counter() - t0
    legs["tiny_t1"] = {"value": round(done0 / el, 1), "unit": "tokens/s",
                       "sample": f"{done0} single-token forwards of the tiny layer, "
                                 f"8 tokens cycled, {el:.2f} s"}
    head = legs["decode_t1"]
    return {"value": head["value"], "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"decode T=1: {head['sample']} (H=6144, I=2048, E=256, K=8 + shared, "
                      f"fp64); experts quantised by the oracle beforehand (untimed)",
            "legs": legs}


# The single-token kernels' sources: the kernel file and the headers it compiles in.
# A committed profile summary carries the sha256 of their concatenation.
NARROW_SRC = ("int4_grouped_expert_amd/csrc/ffn_narrow.hip", "int4_grouped_expert_amd/csrc/wave.h",
              "int4_grouped_expert_amd/csrc/kernels.h")


def source_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def profile_fields(path, kernel_src):
    """The machine-read fields ("- key: value" lines) of a committed profile summary,
    or None when that summary was taken on a different version of the kernel's
    sources."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_sha256(kernel_src):
        return None
    return fields


def profiled_launch_ms(kernel_src):
    """gateup_narrow's kernel-trace average (ms) from profiles/decode_t1_kernels.md, or
    None when the summary is of another source version."""
    f = profile_fields(os.path.join(ROOT, "profiles", "decode_t1_kernels.md"), kernel_src)
    try:
        return None if f is None else float(f["gateup_narrow_avg_us"]) * 1e-3
    except (KeyError, ValueError):
        return None


def profiled_traffic(kernel_src, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<kernel>_decode_t1_traffic.md), or None when that summary was taken
    on a different version of the kernel's sources."""
    f = profile_fields(os.path.join(ROOT, "profiles", f"{kernel}_decode_t1_traffic.md"),
                       kernel_src)
    try:
        return None if f is None else int(f["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every leg after the T=1 one")
    ap.add_argument("--legs", default="single,t32,cache,tiny,formats,prefill",
                    help="comma list of the legs after the T=1 one (default: all)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain elementwise kernel (clamp) that reads and writes "
                         "MIB MiB, the reference for scaling HBM byte counters")
    ap.add_argument("--stack", action="store_true",
                    help="only the 40-layer T=8 stack (218 GB resident) and the quantiser "
                         "timing; prints its own JSON line")
    ap.add_argument("--stack-cfg", type=int, default=4, help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the expert-parallel design for more GPUs is described, not built)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import int4_grouped_expert_amd as coli
    import workloads as W
    assert torch.cuda.is_available()
    torch.cuda.set_device(0)
    c = W.CONFIGS[1]
    if args.copy_probe:
        n = (args.copy_probe << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.clamp(a, min=-1e30, max=1e30, out=b)  # reads and writes copy_probe MiB
        torch.cuda.synchronize()
        log(f"[bench] copy probe: clamp kernel, {args.copy_probe} MiB read + written, 3 launches")
        del a, b

    if args.stack:
        log("[bench] stack: building 40 layers")
        steps = args.steps if args.steps != 3000 else 20
        warmup = args.warmup if args.warmup != 300 else 3
        print(json.dumps(run_stack(coli, W, steps, warmup, cfg_id=args.stack_cfg)), flush=True)
        return

    log(f"[bench] building layer ({args.replicas} replicas)")
    layers, nb = build_layer(coli, W, 1, args.replicas)
    log("[bench] decode T=1")
    d = run_decode(coli, W, layers, 1, 1, args.steps, args.warmup)
    ms_step = d["ms"] / d["steps"]
    U = 8  # T=1, top-8: always 8 distinct routed experts + the shared one
    step_bytes = decode_bytes(c, U, 1)
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    gu_bytes = gateup_bytes(c, U, 1)
    gu_ms = d["stage_ms"][1]
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(1.0 / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode: MoE layer H=6144 I=2048, 256 routed experts top-8 + 1 "
                               "shared, int4-g64 planar, T=1 fp32 token",
                   "replicas": args.replicas, "token_pool": 64},
        "hbm": {"bytes_per_step": step_bytes, "gbps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBS, 4)},
        "step_ms": d["step_ms"],
        "stage_ms": {"route": round(d["stage_ms"][0], 5), "gateup": round(d["stage_ms"][1], 5),
                     "down_combine": round(d["stage_ms"][2], 5)},
        "roofline": {"kernel": "gateup_narrow", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(NARROW_SRC, "gateup_narrow"),
                     "bytes_per_launch": gu_bytes, "avg_launch_ms": round(gu_ms, 5)},
    }
    prof_ms = profiled_launch_ms(NARROW_SRC)
    if prof_ms is not None:
        # the committed kernel-trace average of the same source (profiles/)
        result["roofline"]["profiled_avg_launch_ms"] = round(prof_ms, 5)
        result["roofline"]["profiled_frac"] = round(gu_bytes / prof_ms * 1e-6 / HBM_PEAK_GBS, 4)
    legs = set() if args.no_extras else set(args.legs.split(","))
    if "single" in legs:
        log("[bench] decode T=1, one replica (its 191 MB fit the 256 MB Infinity Cache)")
        d1 = run_decode(coli, W, layers[:1], 1, 1, max(100, args.steps // 3),
                        min(100, args.warmup))
        ms1 = d1["ms"] / d1["steps"]
        result["single_replica_cached"] = {
            "note": "the same step on one copy of the layer: weights may be served from "
                    "the Infinity Cache, so this is not an HBM figure",
            "tokens_per_s": round(1.0 / (ms1 * 1e-3), 1), "ms_per_step": round(ms1, 5),
            "step_ms": d1["step_ms"],
            "stage_ms": [round(x, 5) for x in d1["stage_ms"]]}
    if "t32" in legs or "cache" in legs:
        zl, _ = build_layer_bias(coli, W, layers)
    if "t32" in legs:
        log("[bench] decode T=32 zipf")
        d32 = run_decode(coli, W, zl, 2, 32, max(20, args.steps // 10), min(20, args.warmup))
        U32 = d32["u_mean"]
        ms32 = d32["ms"] / d32["steps"]
        b32 = decode_bytes(W.CONFIGS[2], U32, 32)
        result["decode_t32_zipf"] = {
            "tokens_per_s": round(32 / (ms32 * 1e-3), 1), "ms_per_step": round(ms32, 4),
            "step_ms": d32["step_ms"],
            "unique_experts_mean": round(U32, 2),
            "bytes_per_step": int(b32),
            "gbps": round(b32 / (ms32 * 1e-3) / 1e9, 1),
            "frac": round(b32 / (ms32 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "stage_ms": [round(s, 4) for s in d32["stage_ms"]],
            "compute_ceiling": t32_compute_ceiling(W.CONFIGS[2])}
    if "cache" in legs:
        log("[bench] decode T=32 zipf through the HBM expert cache")
        result["expert_cache_t32_zipf"] = run_cache(coli, W, zl[0],
                                                    max(32, min(200, args.steps // 15)), 40)
    if "t32" in legs or "cache" in legs:
        del zl
    if "tiny" in legs:
        log("[bench] tiny T=1")
        tl, _ = build_layer(coli, W, 0, 1)
        dt = run_decode(coli, W, tl, 0, 1, max(100, args.steps // 3), min(100, args.warmup))
        mst = dt["ms"] / dt["steps"]
        result["tiny_t1"] = {
            "workload": "tiny: H=256 I=128, 16 experts top-4 + 1 shared, T=1 fp32 token "
                        "(launch and latency bound; no roofline)",
            "us_per_step": round(mst * 1e3, 2), "tokens_per_s": round(1.0 / (mst * 1e-3), 1),
            "stage_us": [round(1e3 * x, 2) for x in dt["stage_ms"]]}
        del tl
    if "formats" in legs:
        log("[bench] sibling-format matrix-vector products")
        result["formats_matvec_t1"] = run_formats(coli, W)
        log("[bench] the decode layer in each format")
        result["formats_layer_t1"] = run_format_layers(coli, W)
    if "prefill" in legs:
        log("[bench] prefill T=2048")
        result["prefill"] = run_prefill(coli, W, layers[0],
                                        steps=max(2, min(10, args.steps // 300)))
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(coli, W)
    print(json.dumps(result), flush=True)


def run_stack(coli, W, steps, warmup, pool_n=4, cfg_id=4, layers=None):
    """The 40-layer stack at T=8: all layers resident, RMSNorm between layers.

    Every expert of every layer is quantised by the library from its own seeded
    N(0, 0.02) draw; the 256 routed experts of layer 0 time the quantiser (all
    drawn first, then quantised back to back, after a first pass of each form).  A step feeds one batch
    of 8 tokens through the 40 layers; U per layer is measured on the last step."""
    import torch
    c = W.CONFIGS[cfg_id]
    H, I, E, K, T = c["H"], c["I"], c["E"], c["K"], c["T"]
    NL = c["layers"] if layers is None else layers
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    layers = []
    # the quantiser: layer 0's routed experts, drawn first (fp32, all resident),
    # then quantised back to back.  A first pass over the layer reads 10-15 %
    # slower than the passes after it (measured), so one pass of each form runs
    # first (reported as first_pass_ms), then the per-matrix form is timed once and
    # the batched form three times (median).
    experts0, shared0, nb = coli.alloc_layer_blobs(H, I, E)
    draws = [W.expert_weights(cfg_id, e, "cuda", 0) for e in range(E)]
    views = [coli.coli_expert_views(experts0.data_ptr() + e * nb, H, I) for e in range(E)]

    def ptrs(vals):
        return torch.tensor(vals, dtype=torch.int64, device="cuda")
    # the same 768 matrices in two batched launches (gate and up [I, H], down [H, I])
    gu_w = ptrs([draws[e][m].data_ptr() for e in range(E) for m in (0, 1)])
    gu_q = ptrs([views[e][m][0] for e in range(E) for m in (0, 1)])
    gu_s = ptrs([views[e][m][1] for e in range(E) for m in (0, 1)])
    d_w = ptrs([draws[e][2].data_ptr() for e in range(E)])
    d_q = ptrs([views[e][2][0] for e in range(E)])
    d_s = ptrs([views[e][2][1] for e in range(E)])
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def per_matrix():
        for e in range(E):
            coli.coli_quant_expert(experts0.data_ptr() + e * nb, H, I, *draws[e], status,
                                   finish=False)

    def batched():
        coli.coli_quant_int4_g64_many(gu_w, gu_q, gu_s, 2 * E, I, H, status)
        coli.coli_quant_int4_g64_many(d_w, d_q, d_s, E, H, I, status)

    def timed(fn):
        a, b = ev(), ev()
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    q_first = timed(per_matrix)
    qm_first = timed(batched)
    q_ms = timed(per_matrix)
    qm_all = [timed(batched) for _ in range(3)]
    qm_ms = sorted(qm_all)[1]
    for e in range(E):  # the group-major scale copies, outside the timed regions
        coli.coli_expert_finish(experts0.data_ptr() + e * nb, H, I)
    torch.cuda.synchronize()
    del draws
    torch.cuda.empty_cache()
    for l in range(NL):
        experts, shared, nb = (experts0, shared0, nb) if l == 0 else coli.alloc_layer_blobs(H, I, E)
        for e in range(E + 1):
            if l == 0 and e < E:
                continue
            wg, wu, wd = W.expert_weights(cfg_id, e, "cuda", l)
            ptr = shared.data_ptr() if e == E else experts.data_ptr() + e * nb
            coli.coli_quant_expert(ptr, H, I, wg, wu, wd, status)
            del wg, wu, wd
        wr = W.router_weights(cfg_id, "cuda", l).contiguous()
        b = torch.from_numpy(W.router_bias(cfg_id, l)).cuda()
        layers.append(coli.MoELayer(H, I, E, K, wr, experts, shared, b))
        if l % 10 == 9:
            log(f"[bench] stack: {l + 1} layers resident")
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ex_bytes = 3 * (I * (H // 64) * 32 + I * (H // 64) * 4)  # one expert: nibbles + scales
    q_bytes = E * (3 * H * I * 4 + ex_bytes)  # fp32 weights in, packed bytes and scales out
    pool = W.token_pool(cfg_id, pool_n * T, "cuda").reshape(pool_n, T, H).contiguous()
    x = torch.empty((T, H), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    ws = torch.empty(layers[0].workspace_bytes(T, coli.COLI_DECODE), dtype=torch.uint8,
                     device="cuda")
    idx = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(NL)]
    gates = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(NL)]
    callers = [Caller(coli, layers[l], coli.COLI_DECODE, x, y, ws, idx[l], gates[l])
               for l in range(NL)]

    def step(i):
        x.copy_(pool[i % pool_n])
        for l in range(NL):
            callers[l]()
            if l + 1 < NL:
                coli.coli_rmsnorm_f32(y, x, 1e-6)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    U = [int(torch.unique(t).numel()) for t in idx]
    rbytes = E * H * (2 if c["router"] == "bf16" else 4)
    step_bytes = sum(rbytes + (u + 1) * ex_bytes + 2 * T * H * 4 for u in U)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    return {
        "metric": "stack decode: ms per step (one batch of tokens through every layer); "
                  "quantiser ms for one layer's routed experts",
        "workload": f"stack: {NL} resident layers of H={H} I={I}, {E} experts top-{K} + 1 "
                    f"shared, int4-g64 planar, Zipf router bias per layer, RMSNorm between "
                    f"layers, T={T} fp32 tokens",
        "resident_bytes": NL * (E + 1) * nb, "expert_bytes_read": ex_bytes,
        "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
        "unique_experts_per_layer": {"mean": round(sum(U) / NL, 1), "min": min(U),
                                     "max": max(U)},
        "hbm": {"bytes_per_step": step_bytes, "gbps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBS, 4)},
        "quantiser": {"experts": E, "launches": 2, "ms": round(qm_ms, 3), "bytes": q_bytes,
                      "gbps": round(q_bytes / (qm_ms * 1e-3) / 1e9, 1),
                      "frac": round(q_bytes / (qm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "timed_ms": [round(v, 3) for v in qm_all],
                      "first_pass_ms": round(qm_first, 3),
                      "per_matrix_launches": {"launches": 3 * E, "ms": round(q_ms, 3),
                                              "first_pass_ms": round(q_first, 3),
                                              "gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1)}},
        "data": "synthetic", "dtype": "f32",
    }


def run_cache(coli, W, layer, steps, warmup, S=128, pool_n=16, repin_every=8,
              decay_every=64):
    """The T=32 Zipf decode with its routed experts in S HBM slots over pinned host
    memory (coli_cache_*): every step routes the batch (coli_moe_route), plans the
    loads (REPIN at the step boundary, then admission), stages the missing blobs
    over PCIe and runs the experts (coli_moe_experts) from the slots.

    Two batches are in flight: batch b routes on its own stream while batch b-1's
    experts run, and b's blob copies run on a copy stream at the same time, except
    the copies into a slot that batch b-1 still reads, which wait for it.  Workspace,
    slot map and ids are double-buffered by batch parity."""
    import numpy as np
    import torch
    c = W.CONFIGS[2]
    T, H, I, E, K = c["T"], c["H"], c["I"], c["E"], c["K"]
    nb = coli.coli_expert_blob_bytes(H, I)
    host = torch.empty(E * nb, dtype=torch.uint8, pin_memory=True)
    host.copy_(layer.experts)
    slots = torch.empty(S * nb, dtype=torch.uint8, device="cuda")
    smaps = [torch.full((E,), -1, dtype=torch.int32, device="cuda") for _ in range(2)]
    hmaps = [torch.empty(E, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    lays = [coli.MoELayer(H, I, E, K, layer.w_router, slots, layer.shared, layer.bias,
                          slot_map=smaps[j]) for j in range(2)]
    cache = coli.Cache(E, S)
    pool = W.token_pool(2, pool_n * T, "cuda").reshape(pool_n, T, H).contiguous()
    wsb = lays[0].workspace_bytes(T, coli.COLI_DECODE)
    ws = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    idx = [torch.empty((T, K), dtype=torch.int32, device="cuda") for _ in range(2)]
    gates = [torch.empty((T, K), dtype=torch.float32, device="cuda") for _ in range(2)]
    y = [torch.empty((T, H), dtype=torch.float32, device="cuda") for _ in range(2)]
    uq = [torch.empty(E + 1, dtype=torch.int32, device="cuda") for _ in range(2)]
    uq_h = [torch.empty(E + 1, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    sR, sC, sP = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    c_ev = [None, None]          # experts done, per parity
    used_prev = set()            # slots batch b-1 reads
    stats = dict(needed=0, misses=0, swaps=0, deferred=0, loads=0)
    torch.cuda.synchronize()

    def step(b, count):
        nonlocal used_prev
        j = b % 2
        x = pool[b % pool_n]
        with torch.cuda.stream(sR):
            if c_ev[j] is not None:
                sR.wait_event(c_ev[j])  # batch b-2 done with this parity's buffers
            coli.coli_moe_route(lays[j], coli.COLI_DECODE, x, ws[j], idx[j], gates[j],
                                uq[j][:E], uq[j][E:], stream=sR)
            uq_h[j].copy_(uq[j], non_blocking=True)
            r_ev = torch.cuda.Event()
            r_ev.record(sR)
        r_ev.synchronize()
        n = int(uq_h[j][E])
        needed = uq_h[j].numpy()[:n]
        loads = []
        if b % decay_every == decay_every - 1:
            cache.decay()
        if b % repin_every == repin_every - 1:
            sw = cache.repin(4)
            loads += [(h, s_) for h, s_, _ in sw]
            if count:
                stats["swaps"] += len(sw)
        adm = cache.admit(needed)
        loads += adm
        now = [ld for ld in loads if ld[1] not in used_prev]
        later = [ld for ld in loads if ld[1] in used_prev]
        if count:
            stats["needed"] += n
            stats["misses"] += len(adm)
            stats["deferred"] += len(later)
            stats["loads"] += len(loads)
        hmaps[j].numpy()[:] = cache.slot_of
        with torch.cuda.stream(sP):
            if now:
                coli.coli_cache_stage(host, slots, nb, now, stream=sP)
            prev = c_ev[1 - j]
            if prev is not None:
                sP.wait_event(prev)  # batch b-1's experts: its slots and map are free
            if later:
                coli.coli_cache_stage(host, slots, nb, later, stream=sP)
            smaps[j].copy_(hmaps[j], non_blocking=True)
            p_ev = torch.cuda.Event()
            p_ev.record(sP)
        with torch.cuda.stream(sC):
            sC.wait_event(p_ev)
            sC.wait_event(r_ev)
            coli.coli_moe_experts(lays[j], coli.COLI_DECODE, x, y[j], ws[j], idx[j], gates[j],
                                  stream=sC, status=status)
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(sC)
            c_ev[j] = ev
        used_prev = {int(cache.slot_of[e]) for e in needed}
        return ev

    for b in range(warmup):
        step(b, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    first = step(warmup, True)
    for b in range(warmup + 1, warmup + steps):
        last = step(b, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = first.elapsed_time(last) / (steps - 1)
    assert int(status.item()) == 0, "a routed expert was not resident"
    # the PCIe ceiling: one large pinned host -> device copy
    big = min(E, 64) * nb
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    slots[:min(big, S * nb)].copy_(host[:min(big, S * nb)], non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d = min(big, S * nb) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    staged = stats["loads"] * nb
    out = dict(
        workload=f"T=32 Zipf decode of the decode-shaped layer with {S} of {E} expert blobs "
                 f"in HBM slots, all {E} in pinned host memory; REPIN every {repin_every} "
                 f"steps, heat halved every {decay_every}",
        slots=S, blob_bytes=nb, steps=steps, warmup=warmup,
        ms_per_step=round(ms, 4), wall_ms_per_step=round(1e3 * wall / steps, 4),
        tokens_per_s=round(T / (ms * 1e-3), 1),
        unique_experts_mean=round(stats["needed"] / steps, 2),
        hit_rate=round(1.0 - stats["misses"] / max(1, stats["needed"]), 4),
        misses_per_step=round(stats["misses"] / steps, 3),
        repin_swaps_per_step=round(stats["swaps"] / steps, 3),
        deferred_frac=round(stats["deferred"] / max(1, stats["loads"]), 4),
        staged_gbps=round(staged / (ms * 1e-3 * steps) / 1e9, 2),
        h2d_copy_gbps=round(h2d, 2))
    del host, slots
    torch.cuda.empty_cache()
    return out


def run_formats(coli, W, steps=50, warmup=5):
    """The dequantising matrix-vector product of each weight format on the gate and
    up rows of one single-token step (9 units x 2 x 2048 rows, I = 6144), T = 1:
    HBM GB/s of the packed bytes + scales per launch.  Copies of the matrix are
    rotated so that at least 1 GiB is streamed between reuses (the 256 MB
    Infinity Cache cannot serve it)."""
    import torch
    O, I = 9 * 2 * 2048, 6144
    out = {}
    w = torch.randn((O, I), device="cuda") * 0.02
    x = torch.randn((1, I), device="cuda")
    y = torch.empty((1, O), device="cuda")
    for fmt, name in ((4, "int4-g64"), (5, "int3-g64"), (7, "mxfp4"), (8, "fp8-e4m3-b128")):
        nw, ns = coli.coli_fmt_bytes(fmt, O, I)
        ncopy = max(2, -(-(1 << 30) // (nw + ns)))
        pk = [torch.empty(nw, dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        sc = [torch.empty(max(ns, 16), dtype=torch.uint8, device="cuda") for _ in range(ncopy)]
        coli.coli_quant_fmt(fmt, w, pk[0], sc[0])
        for j in range(1, ncopy):
            pk[j].copy_(pk[0])
            sc[j].copy_(sc[0])
        args = [(fmt, ctypes.c_void_p(pk[j].data_ptr()), ctypes.c_void_p(sc[j].data_ptr()), O, I,
                 ctypes.c_void_p(x.data_ptr()), 1, ctypes.c_void_p(y.data_ptr()),
                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
                for j in range(ncopy)]
        for i in range(warmup):
            coli.lib.coli_matvec_fmt(*args[i % ncopy])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            st = coli.lib.coli_matvec_fmt(*args[i % ncopy])
            if st:
                raise RuntimeError(f"coli_matvec_fmt: {st}")
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbytes = nw + ns + I * 4 + O * 4
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us_per_launch": round(1e3 * ms, 2), "bytes_per_launch": nbytes,
                     "gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBS, 4),
                     "bits_per_weight": round(8.0 * (nw + ns) / (O * I), 3)}
        del pk, sc
    torch.cuda.empty_cache()
    return {"workload": f"y = W^ x, W [{O}, {I}] (the gate and up rows of 9 units), T = 1 "
                        "fp32 token", "formats": out}


def run_format_layers(coli, W, steps=200, warmup=20, pool_n=64):
    """The single-token decode layer with its experts in each sibling format
    (coli_moe_forward_fmt): tokens/s and HBM GB/s over the algorithmic bytes of a
    step (router, the 9 units' blobs in the format, x and y).  One copy of each
    layer (257 blobs), rotating 64 tokens, so consecutive steps read different
    experts and the Infinity Cache serves little."""
    import torch
    c = W.CONFIGS[1]
    H, I, E, K = c["H"], c["I"], c["E"], c["K"]
    wr = W.router_weights(1, "cuda").contiguous()
    pool = W.token_pool(1, pool_n, "cuda").contiguous()
    out = {}
    for fmt, name in ((4, "int4-g64"), (5, "int3-g64"), (7, "mxfp4"), (8, "fp8-e4m3-b128")):
        nb = coli.coli_fmt_blob_bytes(fmt, H, I)
        experts = torch.empty(E * nb, dtype=torch.uint8, device="cuda")
        shared = torch.empty(nb, dtype=torch.uint8, device="cuda")
        for e in range(E + 1):
            wg, wu, wd = W.expert_weights(1, e, "cuda")
            ptr = shared.data_ptr() if e == E else experts.data_ptr() + e * nb
            coli.coli_quant_expert_fmt(fmt, ptr, H, I, wg, wu, wd)
            del wg, wu, wd
        L = coli.MoELayer(H, I, E, K, wr, experts, shared)
        ws = torch.empty(coli.coli_moe_fmt_workspace_bytes(L, fmt, 1), dtype=torch.uint8,
                         device="cuda")
        y = torch.empty((1, H), device="cuda")
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = [(ctypes.byref(L.c), fmt, ctypes.c_void_p(pool[p:p + 1].data_ptr()), 1,
                 ctypes.c_void_p(y.data_ptr()), None, None, None,
                 ctypes.c_void_p(ws.data_ptr()), ws.numel(), st) for p in range(pool_n)]
        for i in range(warmup):
            coli.lib.coli_moe_forward_fmt(*args[i % pool_n])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            rc = coli.lib.coli_moe_forward_fmt(*args[i % pool_n])
            if rc:
                raise RuntimeError(f"coli_moe_forward_fmt: {rc}")
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        wq = 2 * sum(coli.coli_fmt_bytes(fmt, I, H)) + sum(coli.coli_fmt_bytes(fmt, H, I))
        nbytes = E * H * 2 + (K + 1) * wq + 2 * H * 4
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us_per_step": round(1e3 * ms, 2), "tokens_per_s": round(1e3 / ms, 1),
                     "bytes_per_step": nbytes, "gbps": round(gbps, 1),
                     "frac": round(gbps / HBM_PEAK_GBS, 4)}
        del experts, shared, L, ws
        torch.cuda.empty_cache()
    return {"workload": "decode T=1 of the H=6144 I=2048, 256 experts top-8 + 1 shared layer "
                        "with its experts in each format (one copy, 64-token pool)",
            "formats": out}


def build_layer_bias(coli, W, layers):
    """The T=32 workload shares the decode layer's weights, with the Zipf router bias."""
    import torch
    b = torch.from_numpy(W.router_bias(2)).cuda()
    out = []
    for L in layers:
        out.append(coli.MoELayer(L.H, L.I, L.E, L.K, L.w_router, L.experts, L.shared, b))
    return out, None


if __name__ == "__main__":
    main()
