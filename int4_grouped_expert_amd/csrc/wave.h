// wave.h -- wave-level building blocks shared by the routing and decode
// kernels: DPP reductions (every lane gets the same value, combined in a
// fixed order) and the per-token top-K with renormalised gates.
//
// Top-K: page "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
// section 十一 (per-token top-k experts; its GLM router scores with a sigmoid,
// one expert group, a selection-only bias); gates normalised over the selected
// experts (page "colibrì 路由遥测全解析", section 分离计数与追踪); NaN logits
// never win (same page, section 测试与 CI 保障).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace coli {

constexpr int kWaveLanes = 64;

// Wave-wide reductions: an all-reduce inside each 16-lane DPP row (quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror pair every lane
// with a disjoint partner set, doubling it each step), then the four row
// results are read with v_readlane and combined in a fixed order, so every
// lane gets the same, deterministic value.
template <int kCtrl>
__device__ inline float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ inline float rdlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ inline float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (rdlane_f(v, 0) + rdlane_f(v, 16)) + (rdlane_f(v, 32) + rdlane_f(v, 48));
}
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(rdlane_f(v, 0), rdlane_f(v, 16)), fmaxf(rdlane_f(v, 32), rdlane_f(v, 48)));
}
// (value, id) arg-max: larger value wins, equal values go to the lower id,
// id < 0 marks "no candidate".
__device__ inline void take_better(float &bv, int &bi, float ov, int oi) {
  const bool take = oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}
__device__ inline void wave_argmax(float &bv, int &bi) {
#define COLI_ARG_STEP(ctrl)                                                          \
  {                                                                                  \
    const float ov = dpp_f<ctrl>(bv);                                                \
    const int oi = __builtin_amdgcn_update_dpp(-1, bi, ctrl, 0xF, 0xF, false);       \
    take_better(bv, bi, ov, oi);                                                     \
  }
  COLI_ARG_STEP(0xB1)
  COLI_ARG_STEP(0x4E)
  COLI_ARG_STEP(0x141)
  COLI_ARG_STEP(0x140)
#undef COLI_ARG_STEP
  float v = rdlane_f(bv, 0);
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    take_better(v, i, rdlane_f(bv, 16 * r), __builtin_amdgcn_readlane(bi, 16 * r));
  bv = v;
  bi = i;
}

template <int kCtrl>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kCtrl, 0xF, 0xF, false));
}
// Wave maximum of an unsigned value (same DPP pattern as wave_max).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const uint32_t r0 = __builtin_amdgcn_readlane(int(v), 0), r1 = __builtin_amdgcn_readlane(int(v), 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(int(v), 32), r3 = __builtin_amdgcn_readlane(int(v), 48);
  return max(max(r0, r1), max(r2, r3));
}
// Order-preserving bits of a float: the unsigned order of the results is the
// order of the values, and equal values (-0 and +0 included: v + 0 turns -0
// into +0) give equal bits; never 0 for a non-NaN value.
__device__ inline uint32_t order_bits(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// K rounds of wave arg-max over the keys v (PL per lane, lane l holds ids
// l, l + 64, ...): a round takes the largest key not yet taken, ties to the
// lowest id; a round with no valid candidate left (NaN keys) takes id `round`
// if free, else the lowest free id.  Sets bit j of `taken` for each pick of
// this lane.  Each lane keeps its best untaken candidate (order bits, 0 for
// none, and its slot j); after a round only the winner's lane rescans.
template <int PL>
__device__ __attribute__((always_inline)) inline void topk_rounds(const float (&v)[PL], int E,
                                                                   int K, int lane,
                                                                   uint32_t &taken) {
  uint32_t lk = 0;
  int lj = 0;
  auto rescan = [&]() {
    lk = 0;
    lj = 0;
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = lane + kWaveLanes * j;
      const bool cand = e < E && !__builtin_isnan(v[j]) && !((taken >> j) & 1u);
      const uint32_t o = cand ? order_bits(v[j]) : 0u;
      lj = o > lk ? j : lj;
      lk = o > lk ? o : lk;
    }
  };
  rescan();
  for (int round = 0; round < K; ++round) {
    const uint32_t wk = wave_max_u32(lk);
    int bi;
    if (wk != 0) {
      const uint64_t hold = __ballot(lk == wk);
      if (__popcll(hold) == 1) {
        const int wl = __ffsll((unsigned long long)hold) - 1;
        bi = wl + kWaveLanes * __builtin_amdgcn_readlane(lj, wl);
      } else {
        int id = lk == wk ? lane + kWaveLanes * lj : 0x7fffffff;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) id = min(id, __shfl_xor(id, m, kWaveLanes));
        bi = id;
      }
    } else {
      // No valid candidate: id `round` if free, else the lowest free id.
      int free_lo = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const int e = lane + kWaveLanes * j;
        if (e < E && !((taken >> j) & 1u)) free_lo = min(free_lo, e);
      }
      int own_free = 0;
      if (round < E && (round % kWaveLanes) == lane) own_free = !((taken >> (round / kWaveLanes)) & 1u);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {  // rare path (NaN logits)
        free_lo = min(free_lo, __shfl_xor(free_lo, m, kWaveLanes));
        own_free |= __shfl_xor(own_free, m, kWaveLanes);
      }
      bi = own_free ? round : free_lo;
    }
    if ((bi % kWaveLanes) == lane) {
      taken |= 1u << (bi / kWaveLanes);
      rescan();
    }
  }
}

// Wave maximum of an unsigned value, in every lane, without leaving the VGPRs:
// the DPP row steps of wave_max_u32, then the row pairs (v_permlane16_swap) and
// the wave halves (v_permlane32_swap).
__device__ inline uint32_t wave_max_u32_v(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(uint32_t(a[0]), uint32_t(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(uint32_t(b[0]), uint32_t(b[1]));
}

// K picks over keys with at least K nonzero (order bits; 0 = no candidate),
// PL <= 4 per lane (lane l holds ids l, l + 64, ...): largest key first, equal
// keys to the lowest id.  Each lane sorts its (key, slot) pairs once, largest
// key first and equal keys by slot; a round is the wave maximum of the lanes'
// head keys, its holder (the lowest id among several: rare) records the head's
// slot in `taken` and pops it.
template <int PL>
__device__ __attribute__((always_inline)) inline void topk_sorted_heads(const uint32_t (&key)[PL],
                                                                         int K, int lane,
                                                                         uint32_t &taken) {
  // composite (key, PL - 1 - slot): a larger composite is the better candidate
  static_assert(PL == 1 || PL == 2 || PL == 4, "sorted heads: 1, 2 or 4 keys per lane");
  uint64_t c[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) c[j] = (uint64_t(key[j]) << 8) | uint64_t(PL - 1 - j);
  auto cas = [&](int a, int b) {
    const uint64_t hi = c[a] > c[b] ? c[a] : c[b], lo = c[a] > c[b] ? c[b] : c[a];
    c[a] = hi;
    c[b] = lo;
  };
  if (PL == 2) cas(0, 1);
  if (PL == 4) {
    cas(0, 1); cas(2, 3); cas(0, 2); cas(1, 3); cas(1, 2);
  }
  for (int round = 0; round < K; ++round) {
    const uint32_t hk = uint32_t(c[0] >> 8);
    const uint32_t wk = wave_max_u32_v(hk);  // nonzero: K candidates exist
    const uint64_t hold = __ballot(hk == wk);
    int wl;
    if (__popcll(hold) == 1) {
      wl = __ffsll((unsigned long long)hold) - 1;
    } else {
      // equal keys in several lanes: the lowest id among them
      int id = hk == wk ? lane + kWaveLanes * (PL - 1 - int(c[0] & 0xFF)) : 0x7fffffff;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) id = min(id, __shfl_xor(id, m, kWaveLanes));
      wl = id % kWaveLanes;
    }
    if (lane == wl) {
      taken |= 1u << (PL - 1 - int(c[0] & 0xFF));
#pragma unroll
      for (int j = 0; j + 1 < PL; ++j) c[j] = c[j + 1];
      c[PL - 1] = 0;
    }
  }
}

// Wave-wide top-K of one token, PL logits per lane (E <= 64 PL).  Writes
// idx/gates in ascending id order.
// The token's logits, PL per lane (lane l holds ids l, l + 64, ...).
template <int PL>
__device__ __attribute__((always_inline)) inline void topk_load(const float *__restrict__ lrow,
                                                                 int E, int lane, float (&v)[PL]) {
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + kWaveLanes * j;
    v[j] = e < E ? lrow[e] : 0.0f;
  }
}

// Selection and gates from logits already in registers (see topk_load).
template <int PL>
__device__ __attribute__((always_inline)) inline void topk_select(
    const float (&v_in)[PL], int E, int K, int lane, int32_t *__restrict__ idx_out,
    float *__restrict__ gate_out, Scoring sc = Scoring{0, nullptr}) {
  // keys of the selection (the logits themselves, or the biased sigmoid scores)
  float v[PL], sgm[PL];
  if (sc.sigmoid) {
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = lane + kWaveLanes * j;
      sgm[j] = 1.0f / (1.0f + expf(-v_in[j]));
      v[j] = sgm[j] + ((sc.bias && e < E) ? sc.bias[e] : 0.0f);
    }
  } else {
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      v[j] = v_in[j];
      sgm[j] = 0.0f;
    }
  }
  // Keys are the order bits (0: no candidate, for NaN and ids >= E).  With at
  // least K candidates and PL <= 4 each lane sorts its keys once (largest
  // first, equal keys by slot), so a round is a wave maximum of the lanes'
  // head keys and a pop in the winning lane; otherwise the rounds rescan.
  uint32_t taken = 0;
  int nvalid = 0;
  uint32_t key[PL];
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const int e = lane + kWaveLanes * j;
    key[j] = (e < E && !__builtin_isnan(v[j])) ? order_bits(v[j]) : 0u;
    nvalid += __popcll(__ballot(key[j] != 0u));
  }
  if constexpr (PL <= 4) {
    if (nvalid >= K)
      topk_sorted_heads<PL>(key, K, lane, taken);
    else
      topk_rounds<PL>(v, E, K, lane, taken);
  } else {
    topk_rounds<PL>(v, E, K, lane, taken);
  }
  // gate numerators: exp(l - m) over the selected logits (softmax), or the
  // selected scores (sigmoid); the normaliser is their wave sum (identical on
  // every lane)
  float num[PL];
  if (sc.sigmoid) {
#pragma unroll
    for (int j = 0; j < PL; ++j) num[j] = sgm[j];
  } else {
    float m = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < PL; ++j)
      if ((taken >> j) & 1u) m = fmaxf(m, v[j]);
    m = wave_max(m);
#pragma unroll
    for (int j = 0; j < PL; ++j) num[j] = expf(v[j] - m);
  }
  float z = 0.0f;
#pragma unroll
  for (int j = 0; j < PL; ++j)
    if ((taken >> j) & 1u) z += num[j];
  z = wave_sum(z);
  int before = 0;
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const uint64_t bal = __ballot((taken >> j) & 1u);
    if ((taken >> j) & 1u) {
      const int rank = before + __popcll(bal & ((1ull << lane) - 1ull));
      idx_out[rank] = lane + kWaveLanes * j;
      gate_out[rank] = num[j] / z;
    }
    before += __popcll(bal);
  }
}

template <int PL>
__device__ __attribute__((always_inline)) inline void wave_topk_pl(
    const float *__restrict__ lrow, int E, int K, int lane, int32_t *__restrict__ idx_out,
    float *__restrict__ gate_out, Scoring sc) {
  float v[PL];
  topk_load<PL>(lrow, E, lane, v);
  topk_select<PL>(v, E, K, lane, idx_out, gate_out, sc);
}

// Dispatch on the logits per lane, ceil(E / 64) rounded up to 1, 2, 4, 8, 16.
__device__ __attribute__((always_inline)) inline void wave_topk(
    const float *__restrict__ lrow, int E, int K, int lane, int32_t *__restrict__ idx_out,
    float *__restrict__ gate_out, Scoring sc = Scoring{0, nullptr}) {
  if (E <= 64) wave_topk_pl<1>(lrow, E, K, lane, idx_out, gate_out, sc);
  else if (E <= 128) wave_topk_pl<2>(lrow, E, K, lane, idx_out, gate_out, sc);
  else if (E <= 256) wave_topk_pl<4>(lrow, E, K, lane, idx_out, gate_out, sc);
  else if (E <= 512) wave_topk_pl<8>(lrow, E, K, lane, idx_out, gate_out, sc);
  else wave_topk_pl<16>(lrow, E, K, lane, idx_out, gate_out, sc);
}

// ---- digit planes (single-token decode activations) ----------------------
template <int kCtrl>
__device__ inline int dpp_row_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
// Sum over the 16 lanes of each DPP row (every lane of the row gets it).
__device__ inline int row16_sum_i(int v) {
  v += dpp_row_i<0xB1>(v);
  v += dpp_row_i<0x4E>(v);
  v += dpp_row_i<0x141>(v);
  v += dpp_row_i<0x140>(v);
  return v;
}

// Four balanced base-128 digits of rint(v * 2^e) (|v * 2^e| <= 2^27; the
// clamp only matters for non-finite v, whose result is flagged elsewhere).
__device__ inline void digits4(float v, int e, int d[4]) {
  const float sv = fminf(fmaxf(ldexpf(v, e), -134217728.0f), 134217728.0f);
  int a = int(rintf(sv));
  d[3] = ((a + 64) & 127) - 64;
  a = (a - d[3]) >> 7;
  d[2] = ((a + 64) & 127) - 64;
  a = (a - d[2]) >> 7;
  d[1] = ((a + 64) & 127) - 64;
  a = (a - d[1]) >> 7;
  d[0] = a;
}

// 4-element runs: digits of elements el .. el+3 (el % 4 == 0) of a 64-element
// group sit at this byte offset of the group's 64-byte plane ("A order": run
// rho = elements 8 rho .. 8 rho + 7, then 32 + 8 rho .. 32 + 8 rho + 7).
__device__ inline int aorder_pos(int el) {
  return el < 32 ? 16 * (el / 8) + (el % 8) : 16 * ((el - 32) / 8) + 8 + (el % 8);
}
// Pack plane p of four elements' digits into one little-endian word.
__device__ inline uint32_t pack_plane(const int d[4][4], int p) {
  return (uint32_t(d[0][p]) & 0xFFu) | ((uint32_t(d[1][p]) & 0xFFu) << 8) |
         ((uint32_t(d[2][p]) & 0xFFu) << 16) | ((uint32_t(d[3][p]) & 0xFFu) << 24);
}
// Scale exponent e of a vector with max |v| = m: m * 2^e in [2^26, 2^27).
__device__ inline int digit_exponent(float m) {
  int ex = 0;
  (void)frexpf(m, &ex);
  return m > 0.0f ? 27 - ex : 0;
}

}  // namespace coli
