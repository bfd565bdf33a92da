// gemm_stream.h -- building blocks of the grouped int4-g64 GEMMs (prefill and
// decode batch): buffer-resource loads, the LDS DMA, the whole-line weight
// exchange, the staged activation order and the (chunk, N-tile) work items.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 (planar int4-g64 rows: byte k of a group holds element k
// in its low nibble, element k + 32 in its high nibble); batch union, page
// "Colibrì 深度解析", section 四 (work items walk the unique experts of the
// batch, each applied to all of its tokens).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace coli {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;                      // one per SIMD
constexpr int kThreads = kWave * kWaves;
constexpr int kRowB = 512;                     // staged bytes per chunk row per super-step
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ inline uint32_t pack_f16x2(_Float16 a, _Float16 b) {
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Position of element e (0..63) of a group inside the group's 64 staged slots.
__device__ inline int grp_pos(int e) {
  const int c = 4 * ((e >> 4) & 1) + ((e >> 2) & 3);
  const int i = ((e & 1) << 2) | (((e >> 5) & 1) << 1) | ((e >> 1) & 1);
  return 8 * c + i;
}

// Item decode shared by the two GEMMs.  chunk: the batch's per-unit chunk
// prefix (r.chunk, or a copy of it in LDS), nu = units + 1 (the shared one last).
struct Item {
  int unit, mchunk, ntile;
  bool shared;
  bool missing;  // a routed expert with no slot in the layer's slot map
  const uint8_t *blob;
  int jb, je;  // token rows of the chunk: j in [jb, je)
};
__device__ inline void decode_item(const LayerDev &L, const Routing &r, int T, int item, int n_nt,
                                   Item &it, int mc, const int *chunk, int nu) {
  const int c = item / n_nt;
  it.ntile = item % n_nt;
  int lo = 0, hi = nu - 1;  // last u with chunk[u] <= c
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk[mid] <= c) lo = mid; else hi = mid - 1;
  }
  it.unit = lo;
  it.mchunk = c - chunk[lo];
  it.shared = lo == nu - 1;
  int jb0, je0;
  it.missing = false;
  if (!it.shared) {
    const int e = r.unique[lo];
    bool miss;
    it.blob = expert_blob(L, e, miss);
    it.missing = miss;
    jb0 = r.offsets[e];
    je0 = r.offsets[e + 1];
  } else {
    it.blob = L.shared;
    jb0 = 0;
    je0 = T;
  }
  it.jb = jb0 + it.mchunk * mc;
  it.je = min(je0, it.jb + mc);
}

__device__ inline uint32_t word_of(const uint4 &v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// SiLU with the hardware exp2 and reciprocal (relative error ~1e-6, far below
// the fp16 rounding of h that follows)
__device__ inline float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * z));
}

// Buffer resource over [p, p + bytes): raw buffer loads at offsets >= bytes
// return zeros, so masked lanes take the offset kOff and no branch.
constexpr uint32_t kOff = 0x80000000u;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, int(bytes), 0x00020000);
}
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return uint4{uint32_t(v[0]), uint32_t(v[1]), uint32_t(v[2]), uint32_t(v[3])};
}
__device__ inline float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, uint32_t(__builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0)));
}

// 4x4 exchange of a fragment's four loads with lane bits 3 and 4: on return
// D[d] of lane L is R[(L & 31) / 8] of lane (L & ~24) | 8 d, i.e. register d
// takes what the lane's row-mate with bits 3-4 = d loaded into register
// (bits 3-4 of L).  DPP half-row moves for bit 3, v_permlane16_swap for bit 4.
__device__ inline void exchange_rows(const uint4 (&R)[4], uint4 (&D)[4]) {
  uint4 Q[4];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t xs[4] = {R[2 * e].x, R[2 * e].y, R[2 * e].z, R[2 * e].w};
    const uint32_t ys[4] = {R[2 * e + 1].x, R[2 * e + 1].y, R[2 * e + 1].z, R[2 * e + 1].w};
    uint32_t xo[4], yo[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // lanes 8..15 of each 16-lane row take the other register's lanes 0..7, and back
      xo[d] = uint32_t(__builtin_amdgcn_update_dpp(int(xs[d]), int(ys[d]), 0x118, 0xF, 0xC, false));
      yo[d] = uint32_t(__builtin_amdgcn_update_dpp(int(ys[d]), int(xs[d]), 0x108, 0xF, 0x3, false));
    }
    Q[2 * e] = uint4{xo[0], xo[1], xo[2], xo[3]};
    Q[2 * e + 1] = uint4{yo[0], yo[1], yo[2], yo[3]};
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const uint32_t qa[4] = {Q[x].x, Q[x].y, Q[x].z, Q[x].w};
    const uint32_t qb[4] = {Q[2 + x].x, Q[2 + x].y, Q[2 + x].z, Q[2 + x].w};
    uint32_t da[4], db[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // odd 16-lane rows of the first register <-> even rows of the second
      const auto sw = __builtin_amdgcn_permlane16_swap(qa[d], qb[d], false, false);
      da[d] = uint32_t(sw[0]);
      db[d] = uint32_t(sw[1]);
    }
    D[x] = uint4{da[0], da[1], da[2], da[3]};
    D[2 + x] = uint4{db[0], db[1], db[2], db[3]};
  }
}

typedef __attribute__((address_space(3))) void lds_void;
__device__ inline void dma16(__amdgpu_buffer_rsrc_t r, uint8_t *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(lds), 16, voff, soff, 0, 0);
}

inline int cus_of_device() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  return n;
}

}  // namespace
}  // namespace coli
