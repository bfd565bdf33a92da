// tier.cpp -- expert placement: an HBM cache of expert blobs over host memory.
//
// Rules (page "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本",
// section 三, and page "为什么Colibrì越用越快：路由热度学习缓存与专家自动固定机制
// 深度解析", section 实时重固定REPIN): a hot expert replaces a cold one only past
// a hysteresis of 25 % + 4 counts (computed wide, so a saturated 32-bit heat
// stays put); experts are ranked by an LFRU score in which one routing counts
// 256 and recency at most 255; heat halves over time; at most four swaps per
// check.
//
// The cache: S slots in HBM, all E blobs in pinned host memory.  Admission puts
// every expert a batch needs into a slot (a free one, lowest index first, else
// the slot of the resident the batch does not need with the lowest score, ties
// to the lower id); REPIN moves hot non-resident experts in ahead of need.  The
// state is host memory owned by the caller; these functions only plan.  Copies
// (coli_cache_stage, coli_cache_slot_map) go on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "coli.h"

namespace {

constexpr uint32_t kU32 = 0xFFFFFFFFu;

bool state_ok(const coli_cache *c) {
  return c && c->E >= 1 && c->E <= COLI_MAX_EXPERTS && c->S >= 1 && c->S <= c->E && c->heat &&
         c->last && c->slot_of && c->expert_of;
}

uint64_t score_of(const coli_cache *c, int e) {
  return coli_tier_lfru_score(c->heat[e], c->last[e], c->clock);
}

void place(coli_cache *c, int e, int s) {
  const int old = c->expert_of[s];
  if (old >= 0) c->slot_of[old] = -1;
  c->expert_of[s] = e;
  c->slot_of[e] = s;
}

}  // namespace

extern "C" {

int coli_tier_should_promote(uint32_t hot, uint32_t cold) {
  const uint64_t threshold = uint64_t(cold) + (uint64_t(cold) >> 2) + 4u;
  return uint64_t(hot) > threshold ? 1 : 0;
}

uint64_t coli_tier_lfru_score(uint32_t heat, uint32_t last, uint32_t clock) {
  const uint32_t age = clock - last;  // modulo 2^32
  const uint32_t recent = age < 255u ? 255u - age : 0u;
  return (uint64_t(heat) << 8) | recent;
}

int coli_cache_init(coli_cache *c) {
  if (!state_ok(c)) return c ? COLI_ESHAPE : COLI_EINVAL;
  c->clock = 0;
  for (int e = 0; e < c->E; ++e) {
    c->heat[e] = 0;
    c->last[e] = 0;
    c->slot_of[e] = -1;
  }
  for (int s = 0; s < c->S; ++s) c->expert_of[s] = -1;
  return COLI_OK;
}

int coli_cache_decay(coli_cache *c) {
  if (!state_ok(c)) return c ? COLI_ESHAPE : COLI_EINVAL;
  for (int e = 0; e < c->E; ++e) c->heat[e] >>= 1;
  return COLI_OK;
}

int coli_cache_admit(coli_cache *c, const int32_t *needed, int n, int32_t *load_expert,
                     int32_t *load_slot, int *n_loads) {
  if (!c || (!needed && n > 0) || !load_expert || !load_slot || !n_loads) return COLI_EINVAL;
  if (!state_ok(c) || n < 0) return COLI_ESHAPE;
  // the batch's experts, each once, in first-named order; all checked first
  std::vector<int> need;
  std::vector<char> in_need(size_t(c->E), 0);
  for (int i = 0; i < n; ++i) {
    const int e = needed[i];
    if (e < 0 || e >= c->E) return COLI_EINVAL;
    if (!in_need[size_t(e)]) {
      in_need[size_t(e)] = 1;
      need.push_back(e);
    }
  }
  if (int(need.size()) > c->S) return COLI_ESHAPE;  // more than the cache holds
  c->clock += 1u;
  for (int e : need) {
    if (c->heat[e] != kU32) c->heat[e] += 1u;
    c->last[e] = c->clock;
  }
  int nl = 0;
  for (int e : need) {
    if (c->slot_of[e] >= 0) continue;
    int s = -1;
    for (int t = 0; t < c->S && s < 0; ++t)
      if (c->expert_of[t] < 0) s = t;
    if (s < 0) {
      int victim = -1;
      uint64_t vs = 0;
      for (int t = 0; t < c->S; ++t) {
        const int r = c->expert_of[t];
        if (in_need[size_t(r)]) continue;
        const uint64_t sc = score_of(c, r);
        if (victim < 0 || sc < vs || (sc == vs && r < victim)) {
          victim = r;
          vs = sc;
        }
      }
      s = c->slot_of[victim];  // a victim exists: the batch needs at most S experts
    }
    place(c, e, s);
    load_expert[nl] = e;
    load_slot[nl] = s;
    ++nl;
  }
  *n_loads = nl;
  return COLI_OK;
}

int coli_cache_repin(coli_cache *c, int max_swaps, int32_t *load_expert, int32_t *load_slot,
                     int32_t *evicted, int *n_swaps) {
  if (!c || !load_expert || !load_slot || !evicted || !n_swaps) return COLI_EINVAL;
  if (!state_ok(c) || max_swaps < 0) return COLI_ESHAPE;
  // candidates: non-resident, hottest first; residents: coldest first (ties: lower id)
  std::vector<int> hot, cold;
  for (int e = 0; e < c->E; ++e)
    if (c->slot_of[e] < 0) hot.push_back(e);
  for (int s = 0; s < c->S; ++s)
    if (c->expert_of[s] >= 0) cold.push_back(c->expert_of[s]);
  auto hotter = [&](int a, int b) {
    const uint64_t sa = score_of(c, a), sb = score_of(c, b);
    return sa != sb ? sa > sb : a < b;
  };
  auto colder = [&](int a, int b) {
    const uint64_t sa = score_of(c, a), sb = score_of(c, b);
    return sa != sb ? sa < sb : a < b;
  };
  // selection sorts (E <= 1024): the first max_swaps of each order are enough
  const int k = max_swaps < int(hot.size()) ? max_swaps : int(hot.size());
  for (int i = 0; i < k; ++i)
    for (size_t j = size_t(i) + 1; j < hot.size(); ++j)
      if (hotter(hot[j], hot[size_t(i)])) std::swap(hot[j], hot[size_t(i)]);
  const int kc = k < int(cold.size()) ? k : int(cold.size());
  for (int i = 0; i < kc; ++i)
    for (size_t j = size_t(i) + 1; j < cold.size(); ++j)
      if (colder(cold[j], cold[size_t(i)])) std::swap(cold[j], cold[size_t(i)]);
  int ns = 0;
  for (int i = 0; i < kc; ++i) {
    const int h = hot[size_t(i)], cd = cold[size_t(i)];
    if (!coli_tier_should_promote(c->heat[h], c->heat[cd])) break;
    const int s = c->slot_of[cd];
    place(c, h, s);
    load_expert[ns] = h;
    load_slot[ns] = s;
    evicted[ns] = cd;
    ++ns;
  }
  *n_swaps = ns;
  return COLI_OK;
}

int coli_cache_stage(const uint8_t *host_blobs, uint8_t *slots, size_t blob_bytes,
                     const int32_t *load_expert, const int32_t *load_slot, int n_loads,
                     void *stream) {
  if ((!host_blobs || !slots || !load_expert || !load_slot) && n_loads > 0) return COLI_EINVAL;
  if (n_loads < 0 || blob_bytes == 0) return COLI_ESHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < n_loads; ++i) {
    if (load_expert[i] < 0 || load_slot[i] < 0) return COLI_EINVAL;
  }
  for (int i = 0; i < n_loads; ++i) {
    const hipError_t e = hipMemcpyAsync(slots + size_t(load_slot[i]) * blob_bytes,
                                        host_blobs + size_t(load_expert[i]) * blob_bytes,
                                        blob_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return COLI_EDEVICE;
  }
  return COLI_OK;
}

int coli_cache_slot_map(const coli_cache *c, int32_t *slot_map, void *stream) {
  if (!c || !slot_map) return COLI_EINVAL;
  if (!state_ok(c)) return COLI_ESHAPE;
  const hipError_t e = hipMemcpyAsync(slot_map, c->slot_of, sizeof(int32_t) * size_t(c->E),
                                      hipMemcpyHostToDevice,
                                      reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

}  // extern "C"
