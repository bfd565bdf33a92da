// usage.hip -- routing counters and the routing-history file .coli_usage.
//
// Page "colibrì 路由遥测全解析：.coli_usage专家历史、ROUTE_TRACE追踪流与
// route_trace.h统一格式": the engine adds every routing decision (which expert a
// layer chose) to in-memory counters, and writes them back at a safe point as
// a sparse text history (sections 历史文件 and 头部记录为什么长这样): the records
// "-1 n_layers n_experts" and "-2 format_version engine_hash", then one
// "layer expert count" triple per non-zero counter; exactly three numeric
// fields per record (三条铁律); an empty history is a zero-byte file (空历史 =
// 零字节文件); the file is replaced through a temporary file and a rename.
// The reader (可信读取, 仍然兼容读取的旧布局) checks geometry, version and
// identity (trust relaxes identity only), accepts header-less legacy files and
// the dense IKU1 layout of the engine "inkling", skips records it cannot place,
// and reports the total of the accepted counts only.
//
// The counters live on the device: coli_usage_count adds one layer's routing
// (the top-K ids of a forward) with 64-bit integer atomics, so the result is
// exact and independent of the order.  The file functions run on the host.
#include <hip/hip_runtime.h>

#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "coli.h"
#include "kernels.h"

namespace coli {
namespace {

// counts[e] += number of (token, slot) pairs that chose e (ids outside [0, E)
// are not counted).  Per block: an LDS histogram, then one global atomic per
// expert with a non-zero count.
__global__ __launch_bounds__(256) void usage_count_kernel(const int32_t *__restrict__ idx,
                                                          int64_t P, int E,
                                                          unsigned long long *__restrict__ counts) {
  __shared__ unsigned int hist[COLI_MAX_EXPERTS];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0u;
  __syncthreads();
  for (int64_t p = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; p < P;
       p += int64_t(gridDim.x) * blockDim.x) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1u);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    if (hist[e]) atomicAdd(&counts[e], (unsigned long long)hist[e]);
}

constexpr uint32_t kIku1Magic = 0x31554B49u;  // "IKU1", little-endian

uint32_t fnv1a32(const char *s) {
  uint32_t h = 0x811C9DC5u;
  for (; *s; ++s) {
    h ^= uint32_t(uint8_t(*s));
    h *= 0x01000193u;
  }
  return h;
}

// round(c * decay), but a non-zero count never rounds to zero; decay outside
// (0, 1] (or exactly 1) leaves the count as it is
uint64_t decayed(uint64_t c, double decay) {
  if (!(decay > 0.0 && decay < 1.0)) return c;
  const uint64_t v = uint64_t(double(c) * decay + 0.5);
  return (c > 0 && v == 0) ? 1 : v;
}

}  // namespace
}  // namespace coli

using namespace coli;

extern "C" {

int coli_usage_count(const int32_t *topk_idx, int T, int K, int n_experts, int layer,
                     int n_layers, uint64_t *counts, void *stream) {
  if ((!topk_idx && T > 0) || !counts) return COLI_EINVAL;
  if (T < 0 || T > COLI_MAX_TOKENS || K < 1 || K > COLI_MAX_EXPERTS || n_experts < 1 ||
      n_experts > COLI_MAX_EXPERTS || n_layers < 1 || layer < 0 || layer >= n_layers)
    return COLI_ESHAPE;
  if ((reinterpret_cast<uintptr_t>(topk_idx) & 3) || (reinterpret_cast<uintptr_t>(counts) & 7))
    return COLI_EALIGN;
  if (T == 0) return COLI_OK;
  const int64_t P = int64_t(T) * K;
  int64_t blocks = (P + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  usage_count_kernel<<<dim3(unsigned(blocks)), 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      topk_idx, P, n_experts,
      reinterpret_cast<unsigned long long *>(counts) + size_t(layer) * n_experts);
  return hipGetLastError() == hipSuccess ? COLI_OK : COLI_EDEVICE;
}

uint32_t coli_usage_engine_hash(const char *name) { return name ? fnv1a32(name) : 0u; }

int coli_usage_save(const char *path, const uint64_t *counts, int n_layers, int n_experts,
                    uint32_t engine_hash, double decay, const uint8_t *dropped) {
  if (!path || !counts) return COLI_EINVAL;
  if (n_layers < 1 || n_experts < 1 || n_experts > COLI_MAX_EXPERTS) return COLI_ESHAPE;
  // the temporary path is built, and checked, before the file system is touched:
  // a truncated or failed format would write (and rename) a path nobody asked for
  char tmp[4096];
  const int n = std::snprintf(tmp, sizeof tmp, "%s.tmp.%ld", path, long(getpid()));
  if (n < 0 || size_t(n) >= sizeof tmp) return COLI_EINVAL;
  uint64_t total = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (dropped && dropped[l]) continue;
    for (int e = 0; e < n_experts; ++e) total += decayed(counts[size_t(l) * n_experts + e], decay);
  }
  FILE *f = std::fopen(tmp, "wb");
  if (!f) return COLI_EIO;
  bool ok = true;
  if (total > 0) {
    // no record before the first count: an empty history stays a zero-byte file
    ok = std::fprintf(f, "-1 %d %d\n-2 %d %u\n", n_layers, n_experts, COLI_USAGE_VERSION,
                      unsigned(engine_hash)) > 0;
    for (int l = 0; ok && l < n_layers; ++l) {
      if (dropped && dropped[l]) continue;
      for (int e = 0; ok && e < n_experts; ++e) {
        uint64_t c = decayed(counts[size_t(l) * n_experts + e], decay);
        if (!c) continue;
        if (c > 0xFFFFFFFFull) c = 0xFFFFFFFFull;  // the field is read as unsigned 32-bit
        ok = std::fprintf(f, "%d %d %u\n", l, e, unsigned(c)) > 0;
      }
    }
  }
  ok = (std::fflush(f) == 0) && ok && !std::ferror(f);
  ok = (std::fclose(f) == 0) && ok;
  if (!ok || std::rename(tmp, path) != 0) {
    std::remove(tmp);
    return COLI_EIO;
  }
  return COLI_OK;
}

int coli_usage_load(const char *path, uint64_t *counts, int n_layers, int n_experts,
                    uint32_t engine_hash, int trusted, const uint8_t *dropped,
                    uint64_t *accepted_total) {
  if (!path || !counts) return COLI_EINVAL;
  if (n_layers < 1 || n_experts < 1 || n_experts > COLI_MAX_EXPERTS) return COLI_ESHAPE;
  FILE *f = std::fopen(path, "rb");
  if (!f) return COLI_EIO;
  uint64_t total = 0;
  int rc = COLI_OK;
  uint32_t head[3] = {0u, 0u, 0u};
  const size_t got = std::fread(head, 4, 3, f);
  if (got >= 1 && head[0] == kIku1Magic) {
    // dense layout: uint32 {magic, n_layers, n_experts}, uint32 [n_layers][n_experts];
    // read only by inkling, and only with matching geometry
    if (engine_hash != fnv1a32("inkling")) rc = COLI_EUSAGE;
    else if (got < 3 || int64_t(head[1]) != n_layers || int64_t(head[2]) != n_experts)
      rc = COLI_EUSAGE;
    for (int l = 0; rc == COLI_OK && l < n_layers; ++l)
      for (int e = 0; e < n_experts; ++e) {
        uint32_t c = 0;
        if (std::fread(&c, 4, 1, f) != 1) {
          rc = COLI_EUSAGE;
          break;
        }
        if (dropped && dropped[l]) continue;
        counts[size_t(l) * n_experts + e] += c;
        total += c;
      }
  } else {
    std::rewind(f);
    long long a = 0, b = 0, c = 0;
    // three numbers at a time, as every reader of the format loops
    while (rc == COLI_OK && std::fscanf(f, "%lld %lld %lld", &a, &b, &c) == 3) {
      if (a == -1) {
        if (b != n_layers || c != n_experts) rc = COLI_EUSAGE;  // never relaxed
        continue;
      }
      if (a == -2) {
        if (b != COLI_USAGE_VERSION) rc = COLI_EUSAGE;  // never relaxed
        else if (uint32_t(c) != engine_hash && !trusted) rc = COLI_EUSAGE;
        continue;
      }
      if (a < 0) continue;  // a record type this reader does not know
      if (a >= n_layers || b < 0 || b >= n_experts || c < 0) continue;
      if (dropped && dropped[a]) continue;
      counts[size_t(a) * n_experts + size_t(b)] += uint64_t(c);
      total += uint64_t(c);
    }
  }
  std::fclose(f);
  if (accepted_total) *accepted_total = rc == COLI_OK ? total : 0;
  return rc;
}

}  // extern "C"
