// ffn_narrow.hip -- the routed + shared expert FFN of one decode token:
// int4-g64 planar weights streamed from HBM straight into int8 matrix-core
// products.
//
// Method: page "从源码开始colibri纯C引擎的编译、权重转换与.bin直映射实战",
// section 权重转换 -- the expert FFN reads the planar bytes as they are (byte k
// of a 64-group: element k low nibble, element k+32 high nibble, u = q + 8;
// weight = s * (u - 8)); SiLU(gate) * up, then down, then the gate-weighted
// sum over the selected experts plus the shared expert (page "Colibrì 深度解析",
// sections 四 and 十一).  The token's top-K runs inside the gate/up kernel.
//
// Arithmetic.  An activation vector a is held in fixed point, a = A * 2^-e
// with one power-of-two scale per vector and |A| <= 2^27, and A is split into
// four balanced base-128 digits, A = d0 2^21 + d1 2^14 + d2 2^7 + d3, each in
// [-64, 64] (int8).  A weight nibble u (0..15) is already an int8, so the
// v_mfma_i32_16x16x64_i8 sum over a group, sum_k d_k u_k, is exact in int32;
// the format's -8 enters as the accumulator's initial value, -8 * sum_k d_k,
// stored with the digits.  Per group the four plane sums are recombined
// exactly in int32 pairs, rounded once to fp32 and scaled by the fp32 group
// scale.  Every element within a factor 16 of the vector's largest is
// represented exactly, smaller ones to 2^-28 of it: the products are at least
// as accurate as an fp32 dot product.  The unpack costs 3 32-bit operations
// per 8 weights.  The down kernel digitises h' itself, in unbalanced digits
// (d1..d3 in [0, 127], d0 = A >> 21 in [-64, 64]: one bit-field extract each),
// and forms its -8 * sum_k d_k with two more products against a B operand of
// -8 bytes; every plane sum stays below 2^16 in magnitude, so the recombined
// value is the same exact integer and rounds the same way.
//
// MFMA layout (16x16x64 i8: lane l holds A row / B column l % 16 and 16
// bytes of k for the k-quarter l / 16; the result lane l holds rows
// 4*(l/16)+i, column l % 16).  One token leaves 15 of 16 A rows free; they
// carry work instead.  A row m = 4 s + p is digit plane p of slot s, and slot
// s = (kappa, j) = (s / 2, s % 2) names one of four groups.  B column
// n = r + 8 kappa is weight row r of an 8-row fragment, and its lane quarter q
// loads bytes 16 (q % 2) .. +15 of group 4c + 2 kappa + q / 2 (so the 8 lanes
// of a row read one contiguous 128-byte run: groups 4c .. 4c+3).  A row m is
// zero in the k-quarters whose group is not its slot's (q / 2 != j), so result
// row 4 s + p of column n is the plane-p sum over group 4c + 2 kappa_s + j_s
// of weight row r: meaningful where kappa_s = kappa(n), ignored elsewhere.
// Each 16-byte lane load feeds two MFMAs, one per 8-byte half.
//
// Digit runs ("A order"): the 64 digits of a (vector, group, plane) are four
// 16-byte runs; run rho holds the digits of elements 8 rho .. 8 rho + 7, then
// 32 + 8 rho .. 32 + 8 rho + 7 -- the k order of the B half that holds group
// bytes 8 rho .. 8 rho + 7 after the unpack {d0 & M, d1 & M, (d0 >> 4) & M,
// (d1 >> 4) & M}, M = 0x0F0F0F0F (d0, d1 = the half's two dwords).
//
// Kernels
//   gateup_narrow  persistent; item = (unit, 8 rows of I): a gate and an up
//                  fragment.  The block's waves split the K groups; each wave
//                  keeps the x digits of its K slice in registers for the
//                  whole launch and a register ring one item deep of weight
//                  loads.  Partials meet in LDS; one wave (rotating) writes
//                  h' = gate_weight * SiLU(gate) * up in fp32.
//   down_narrow    persistent, output-stationary; item = 8 rows of y, all
//                  units.  Wave w owns K chunk w (256 columns of I) of every
//                  unit and streams (item, unit) steps through a register
//                  ring two units deep; it turns unit u + 1's slice of h'
//                  into digits in its own LDS area during step u, while the
//                  weights are in flight.  The gates sit in h', so the combine
//                  is the accumulation itself, in a fixed order (no atomics).
#include <hip/hip_ext.h>

#include <atomic>

#include "kernels.h"
#include "wave.h"

namespace coli {
namespace {

constexpr int kW = 64;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ inline i32x4 mfma_i8(const i32x4 &a, const i32x4 &b, const i32x4 &c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// The B operand of one 8-byte half (dwords d0, d1 = bytes 8h .. 8h+7 of a
// lane's 16): low nibbles of the 8 bytes, then high nibbles.
__device__ inline i32x4 unpack_half(uint32_t d0, uint32_t d1) {
  const uint32_t M = 0x0F0F0F0Fu;
  return i32x4{int(d0 & M), int(d1 & M), int((d0 >> 4) & M), int((d1 >> 4) & M)};
}

// Plane sums r0..r3 (|r| < 2^17) -> one fp32 value
// (r0 2^7 + r1) 2^14 + (r2 2^7 + r3); both halves are exact in fp32.
__device__ inline float planes_to_f32(const i32x4 &r) {
  const int hi = r[0] * 128 + r[1];
  const int lo = r[2] * 128 + r[3];
  return fmaf(float(hi), 16384.0f, float(lo));
}

template <int kCtrl>
__device__ inline float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
// A register copy the compiler cannot fold away: the copy is made now, so the
// source register is free for the slot's next load.
__device__ inline float keep(float v) {
  float o;
  asm volatile("v_mov_b32 %0, %1" : "=v"(o) : "v"(v));
  return o;
}

// s_waitcnt vmcnt(0) as an instruction the compiler's wait tracking sees: after
// it nothing is pending, so loads issued before a loop in an order the loop
// does not follow cannot leave the loop waiting for all of them every trip.
__device__ inline void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Step boundary of a ring: nothing is scheduled across it.  The refills must
// leave in the order their slots are consumed and no slot may be touched
// before its turn (the load counter retires in issue order, so an early use
// of a late slot waits for nearly every load in flight).
__device__ inline void step_fence() { __builtin_amdgcn_sched_barrier(0); }

// Barrier for LDS traffic only: vector-memory loads stay in flight.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Result lanes whose slot belongs to the lane's column (kappa_s = kappa(n)).
__device__ inline bool result_valid(int lane) { return ((lane / 16) >> 1) == ((lane % 16) >> 3); }

// Per-row total of a result value over the valid lanes of the wave: lane r
// (r < 8) receives the sum for fragment row r.
__device__ inline float fold_rows(float v, int lane) {
  v = result_valid(lane) ? v : 0.0f;
  v += dpp_row<0x128>(v);  // row_ror:8 -- columns r and r + 8
  v += __shfl_xor(v, 16, kW);
  v += __shfl_xor(v, 32, kW);
  return v;
}

// Plane p of four fixed-point values a_i (|a_i| <= 2^27) packed one byte per
// value, in base-128 digits a = d0 2^21 + d1 2^14 + d2 2^7 + d3 with
// d1..d3 in [0, 127] and d0 = a >> 21 in [-64, 64].
__device__ inline uint32_t pack_digits(const int (&a)[4], int p) {
  const uint32_t pos = p == 0 ? 21u : 7u * uint32_t(3 - p), w = p == 0 ? 8u : 7u;
  uint32_t r = __builtin_amdgcn_ubfe(uint32_t(a[0]), pos, w);
  r |= __builtin_amdgcn_ubfe(uint32_t(a[1]), pos, w) << 8;
  r |= __builtin_amdgcn_ubfe(uint32_t(a[2]), pos, w) << 16;
  return r | (__builtin_amdgcn_ubfe(uint32_t(a[3]), pos, w) << 24);
}

// ------------------------------------------------------------------ gate/up
constexpr int kMaxWaves = 16;
constexpr int kGateupMaxWaves = 8;
constexpr int kMaxItems = 8;  // items per block (the grid is sized for it)
constexpr int kGateupItems = COLI_NARROW_MAX_K + 1;  // one per unit

template <int NC>
__global__ __launch_bounds__(kW * 8) __attribute__((amdgpu_waves_per_eu(2)))
void gateup_narrow(NarrowBufs nb, LayerDev L, const float *__restrict__ logits,
                   int32_t *__restrict__ idx_out, float *__restrict__ gate_out, int pre_routed) {
  __shared__ int32_t sidx[COLI_NARROW_MAX_K];
  __shared__ int32_t sslot[COLI_NARROW_MAX_K];  // with a slot map: the experts' slots (-1: none)
  __shared__ float sgate[COLI_NARROW_MAX_K];
  __shared__ float red[kGateupItems][kGateupMaxWaves][2][8];
  // per wave, double-buffered: the item's group scales [frag][4 NC groups][8 rows]
  __shared__ __align__(16) float ssc[kGateupMaxWaves][2][2][32 * NC];
  const int lane = threadIdx.x % kW, wave = threadIdx.x / kW;
  const int nw = blockDim.x / kW;
  const int I = L.I, E = L.E, K = L.K;
  const int GH = int(L.lay.GH);
  const int nrb = I / 8;
  const int n_items = (K + 1) * nrb;
  if (int(blockIdx.x) >= n_items) return;


  const int n = lane % 16, q = lane / 16;
  const int r = n % 8, kap = n / 8;
  // x digits of this wave's K slice (chunks wave*NC .. +NC-1), A rows
  const int sA = n / 4, pA = n % 4;  // A row n: slot sA, plane pA
  const int ksA = sA / 2, jsA = sA % 2;
  const bool actA = (q / 2) == jsA;
  const int rho0 = 2 * (q % 2);
  i32x4 A[NC][2], C[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int g0 = 4 * (wave * NC + c);
    const int8_t *base = nb.xdig + (size_t(g0 + 2 * ksA + jsA) * 4 + pA) * 64 + 16 * rho0;
    const i32x4 z = {0, 0, 0, 0};
    A[c][0] = actA ? *reinterpret_cast<const i32x4 *>(base) : z;
    A[c][1] = actA ? *reinterpret_cast<const i32x4 *>(base + 16) : z;
    C[c] = *reinterpret_cast<const i32x4 *>(nb.xcorr + size_t(g0 + q) * 4);
  }
  const float xs = nb.xsc[0];

  // item -> this lane's weight pointers (chunk 0 of its K slice; B lane group
  // 4c + 2 kappa + q / 2) and its scale run.  The item's scales of the K slice
  // are one contiguous run of 8 NC float4 in the 8-row blocked copy
  // ([group][row]); lane l < 8 NC loads float4 l of it (the others re-load
  // float4 0 and keep it).
  const size_t goff = size_t(wave) * NC * 4 + 2 * kap + q / 2;
  const int sl = lane < 8 * NC ? lane : 0;
  const size_t soff = size_t(wave) * NC * 4 * 8 + 4 * size_t(sl);
  struct Ptrs {
    const uint8_t *wg, *wu;
    const float *sg, *su;
  };
  // item it = (v, rb): unit v (0 = the shared expert, v >= 1 the routed
  // expert sidx[v - 1]), rows 8 rb .. 8 rb + 7 of I
  // the blob of unit v (an expert without a slot reads the shared blob: valid
  // memory, its h' rows are poisoned below)
  auto unit_blob = [&](int v) {
    if (v == 0) return L.shared;
    const int sl = L.slot_map ? sslot[v - 1] : sidx[v - 1];
    return sl < 0 ? L.shared : L.experts + size_t(sl) * L.lay.bytes;
  };
  auto ptrs = [&](int it) {
    const int v = it / nrb, rb = it - v * nrb;
    const uint8_t *blob = unit_blob(v);
    const size_t row = size_t(rb) * 8 + r;
    Ptrs p;
    p.wg = blob + L.lay.gq + (row * GH + goff) * 32 + 16 * (q % 2);
    p.wu = blob + L.lay.uq + (row * GH + goff) * 32 + 16 * (q % 2);
    p.sg = reinterpret_cast<const float *>(blob + L.lay.gsB) + size_t(rb) * GH * 8 + soff;
    p.su = reinterpret_cast<const float *>(blob + L.lay.usB) + size_t(rb) * GH * 8 + soff;
    return p;
  };

  // the token's logits first: the top-K below then waits for them alone, not
  // for the weight loads issued after them
  float lg[4];
  if (wave == 0 && !pre_routed) topk_load<4>(logits, E, lane, lg);
  uint4 rw[2][NC];
  float4 scg, scu;
  int it = blockIdx.x;
  {
    const Ptrs p = ptrs(it);
    scg = *reinterpret_cast<const float4 *>(p.sg);
    scu = *reinterpret_cast<const float4 *>(p.su);
#pragma unroll
    for (int c = 0; c < NC; ++c) rw[0][c] = *reinterpret_cast<const uint4 *>(p.wg + 128 * c);
#pragma unroll
    for (int c = 0; c < NC; ++c) rw[1][c] = *reinterpret_cast<const uint4 *>(p.wu + 128 * c);
  }
  // The first item is the shared expert's (the grid is I / 8 blocks), so its
  // loads are in flight while wave 0 picks the token's experts.
  if (pre_routed) {
    // the token's top-K was selected beforehand (two-phase forward)
    if (int(threadIdx.x) < K) {
      sidx[threadIdx.x] = idx_out[threadIdx.x];
      sgate[threadIdx.x] = gate_out[threadIdx.x];
    }
  } else if (wave == 0) {
    topk_select<4>(lg, E, K, lane, sidx, sgate, L.sc);
  }
  lds_barrier();
  if (L.slot_map) {
    // the selected experts' slots, looked up once (not per item: a global load
    // inside the item loop would drain the weight ring every trip)
    if (int(threadIdx.x) < K) sslot[threadIdx.x] = L.slot_map[sidx[threadIdx.x]];
    lds_barrier();
  }
  if (!pre_routed && blockIdx.x == 0 && int(threadIdx.x) < K) {
    idx_out[threadIdx.x] = sidx[threadIdx.x];
    gate_out[threadIdx.x] = sgate[threadIdx.x];
    // the routing history: one decision per selected expert
    if (L.usage) atomicAdd(L.usage + sidx[threadIdx.x], 1ull);
  }
  wait_all_loads();
  int buf = 0, k_it = 0;
  for (; it < n_items; it += gridDim.x, ++k_it) {
    // the next item's loads replace each slot as it is consumed; past the
    // end they re-read the current item (valid addresses, never used)
    const int nx = it + int(gridDim.x) < n_items ? it + int(gridDim.x) : it;
    const Ptrs np = ptrs(nx);
    // this item's scales -> LDS, then the next item's scale loads
    if (lane < 8 * NC) {
      *reinterpret_cast<float4 *>(&ssc[wave][buf][0][4 * lane]) = scg;
      *reinterpret_cast<float4 *>(&ssc[wave][buf][1][4 * lane]) = scu;
    }
    scg = *reinterpret_cast<const float4 *>(np.sg);
    scu = *reinterpret_cast<const float4 *>(np.su);
    step_fence();
    float sv[2][NC];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int c = 0; c < NC; ++c) sv[f][c] = ssc[wave][buf][f][(4 * c + q) * 8 + r];
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        // consume the slot before its refill is issued (the refill can then
        // land in the same registers: no copies around the loop)
        const i32x4 b0 = unpack_half(rw[f][c].x, rw[f][c].y);
        const i32x4 b1 = unpack_half(rw[f][c].z, rw[f][c].w);
        rw[f][c] = *reinterpret_cast<const uint4 *>((f ? np.wu : np.wg) + 128 * c);
        step_fence();
        i32x4 P = mfma_i8(A[c][0], b0, C[c]);
        P = mfma_i8(A[c][1], b1, P);
        acc[f] = fmaf(planes_to_f32(P), sv[f][c], acc[f]);
      }
    // per-row partials of this wave; the block reduces them once, at the end
    const float vg = fold_rows(acc[0], lane);
    const float vu = fold_rows(acc[1], lane);
    if (lane < 8) {
      red[k_it][wave][0][lane] = vg;
      red[k_it][wave][1][lane] = vu;
    }
    buf ^= 1;
  }
  lds_barrier();
  for (int i = threadIdx.x; i < k_it * 8; i += blockDim.x) {
    const int k = i / 8, rr = i % 8;
    float g = 0.0f, up = 0.0f;
    for (int w = 0; w < nw; ++w) {
      g += red[k][w][0][rr];
      up += red[k][w][1][rr];
    }
    const int itk = int(blockIdx.x) + k * int(gridDim.x);
    const int v = itk / nrb, rb = itk - v * nrb;
    const int u = v > 0 ? v - 1 : K;  // h' rows: routed units in top-K order, shared last
    const float gw = v > 0 ? sgate[v - 1] : 1.0f;
    // a blob without the finish tag has no valid blocked scales: its h' rows
    // become NaN (and so does y) and the status flag says why
    const bool miss = v > 0 && L.slot_map && sslot[v - 1] < 0;
    const uint8_t *blob = unit_blob(v);
    const uint4 tg = *reinterpret_cast<const uint4 *>(blob + L.lay.tag);
    const bool untagged = tg.x != L.tag.x || tg.y != L.tag.y || tg.z != L.tag.z || tg.w != L.tag.w;
    const bool bad = untagged || miss;
    if (rr == 0 && untagged && !miss) raise_status(L.status, COLI_STATUS_UNFINISHED);
    if (rr == 0 && miss) raise_status(L.status, COLI_STATUS_NOT_RESIDENT);
    nb.hn[size_t(u) * I + rb * 8 + rr] =
        bad ? __builtin_nanf("") : gw * silu(g * xs) * (up * xs);
  }
}

// ------------------------------------------------------------------ down
// Per-wave LDS area: digits [NU][4 planes][4 groups][64], then 32 zero bytes
// (the A rows of inactive k-quarters read them).
template <int NU>
constexpr int down_wave_bytes() { return NU * 1024 + 32; }

constexpr int kDownMaxWaves = 8;
constexpr int kDownItems = 3;  // items per down block

template <int NU>
__global__ __launch_bounds__(kW * kDownMaxWaves) void down_narrow(NarrowBufs nb, LayerDev L,
                                                             const int32_t *__restrict__ idx,
                                                             float *__restrict__ y) {
  extern __shared__ __align__(16) uint8_t dyn[];
  __shared__ float red[kMaxItems][kDownMaxWaves][8];
  const int lane = threadIdx.x % kW, wave = threadIdx.x / kW;
  const int nw = blockDim.x / kW;
  const int H = L.H, I = L.I, K = L.K;
  const int GI = int(L.lay.GI);
  const int n_items = H / 8;
  if (int(blockIdx.x) >= n_items) return;
  uint8_t *my = dyn + wave * down_wave_bytes<NU>();
  int8_t *dig = reinterpret_cast<int8_t *>(my);
  uint8_t *zero = my + NU * 1024;

  const int n = lane % 16, q = lane / 16;
  const int r = n % 8, kap = n / 8;
  const uint8_t *blob[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    // an expert without a slot reads the shared blob in its place; its h' rows
    // are NaN already (the gate/up kernel poisoned them)
    bool miss = false;
    blob[u] = u < K ? expert_blob(L, idx[u], miss) : L.shared;
  }

  // weights: the B lane's group (4 wave + 2 kappa + q / 2); scale: the result
  // lane's slot (group 4 wave + q), from the 8-row blocked copy, where a
  // wave's 4 groups of an item are one 128-byte line
  const size_t goff = size_t(wave) * 4 + 2 * kap + q / 2;
  const size_t soff = size_t(wave) * 4 + q;
  auto loff = [&](int it) { return (size_t(it) * 8 + r) * GI + goff; };
  auto sof = [&](int it) { return (size_t(it) * GI + soff) * 8 + r; };
  // Unit-major streaming: the block's items (at most kDownItems: b, b + G,
  // b + 2G) are visited unit by unit, so that at any time the whole grid reads
  // the rows of one or two experts (row-buffer locality).  Ring: the slots of
  // two units (A: even units, B: odd), refilled with the unit two ahead.
  const int G = gridDim.x;
  const int nib = (n_items - int(blockIdx.x) + G - 1) / G;  // items of this block
  size_t lo[kDownItems], so[kDownItems];
#pragma unroll
  for (int k = 0; k < kDownItems; ++k) {
    // items past the end re-read item 0's rows (cached, never stored)
    const int itk = k < nib ? int(blockIdx.x) + k * G : int(blockIdx.x);
    lo[k] = loff(itk) * 32 + 16 * (q % 2);
    so[k] = sof(itk);
  }
  // h' chunk `wave` of unit u.  Lane l holds elements 4l .. 4l+3 of the
  // chunk: group l / 16, element 4 (l % 16).  Units 0..2 are loaded before
  // the weight ring, unit u + 3 at the start of step u, ahead of that step's
  // refills: the load counter retires in issue order, so waiting for a unit's
  // h' never waits for weights that are not yet due.
  float4 hv[NU];
  auto load_h = [&](int u) {
    hv[u] = *reinterpret_cast<const float4 *>(nb.hn + size_t(u) * I + 256 * wave + 4 * lane);
  };
#pragma unroll
  for (int u = 0; u < 3 && u < NU; ++u) load_h(u);
  uint4 rw[2][kDownItems];
  float rs[2][kDownItems];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int k = 0; k < kDownItems; ++k) {
      const int u = h < NU ? h : NU - 1;
      rw[h][k] = *reinterpret_cast<const uint4 *>(blob[u] + L.lay.dq + lo[k]);
      rs[h][k] = reinterpret_cast<const float *>(blob[u] + L.lay.dsB)[so[k]];
    }
  if (lane < 8) reinterpret_cast<uint32_t *>(zero)[lane] = 0u;

  // unit u's slice of h' -> digits in this wave's LDS area.  Unit 0 goes
  // before the stream starts; unit u + 1 during step u, while unit u's
  // weights are still in flight.
  float sa[NU];
  const int gl = lane / 16, pos = aorder_pos(4 * (lane % 16));
  auto digitise = [&](int u) {
    const float v[4] = {hv[u].x, hv[u].y, hv[u].z, hv[u].w};
    // max |v| on the bit patterns: NaN > Inf > every finite value
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    mb = wave_max_u32(mb);
    const int e = digit_exponent(__uint_as_float(mb));
    sa[u] = mb >= 0x7F800000u ? __builtin_nanf("") : ldexpf(1.0f, -e);
    int a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = int(rintf(fminf(fmaxf(ldexpf(v[i], e), -134217728.0f), 134217728.0f)));
#pragma unroll
    for (int p = 0; p < 4; ++p)
      *reinterpret_cast<uint32_t *>(dig + ((u * 4 + p) * 4 + gl) * 64 + pos) = pack_digits(a, p);
  };
  // the wave's own LDS writes, visible to its reads that follow
  auto lds_wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  };
  digitise(0);

  // A-row LDS addresses (inactive k-quarters read the zero bytes) and the
  // correction of the result lane's slot (group q of the chunk)
  const int sA = n / 4, pA = n % 4;
  const bool actA = (q / 2) == (sA % 2);
  const int gA = 2 * (sA / 2) + (sA % 2);
  const int a_base = actA ? ((pA * 4 + gA) * 64 + 16 * (2 * (q % 2))) : NU * 1024;
  // B operand of the correction products: -8 in every byte
  const i32x4 m8 = {int(0xF8F8F8F8u), int(0xF8F8F8F8u), int(0xF8F8F8F8u), int(0xF8F8F8F8u)};
  const i32x4 z4 = {0, 0, 0, 0};
  const int a_step = actA ? 1024 : 0;

  float acc[kDownItems];
#pragma unroll
  for (int k = 0; k < kDownItems; ++k) acc[k] = 0.0f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int h = u & 1;
    const int un = u + 2 < NU ? u + 2 : NU - 1;  // refill: two units ahead
    if (u + 3 < NU) load_h(u + 3);
    if (u + 1 < NU) digitise(u + 1);
    lds_wave_sync();
    const int8_t *ap = dig + a_base + u * a_step;
    const i32x4 a0 = *reinterpret_cast<const i32x4 *>(ap);
    const i32x4 a1 = *reinterpret_cast<const i32x4 *>(ap + 16);
    // -8 times each A row's digit sum, in the result layout: the accumulator
    // start of every item of this unit
    const i32x4 c0 = mfma_i8(a1, m8, mfma_i8(a0, m8, z4));
#pragma unroll
    for (int k = 0; k < kDownItems; ++k) {
      const i32x4 b0 = unpack_half(rw[h][k].x, rw[h][k].y);
      const i32x4 b1 = unpack_half(rw[h][k].z, rw[h][k].w);
      const float sv = keep(rs[h][k]) * sa[u];
      rw[h][k] = *reinterpret_cast<const uint4 *>(blob[un] + L.lay.dq + lo[k]);
      rs[h][k] = reinterpret_cast<const float *>(blob[un] + L.lay.dsB)[so[k]];
      step_fence();
      i32x4 P = mfma_i8(a0, b0, c0);
      P = mfma_i8(a1, b1, P);
      acc[k] = fmaf(planes_to_f32(P), sv, acc[k]);
    }
  }
  const int k_it = nib;
#pragma unroll
  for (int k = 0; k < kDownItems; ++k) {
    const float v = fold_rows(acc[k], lane);
    if (k < nib && lane < 8) red[k][wave][lane] = v;
  }
  lds_barrier();
  bool bad = false;
  for (int i = threadIdx.x; i < k_it * 8; i += blockDim.x) {
    const int k = i / 8, rr = i % 8;
    float t = 0.0f;
    for (int w = 0; w < nw; ++w) t += red[k][w][rr];
    y[(size_t(blockIdx.x) + size_t(k) * gridDim.x) * 8 + rr] = t;
    bad |= !__builtin_isfinite(t);
  }
  if (__any(bad) && lane == 0) raise_status(L.status, COLI_STATUS_NONFINITE);
}

int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  return n;
}

// Waves splitting the gate/up K groups: NCH = H / 256 chunks, NC = NCH / waves
// chunks per wave (1..6).
int gateup_waves(int H, int *nc) {
  const int nch = H / 256;
  const int pref[] = {8, 4, 2, 1};
  for (int w : pref)
    if (nch % w == 0 && nch / w >= 1 && nch / w <= 6) {
      *nc = nch / w;
      return w;
    }
  return 0;
}

template <int NU>
hipError_t launch_down(const LayerDev &L, const NarrowBufs &nb, const int32_t *idx, float *y,
                       int grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  const int nw = L.I / 256;
  const size_t lds = size_t(nw) * down_wave_bytes<NU>();
  // the kernel's dynamic-LDS limit, raised once per device to what the largest
  // block (kDownMaxWaves waves) needs (function attributes are per device)
  static std::atomic<uint64_t> done{0};
  int dev = -1;
  const bool known = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
  const uint64_t bit = known ? (uint64_t(1) << dev) : 0;
  if (!known || !(done.load(std::memory_order_relaxed) & bit)) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&down_narrow<NU>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(kDownMaxWaves * down_wave_bytes<NU>()));
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_relaxed);
  }
  hipExtLaunchKernelGGL(down_narrow<NU>, dim3(grid), dim3(nw * kW), uint32_t(lds), s, start, stop,
                        0, nb, L, idx, y);
  return hipGetLastError();
}

}  // namespace

bool narrow_supported(const LayerDev &L, int T) {
  if (T != 1 || L.H % 256 || L.I % 256 || L.K > COLI_NARROW_MAX_K || L.E > 256) return false;
  int nc = 0;
  if (!gateup_waves(L.H, &nc)) return false;
  const int nw = L.I / 256;
  if (nw > kDownMaxWaves) return false;
  const size_t lds = size_t(nw) * size_t((L.K + 1) * 1024 + 32);
  return lds + sizeof(float) * 2 * kMaxWaves * 8 <= 160 * 1024;
}

hipError_t launch_ffn_narrow(const LayerDev &L, const NarrowBufs &nb, const float *logits,
                             int32_t *idx, float *gates, float *y, hipStream_t s,
                             hipEvent_t *ev, bool pre_routed) {
  const int cus = cu_count();
  int nc = 0;
  const int gw = gateup_waves(L.H, &nc);
  const int n_items = (L.K + 1) * (L.I / 8);
  // block b: row block b of every unit (unit-major in time, shared first)
  const int ggrid = L.I / 8;
  hipEvent_t e0 = ev ? ev[0] : nullptr, e1 = ev ? ev[1] : nullptr;
  hipEvent_t e2 = ev ? ev[2] : nullptr, e3 = ev ? ev[3] : nullptr;
#define COLI_GU(NC)                                                                      \
  case NC:                                                                               \
    hipExtLaunchKernelGGL(gateup_narrow<NC>, dim3(ggrid), dim3(gw * kW), 0, s, e0, e1, 0, nb, L, \
                          logits, idx, gates, int(pre_routed));                          \
    break;
  switch (nc) {
    COLI_GU(1) COLI_GU(2) COLI_GU(3) COLI_GU(4) COLI_GU(5) COLI_GU(6)
    default: return hipErrorInvalidValue;
  }
#undef COLI_GU
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int d_items = L.H / 8;
  int dgrid = d_items < cus ? d_items : cus;
  if (dgrid < (d_items + kDownItems - 1) / kDownItems) dgrid = (d_items + kDownItems - 1) / kDownItems;
#define COLI_DN(NU) \
  case NU: e = launch_down<NU>(L, nb, idx, y, dgrid, s, e2, e3); break;
  switch (L.K + 1) {
    COLI_DN(2) COLI_DN(3) COLI_DN(4) COLI_DN(5) COLI_DN(6) COLI_DN(7) COLI_DN(8) COLI_DN(9)
    COLI_DN(10) COLI_DN(11) COLI_DN(12) COLI_DN(13) COLI_DN(14) COLI_DN(15) COLI_DN(16)
    COLI_DN(17)
    default: return hipErrorInvalidValue;
  }
#undef COLI_DN
  return e;
}

}  // namespace coli
