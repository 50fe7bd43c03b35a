// Load-time TQ4_1S -> int8 block transcode and the int8 decode GEMV on gfx950.
//
// TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160), the note under
// the decode-speed summary, the paragraph on why CUDA differs, and the
// backend item of "适用前提与边界": converting TQ4_1S tensors to q8_0 when the
// model is loaded keeps the TQ4_1S file size and runs decode at the speed of
// the q8_0 path.  q8_0 is read as 32-element blocks of int8 codes with one
// fp16 scale (block amax / 127); the layout here is codes int8 [N][K] and
// scales fp16 [N][K/32], 1.0625 bytes per weight.
//
// Transcode, one thread per block, float32 order fixed so that a CPU
// reference reproduces the codes bit for bit:
//   q_i = fl(d_h * c[idx_i]); u = FWHT32(q) (stages h = 1, 2, 4, 8, 16);
//   w_i = D_i * fl(u_i * fl(1/sqrt 32)); amax = max |w_i|;
//   d = fp16_rne_sat(fl(amax / 127)); code_i = clamp(rint(fl(w_i / d)), +-127)
// (correctly rounded division, ties to even, d = 0 -> 0).  FMA contraction
// would change these roundings, so it is off in this file.
//
// GEMV: y_n = sum_b d[n, b] dx[b] sum_i code[n, b, i] xq[b, i], where the
// activation is quantized once per workgroup the same way (dx = fl(amax_x /
// 127) kept in float32), so each block's dot product is an exact integer:
// eight v_dot4_i32_i8 per 32 weights, then one conversion and two float32
// operations -- about 12 VALU ops per 32 weights, so the kernel streams its
// 1.0625 bytes per weight at the HBM bound with the VALU mostly idle.
// Structure as in the fused TQ4_1S GEMV: lane k of a row slot owns block k
// (TK = 64 * ceil(nb / 64) lanes per slot), one persistent 1024-thread
// workgroup per CU walks row tiles with the next tile's loads in flight, and
// rows split over several wavefronts meet in an LDS ring combined every
// kRing tiles.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "tq_internal.hpp"
#include "tq_codes.hpp"

namespace tq {
namespace {

constexpr int kTcThreads = 256;

__global__ __launch_bounds__(kTcThreads) void q8_transcode_kernel(const uint4* __restrict__ packed,
                                                                  const uint32_t* __restrict__ scales,
                                                                  uint32_t total, uint32_t mask, Codebook cb,
                                                                  uint4* __restrict__ codes,
                                                                  uint16_t* __restrict__ qscales) {
  __shared__ float lut[16];
  stage_centroids(cb, lut);
  __syncthreads();
  const uint32_t g = blockIdx.x * kTcThreads + threadIdx.x;
  if (g >= total) return;
  const uint4 p = packed[g];
  const uint32_t sc = scales[g];
  const float d0 = f16_bits_to_f32(sc & 0xffffu);
  const float d1 = f16_bits_to_f32(sc >> 16);
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = (i < 16 ? d0 : d1) * lut[(w[i >> 3] >> (4 * (i & 7))) & 15u];
  fwht32(v);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = v[i] * kInvSqrt32;
  apply_signs(v, mask);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t dbits = f16_sat(amax / 127.0f);
  const float dd = f16_bits_to_f32(dbits);
  const float r = __builtin_amdgcn_rcpf(dd);
  uint32_t out[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) out[i >> 2] |= q8_code(v[i], dd, r) << (8 * (i & 3));
  codes[2 * (size_t)g] = make_uint4(out[0], out[1], out[2], out[3]);
  codes[2 * (size_t)g + 1] = make_uint4(out[4], out[5], out[6], out[7]);
  qscales[g] = (uint16_t)dbits;
}

// ---------------------------------------------------------------------------
// int8 GEMV
// ---------------------------------------------------------------------------

constexpr int kMaxK = 32768;      // one block per lane, a row slot at most 1024 lanes
constexpr int kRing = 32;         // tiles whose cross-wavefront partial sums wait in LDS

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum of v over the 64 lanes, in lane 0 (and every lane): permlane swaps
// fold the halves and quarters, DPP row rotations and quad permutes the rest.
__device__ __forceinline__ float wave_sum(float v) {
  float a = v, b = v;
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  a = v;
  b = v;
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  v += dpp_f<0x128>(v);            // row_ror 8
  v += dpp_f<0x124>(v);            // row_ror 4
  v += dpp_f<0x4E>(v);             // quad_perm [2,3,0,1]
  v += dpp_f<0xB1>(v);             // quad_perm [1,0,3,2]
  return v;
}

// Maximum of v over the 8 consecutive lanes that hold one activation block.
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  return fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F)));   // lane ^ 4
}

struct Q8Grid {
  int TK;             // lanes per row slot (multiple of 64)
  int S;              // row slots per workgroup
  uint32_t slot_mul;  // slot of wavefront w = (w * slot_mul) >> 8
  uint32_t G;         // workgroups
  uint32_t q, r;      // workgroup g owns tiles g, g + G, ...: q + (g < r) of them
};

struct Q8Raw {
  uint4 a, b;         // the block's 32 int8 codes
  uint32_t s;         // its fp16 scale (low half)
};

// kP: groups of 4 activation elements each thread quantizes (K <= 4 kP nthreads).
template <bool kXbf16, int kP>
__global__ __launch_bounds__(1024) void q8_gemv_kernel(const uint4* __restrict__ codes,
                                                       const uint16_t* __restrict__ qscales, uint32_t N, uint32_t nb,
                                                       const uint8_t* __restrict__ x, float* __restrict__ y,
                                                       Q8Grid gg) {
  __shared__ __attribute__((aligned(16))) uint32_t xq[kMaxK / 4];   // activation codes, 4 per word
  __shared__ float xs[kMaxK / 32];                                   // activation block scales
  __shared__ float red[kRing][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int TK = gg.TK, S = gg.S, nthreads = S * TK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = (int)(((uint32_t)wave * gg.slot_mul) >> 8);
  const int lk = tid - slot * TK;
  const int wk = lk >> 6;
  const int WK = TK >> 6;
  const uint32_t K = nb * 32u;

  // Activation loads first (coalesced: thread t takes elements 4 (t + p nthreads) ..),
  // then the first two tiles' weights.
  uint32_t raw[kP][kXbf16 ? 2 : 4];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const uint32_t e0 = min(4u * (uint32_t)(tid + p * nthreads), K - 4u);
    if constexpr (kXbf16) {
      const uint2 u = *reinterpret_cast<const uint2*>(x + 2 * (size_t)e0);
      raw[p][0] = u.x;
      raw[p][1] = u.y;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(x + 4 * (size_t)e0);
      raw[p][0] = u.x;
      raw[p][1] = u.y;
      raw[p][2] = u.z;
      raw[p][3] = u.w;
    }
  }
  const uint32_t G = gg.G;
  const uint32_t t0 = blockIdx.x;
  const uint32_t n = gg.q + (t0 < gg.r ? 1u : 0u);
  const uint32_t last = t0 + (n - 1u) * G;
  const uint32_t bl = min((uint32_t)lk, nb - 1u);
  auto load_tile = [&](uint32_t t, Q8Raw& w) {
    const uint32_t row = min(t * (uint32_t)S + (uint32_t)slot, N - 1u);
    const size_t blk = (size_t)row * nb + bl;
    w.a = codes[2 * blk];
    w.b = codes[2 * blk + 1];
    w.s = qscales[blk];
  };
  Q8Raw pa, pb;
  load_tile(t0, pa);
  load_tile(min(t0 + G, last), pb);

  // Quantize the activation: 8 lanes per block, 4 elements each.
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const uint32_t e0 = 4u * (uint32_t)(tid + p * nthreads);
    if (e0 >= K) break;                      // whole 8-lane groups leave together (K % 32 == 0)
    float v[4];
    if constexpr (kXbf16) {
      v[0] = bf16_lo(raw[p][0]); v[1] = bf16_hi(raw[p][0]); v[2] = bf16_lo(raw[p][1]); v[3] = bf16_hi(raw[p][1]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(raw[p][e]);
    }
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    m = max8(m);
    const float dx = m / 127.0f;
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float t = dx > 0.f ? rintf(v[e] / dx) : 0.f;
      t = fminf(fmaxf(t, -127.f), 127.f);
      word |= ((uint32_t)(int32_t)t & 0xffu) << (8 * e);
    }
    xq[e0 >> 2] = word;
    if ((e0 & 31u) == 0u) xs[e0 >> 5] = dx;
  }
  __syncthreads();
  const bool inside = (uint32_t)lk < nb;
  const uint4 xa = *reinterpret_cast<const uint4*>(xq + 8 * bl);
  const uint4 xb = *reinterpret_cast<const uint4*>(xq + 8 * bl + 4);
  const float dxl = inside ? xs[bl] : 0.f;  // a lane past the last block contributes zero

  uint32_t ti = 0;
  auto flush = [&](uint32_t first, uint32_t cnt) {
    __syncthreads();
    for (uint32_t e = (uint32_t)tid; e < cnt * (uint32_t)S; e += (uint32_t)nthreads) {
      const uint32_t jl = e / (uint32_t)S, s2 = e - jl * (uint32_t)S;
      const uint32_t li = first + jl;
      const uint32_t row = (t0 + li * G) * (uint32_t)S + s2;
      if (row < N) {
        float sum = 0.f;
        for (int w = 0; w < WK; ++w) sum += red[li % kRing][s2 * WK + w];
        y[row] = sum;
      }
    }
    __syncthreads();
  };
  auto do_tile = [&](uint32_t tt, const Q8Raw& w) {
    int isum = 0;
    isum = __builtin_amdgcn_sdot4((int)w.a.x, (int)xa.x, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.a.y, (int)xa.y, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.a.z, (int)xa.z, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.a.w, (int)xa.w, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.b.x, (int)xb.x, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.b.y, (int)xb.y, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.b.z, (int)xb.z, isum, false);
    isum = __builtin_amdgcn_sdot4((int)w.b.w, (int)xb.w, isum, false);
    const float sc = f16_bits_to_f32(w.s) * dxl;
    const float v = wave_sum((float)isum * sc);   // |isum| <= 32 * 127^2 < 2^24: exact in float32
    const uint32_t row = tt * (uint32_t)S + (uint32_t)slot;
    if (WK == 1) {
      if (lane == 0 && row < N) y[row] = v;
    } else {
      if (lane == 0) red[ti % kRing][slot * WK + wk] = v;
      ++ti;
      if (ti % kRing == 0) flush(ti - kRing, kRing);
    }
  };

  // Fixed trip count, unconditional clamped prefetches, remainder after the
  // loop: every path to a use of a register set carries the same loads, so
  // the compiler's waits leave the other set in flight.
  uint32_t t = t0;
  uint32_t i = 0;
  for (; i + 2 <= n; i += 2) {
    do_tile(t, pa);
    load_tile(min(t + 2 * G, last), pa);
    __builtin_amdgcn_sched_barrier(0);
    t += G;
    do_tile(t, pb);
    load_tile(min(t + 2 * G, last), pb);
    __builtin_amdgcn_sched_barrier(0);
    t += G;
  }
  if (i < n) do_tile(t, pa);
  if (WK > 1 && ti % kRing != 0) flush(ti - ti % kRing, ti % kRing);
}

// Persistent grid: the workgroups all CUs hold at once (runtime occupancy
// calculator), cached per kernel and device.
uint32_t resident(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int>, uint32_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kernel, threads, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int blocks = 0;
  uint32_t g = (uint32_t)device_cu_count();
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, threads, 0) == hipSuccess && blocks > 0)
    g = (uint32_t)(blocks * device_cu_count());
  cache.emplace(key, g);
  return g;
}

template <bool kXbf16, int kP>
void launch_q8_gemv_p(const uint4* codes, const uint16_t* qs, uint32_t N, uint32_t nb, const uint8_t* x, float* y,
                      hipStream_t s) {
  Q8Grid gg;
  gg.TK = (int)((nb + 63u) / 64u * 64u);
  gg.S = 1024 / gg.TK;
  gg.slot_mul = (256u * 64u + (uint32_t)gg.TK - 1u) / (uint32_t)gg.TK;   // ceil(256 / WK)
  const int threads = gg.S * gg.TK;
  const void* kern = (const void*)&q8_gemv_kernel<kXbf16, kP>;
  const uint32_t cap = resident(kern, threads);
  const uint32_t tiles = (N + (uint32_t)gg.S - 1u) / (uint32_t)gg.S;
  const uint32_t per_wg = (tiles + cap - 1u) / cap;
  const uint32_t grid = (tiles + per_wg - 1u) / per_wg;
  gg.G = grid;
  gg.q = tiles / grid;
  gg.r = tiles % grid;
  hipLaunchKernelGGL((q8_gemv_kernel<kXbf16, kP>), dim3(grid), dim3(threads), 0, s, codes, qs, N, nb, x, y, gg);
}

template <bool kXbf16>
void launch_q8_gemv_x(const uint4* codes, const uint16_t* qs, uint32_t N, uint32_t nb, const uint8_t* x, float* y,
                      hipStream_t s) {
  const uint32_t TK = (nb + 63u) / 64u * 64u;
  const uint32_t threads = (1024u / TK) * TK;
  const uint32_t passes = (nb * 32u + 4u * threads - 1u) / (4u * threads);
  if (passes <= 1) launch_q8_gemv_p<kXbf16, 1>(codes, qs, N, nb, x, y, s);
  else if (passes <= 2) launch_q8_gemv_p<kXbf16, 2>(codes, qs, N, nb, x, y, s);
  else if (passes <= 4) launch_q8_gemv_p<kXbf16, 4>(codes, qs, N, nb, x, y, s);
  else launch_q8_gemv_p<kXbf16, 8>(codes, qs, N, nb, x, y, s);
}

}  // namespace

hipError_t launch_transcode_q8(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                               int8_t* codes, uint16_t* qscales, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  const uint64_t total64 = (uint64_t)N * nb;
  // One launch per at most 2^31 blocks (32-bit thread indices).
  const uint64_t step = 1ull << 31;
  for (uint64_t b0 = 0; b0 < total64; b0 += step) {
    const uint32_t total = (uint32_t)std::min<uint64_t>(step, total64 - b0);
    const uint32_t grid = (total + kTcThreads - 1) / kTcThreads;
    hipLaunchKernelGGL(q8_transcode_kernel, dim3(grid), dim3(kTcThreads), 0, s,
                       reinterpret_cast<const uint4*>(packed) + b0, reinterpret_cast<const uint32_t*>(scales) + b0,
                       total, mask, host_codebook(), reinterpret_cast<uint4*>(codes) + 2 * b0, qscales + b0);
  }
  return hipGetLastError();
}

hipError_t launch_q8_gemv(const int8_t* codes, const uint16_t* qscales, int64_t N, int64_t K, const void* x,
                          bool xbf16, float* y, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  const uint4* c = reinterpret_cast<const uint4*>(codes);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (xbf16) launch_q8_gemv_x<true>(c, qscales, (uint32_t)N, nb, xb, y, s);
  else launch_q8_gemv_x<false>(c, qscales, (uint32_t)N, nb, xb, y, s);
  return hipGetLastError();
}

}  // namespace tq
