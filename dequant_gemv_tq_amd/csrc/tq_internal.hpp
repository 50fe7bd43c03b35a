// Internal declarations shared by the libtq translation units.
//
// Every kernel is written for gfx950 (CDNA4): 64-lane wavefronts, 160 KB of
// LDS per CU, 256 CUs in 8 XCDs.  The host entry points in tq_api.cpp
// validate arguments and call the launch_* functions of tq_launch.hpp.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kBlock = 32;           // TQ4_1S block length
constexpr int kHalf = 16;            // elements per scale (d0: 0-15, d1: 16-31)
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;   // float32(1/sqrt(32)) = 0x3E3504F3

// The 16-level Lloyd-Max quantizer for N(0,1) (TQ4 page, "格式原理" item 2 and
// the paragraph after the list): the 8 positive centroids rounded to float32,
// ascending; the law is symmetric, so centroid k < 8 is -kCentroidPos[7 - k].
// They are the fixed point of Lloyd's iteration (cell boundaries at the
// midpoints, each centroid the conditional mean (phi(a) - phi(b)) / (Phi(b) -
// Phi(a)) of its cell) iterated in float64 to a change below 1e-15 and
// rounded once; every value sits well away from a float32 rounding boundary.
// Device code uses them as immediates, so no kernel reads a codebook from
// memory.
constexpr float kCentroidPos[8] = {0x1.06f3fap-3f, 0x1.8d5c88p-2f, 0x1.5042bcp-1f, 0x1.e27a72p-1f,
                                   0x1.41985ep+0f, 0x1.9e384ap+0f, 0x1.08d58ep+1f, 0x1.5dc57ep+1f};
__host__ __device__ constexpr float centroid(int k) { return k < 8 ? -kCentroidPos[7 - k] : kCentroidPos[k - 8]; }

// Codebook handed to kernels by value (kernel-argument segment, read through
// the scalar cache): 16 ascending centroids and the 15 midpoint thresholds.
struct Codebook {
  float c[16];
  float m[15];
};

// Host side (tq_codebook.cpp).
const Codebook& host_codebook();

// Number of compute units of the current device (queried once per device).
int device_cu_count();

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// float32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__half_as_ushort(__float2half_rn(f));
}

// Non-negative finite float32 -> fp16 bits with round-to-nearest-even and
// saturation at 65504, in integer arithmetic (independent of the FP mode
// register, keeps fp16 subnormals).
__device__ __forceinline__ uint32_t f32_to_f16_sat_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if (u >= 0x477fe000u) return 0x7bffu;              // >= 65504 -> max finite
  int e = (int)(u >> 23) - 127;
  uint32_t m = (u & 0x7fffffu) | 0x800000u;
  if (e >= -14) {                                    // normal half
    uint32_t h = ((uint32_t)(e + 15) << 10) | ((m >> 13) & 0x3ffu);
    uint32_t rem = m & 0x1fffu;
    h += (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ? 1u : 0u;
    return h;                                        // carry may round up to the next binade
  }
  if (u == 0u) return 0u;
  int s = -e - 1;                                    // value / 2^-24 = m >> s
  if (s >= 32) return 0u;
  uint32_t q = m >> s;
  uint32_t rem = m & ((1u << s) - 1u);
  uint32_t half = 1u << (s - 1);
  q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  return q;
}

// fp16 bits -> float32, exact, in integer arithmetic (finite inputs).
__device__ __forceinline__ float f16_bits_to_f32_exact(uint32_t h) {
  uint32_t e = (h >> 10) & 0x1fu;
  uint32_t m = h & 0x3ffu;
  uint32_t s = (h & 0x8000u) << 16;
  if (e == 0u) {
    float v = (float)m * 0x1p-24f;                   // exact: m < 2^10
    return __uint_as_float(__float_as_uint(v) | s);
  }
  return __uint_as_float(s | ((e + 112u) << 23) | (m << 13));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)(h & 0xffffu)));
}

// Unnormalised 32-point Walsh-Hadamard transform in registers, Sylvester
// order: stages h = 1, 2, 4, 8, 16; pair (i, i+h) -> (v_i + v_{i+h}, v_i - v_{i+h}).
__device__ __forceinline__ void fwht32(float (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Flip the sign of element i when bit i of mask is set (exact).
__device__ __forceinline__ void apply_signs(float (&v)[32], uint32_t mask) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((mask >> i) & 1u) << 31));
}

// Copy the 16 centroids into LDS.  Compile-time indices keep the reads of the
// by-value codebook argument on the scalar unit (a runtime index would turn
// every read into a dependent vector load from the argument segment).  The
// caller synchronizes before reading lut16.
__device__ __forceinline__ void stage_centroids(const Codebook& cb, float* lut16) {
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) lut16[k] = cb.c[k];
  }
}

// Pair lookup table for decoding packed nibbles: entry e (a byte of two
// indices) holds the float32 pair (c[e & 15], c[e >> 4]), replicated 32
// times; copy l of entry e sits at LDS byte (e << 8) | 8 l, so the 32 lanes an
// LDS pass serves with ds_read_b64 (lane l uses copy l % 32) always hit
// distinct banks, and the address is one v_perm_b32 that places the byte of
// the packed word next to the lane offset.  64 KiB.
constexpr int kCopies = 32;
constexpr int kLutBytes = 256 * kCopies * 8;

// Pair table fill from the codebook constants (immediates: nothing waits on
// memory).  Wavefront w (of 16 virtual ones) writes entries e = 16 w + 4 u +
// lane / 16 (u < 4), copies 2 (lane % 16) and 2 (lane % 16) + 1, so the high
// centroid c[e / 16] = c[w] is a wavefront-uniform choice and the low one
// c[e % 16] = c[4 u + lane / 16] a per-lane choice of four.  Consecutive
// lanes store consecutive 16-byte chunks of the table (no bank conflicts).
__device__ __forceinline__ void fill_pair_lut(uint8_t* lut, int tid, int nthreads) {
  const int lane = tid & 63, g = lane >> 4;
  for (int w = tid >> 6; w < 16; w += nthreads >> 6) {
    const int wu = __builtin_amdgcn_readfirstlane(w);
    float hi = centroid(0);
#pragma unroll
    for (int k = 1; k < 16; ++k) hi = wu == k ? centroid(k) : hi;
    uint8_t* base = lut + ((16 * wu + g) << 8) + 16 * (lane & 15);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float lo = g == 0   ? centroid(4 * u)
                       : g == 1 ? centroid(4 * u + 1)
                       : g == 2 ? centroid(4 * u + 2)
                                : centroid(4 * u + 3);
      *reinterpret_cast<float4*>(base + (u << 10)) = make_float4(lo, hi, lo, hi);
    }
  }
}

// LDS address of the pair entry for byte k (0-3) of packed word w.
__device__ __forceinline__ uint32_t pair_addr(uint32_t w, uint32_t laneoff, int k) {
  return __builtin_amdgcn_perm(w, laneoff, 0x0C0C0000u | ((4u + (uint32_t)k) << 8));
}

// E4M3fn code (no sign) -> float32, exact: bias 7, subnormal step 2^-9.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0u ? (float)m * 0x1p-9f : __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
}

// Load one 32-element block (fp32 or bf16) into registers; p is 16-byte aligned.
template <bool kBf16>
__device__ __forceinline__ void load_block(const void* p, float (&v)[32]) {
  if constexpr (kBf16) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint4 u = q[t];
      v[8 * t + 0] = bf16_lo(u.x); v[8 * t + 1] = bf16_hi(u.x);
      v[8 * t + 2] = bf16_lo(u.y); v[8 * t + 3] = bf16_hi(u.y);
      v[8 * t + 4] = bf16_lo(u.z); v[8 * t + 5] = bf16_hi(u.z);
      v[8 * t + 6] = bf16_lo(u.w); v[8 * t + 7] = bf16_hi(u.w);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float4 u = q[t];
      v[4 * t + 0] = u.x; v[4 * t + 1] = u.y; v[4 * t + 2] = u.z; v[4 * t + 3] = u.w;
    }
  }
}

}  // namespace tq

#include "tq_launch.hpp"
