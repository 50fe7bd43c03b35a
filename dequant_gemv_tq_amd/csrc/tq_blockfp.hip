// NVFP4 and MXFP6 block formats on gfx950: quantizers and fused decode
// GEMV/GEMM (quantizer-tool page "这是我的 llama.cpp NVFP4/MXFP6 GGUF 量化工具",
// sections "目前能实现的部分功能" and "MXFP6 的未来"; llm-compressor page,
// section "NVFP4 + FP8 双格式支持").
//
// The pages name the formats only; the public definitions are used:
//   NVFP4: 16 E2M1 values per block, an E4M3fn block scale and one float32
//          tensor scale s_t = amax|W| / (6 * 448).
//          r_b = amax_b / fl(6 s_t) -> E4M3 (RNE, saturating); eff = fl(dec(sb) s_t);
//          code = E2M1(fl(w / eff)) (RNE, saturating, sign kept).
//   MXFP6: 32 E3M2 values per block and an E8M0 scale 2^e with
//          e = floor(log2 amax_b) - 4 (the E3M2 emax), clamped to [-127, 127];
//          code = E3M2(w * 2^-e).
// The quantizers optionally run an RSF-lite search over nearby block scales
// (quantizer-tool page, "RSF"), unweighted: the candidate with the smallest
// float32 squared reconstruction error wins.
// Every division is the correctly rounded float32 division, and the small
// float encoder is exact (power-of-two scaling + round-half-even), so the
// codes are reproducible bit for bit.
#pragma clang fp contract(off)

#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kThreads = 256;

// floor(log2 |a|) for a normal float32, or a value below every format's
// emin for zero and subnormals.
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t e = (__float_as_uint(a) >> 23) & 0xffu;
  return e == 0u ? -200 : (int)e - 127;
}

// Round a non-negative float32 to the sign-less code of a small float format
// with kM mantissa bits and minimum exponent kEmin (round half to even),
// saturating at kMaxCode.
template <int kM, int kEmin, uint32_t kMaxCode>
__device__ __forceinline__ uint32_t encode_mag(float a) {
  int e = floor_log2(a);
  e = e < kEmin ? kEmin : e;
  float q = __builtin_rintf(__builtin_ldexpf(a, kM - e));   // exact scaling, then RNE to an integer
  uint32_t code = (uint32_t)q + ((uint32_t)(e - kEmin) << kM);
  return code > kMaxCode ? kMaxCode : code;
}

__device__ __forceinline__ uint32_t sign_of(float v) { return __float_as_uint(v) >> 31; }

// encode_mag that also reports whether the scaled value a * 2^(kM - e) lies
// within 1e-5 of a half-integer, the only places where the code changes
// (it is continuous across the powers of two where e steps).
template <int kM, int kEmin, uint32_t kMaxCode>
__device__ __forceinline__ uint32_t encode_mag_near(float a, bool& near) {
  int e = floor_log2(a);
  e = e < kEmin ? kEmin : e;
  const float sc = __builtin_ldexpf(a, kM - e);
  const float q = __builtin_rintf(sc);
  near = fabsf(fabsf(sc - q) - 0.5f) < 1e-5f;
  uint32_t code = (uint32_t)q + ((uint32_t)(e - kEmin) << kM);
  return code > kMaxCode ? kMaxCode : code;
}

// The magnitude an E2M1 code 0..7 stands for: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t m = code & 1u, e = code >> 1;
  return e == 0u ? 0.5f * (float)m : __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
}

// encode_mag that also returns the magnitude the code stands for (exact:
// the rounded integer times a power of two, or the format's largest value).
template <int kM, int kEmin, uint32_t kMaxCode>
__device__ __forceinline__ uint32_t encode_mag_val(float a, float maxval, float& val) {
  int e = floor_log2(a);
  e = e < kEmin ? kEmin : e;
  const float q = __builtin_rintf(__builtin_ldexpf(a, kM - e));
  const uint32_t code = (uint32_t)q + ((uint32_t)(e - kEmin) << kM);
  val = code > kMaxCode ? maxval : __builtin_ldexpf(q, e - kM);
  return code > kMaxCode ? kMaxCode : code;
}

// ((((s0+s1)+(s2+s3))+((s4+s5)+(s6+s7)))+(((s8+s9)+(s10+s11))+((s12+s13)+(s14+s15)))) of s[o .. o+15].
template <int kN>
__device__ __forceinline__ float tree16(const float (&s)[kN], int o) {
  float a[8], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = s[o + 2 * i] + s[o + 2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = a[2 * i] + a[2 * i + 1];
  return (b[0] + b[1]) + (b[2] + b[3]);
}

// RSF-lite candidate order: multiplier 1 + j/16 for j = 0, -1, +1, -2, +2, ...
__device__ __forceinline__ int rsf_step(int t) { return (t & 1) ? -((t + 1) >> 1) : (t >> 1); }

// --------------------------------------------------------------------------
// NVFP4 quantizer, two launches: amax (one partial maximum per workgroup
// into the caller's workspace) -> encode (each workgroup reduces the
// partials, so nothing has to be zeroed first and no atomics are needed;
// workgroup 0 writes the tensor scale).  The maxima are taken on the bit
// patterns of |w|, which order like the values for non-negative floats.
// --------------------------------------------------------------------------

// Partial maxima the amax pass leaves in the workspace (at most).
constexpr uint32_t kAmaxPartials = 1024;
static_assert(kAmaxPartials * 4 == TQ_NVFP4_WORKSPACE_BYTES, "workspace size in the header");

// |w| bit patterns of one 16-byte chunk (the sign bit cleared).
template <bool kBf16>
__device__ __forceinline__ uint32_t chunk_max(const uint4& u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t m = 0u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (kBf16) m = max(m, max((w[t] << 16) & 0x7fff0000u, w[t] & 0x7fff0000u));
    else m = max(m, w[t] & 0x7fffffffu);
  }
  return m;
}

// Grid-stride max with four 16-byte loads in flight per thread, reduced
// across the workgroup in LDS; workgroup g writes partial[g].
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void amax_kernel(const uint8_t* __restrict__ W, size_t n16,
                                                        uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kThreads / 64];
  const uint4* src = reinterpret_cast<const uint4*>(W);
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x;
  uint32_t m = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    m = max(m, max(max(chunk_max<kBf16>(a), chunk_max<kBf16>(b)), max(chunk_max<kBf16>(c), chunk_max<kBf16>(d))));
  }
  for (; i < n16; i += stride) m = max(m, chunk_max<kBf16>(src[i]));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = max(m, red[w]);
    partial[blockIdx.x] = m;
  }
}

// The tensor amax from the amax pass's partials, reduced by the calling
// workgroup (every thread returns it).
__device__ __forceinline__ float reduce_amax(const uint32_t* __restrict__ partial, uint32_t count) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t m = 0u;
  for (uint32_t i = threadIdx.x; i < count; i += kThreads) m = max(m, partial[i]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) m = max(m, red[w]);
  return __uint_as_float(m);
}

// Squared float32 error of a 16-element block encoded with effective scale
// eff (codes +0 when eff = 0), summed as tree16.
// The code of fl(|v| / eff) comes from |v| * rcp(eff) as in the encoder,
// with the correctly rounded division near a rounding boundary.
__device__ __forceinline__ float nvfp4_block_error(const float (&v)[16], float eff) {
  float s[16];
  const bool fast = eff >= 0x1p-100f;
  const float r = __builtin_amdgcn_rcpf(eff);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float qhat = 0.0f;
    if (eff != 0.0f) {
      bool near = true;
      uint32_t code = fast ? encode_mag_near<1, 0, 7u>(fabsf(v[i]) * r, near) : 0u;
      if (near) code = encode_mag<1, 0, 7u>(fabsf(v[i] / eff));
      const float val = e2m1_value(code);
      qhat = (sign_of(v[i]) ? -val : val) * eff;
    }
    const float d = v[i] - qhat;
    s[i] = d * d;
  }
  return tree16(s, 0);
}

// One thread per 16-element block, grid-stride over the blocks.  kRsf: the
// block scale is chosen among the E4M3 roundings of dec(sb_0) * (1 + j/16),
// j = 0, -1, +1, ..., -4, +4, by the smallest float32 squared error (ties
// keep the earlier candidate).
template <bool kBf16, bool kRsf>
__device__ __forceinline__ void nvfp4_encode_block(const uint8_t* __restrict__ W, uint32_t g, float st,
                                                   uint2* __restrict__ codes, uint8_t* __restrict__ bscales) {
  float v[16];
  if constexpr (kBf16) {
    const uint4* q = reinterpret_cast<const uint4*>(W + (size_t)g * 32);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint4 u = q[t];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * t + 2 * k] = bf16_lo(w[k]);
        v[8 * t + 2 * k + 1] = bf16_hi(w[k]);
      }
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(W + (size_t)g * 64);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float4 u = q[t];
      v[4 * t] = u.x; v[4 * t + 1] = u.y; v[4 * t + 2] = u.z; v[4 * t + 3] = u.w;
    }
  }
  uint32_t sb = 0u;
  uint32_t lo = 0u, hi = 0u;
  if (st != 0.0f) {
    float ab = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(v[i]));
    const float six_st = 6.0f * st;
    sb = encode_mag<3, -6, 0x7eu>(ab / six_st);
    if constexpr (kRsf) {
      const float base = e4m3_decode(sb);
      float best = nvfp4_block_error(v, e4m3_decode(sb) * st);
#pragma unroll 1
      for (int t = 1; t < 9; ++t) {
        const uint32_t c = encode_mag<3, -6, 0x7eu>(base * (1.0f + (float)rsf_step(t) * 0.0625f));
        const float err = nvfp4_block_error(v, e4m3_decode(c) * st);
        if (err < best) {
          best = err;
          sb = c;
        }
      }
    }
    const float eff = e4m3_decode(sb) * st;
    if (eff != 0.0f) {
      // The code of fl(|v| / eff) from |v| * rcp(eff): for a normal eff the
      // two differ by less than 1.7e-6 below 8 (rcp within 1 ulp, one product
      // rounding, half an ulp of the quotient), i.e. by less than 3.4e-6 once
      // scaled by 2^(1 - e) <= 2, so the code only needs the correctly
      // rounded division when the scaled value is within 1e-5 of a
      // half-integer.  eff > 0, so the sign is v's.
      const bool fast = eff >= 0x1p-100f;
      const float r = __builtin_amdgcn_rcpf(eff);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        bool near = true;
        uint32_t m = fast ? encode_mag_near<1, 0, 7u>(fabsf(v[i]) * r, near) : 0u;
        if (near) m = encode_mag<1, 0, 7u>(fabsf(v[i] / eff));
        const uint32_t c = m | (sign_of(v[i]) << 3);
        if (i < 8) lo |= c << (4 * i);
        else hi |= c << (4 * (i - 8));
      }
    }
  }
  codes[g] = make_uint2(lo, hi);
  bscales[g] = (uint8_t)sb;
}

// s_t = fl(amax / 2688) from the partial maxima; workgroup 0 of the first
// launch stores it as the tensor scale.
template <bool kBf16, bool kRsf>
__global__ __launch_bounds__(kThreads) void nvfp4_encode_kernel(const uint8_t* __restrict__ W, uint32_t total,
                                                                const uint32_t* __restrict__ partial,
                                                                uint32_t npartial, float* __restrict__ tscale,
                                                                uint2* __restrict__ codes,
                                                                uint8_t* __restrict__ bscales) {
  const float st = reduce_amax(partial, npartial) / 2688.0f;
  if (tscale && blockIdx.x == 0 && threadIdx.x == 0) *tscale = st;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t g = blockIdx.x * kThreads + threadIdx.x; g < total; g += stride)
    nvfp4_encode_block<kBf16, kRsf>(W, g, st, codes, bscales);
}

// --------------------------------------------------------------------------
// MXFP6 quantizer: one thread per 32-element block, 24 bytes of codes.
// kRsf: the scale exponent is chosen among e0, e0 - 1, e0 + 1 (clamped) by
// the smallest float32 squared error, tree16(first half) + tree16(second
// half); ties keep the earlier candidate.
// --------------------------------------------------------------------------

__device__ __forceinline__ float mxfp6_block_error(const float (&v)[32], int e) {
  float s[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float q = __builtin_ldexpf(v[i], -e);
    float val;
    encode_mag_val<2, -2, 0x1fu>(fabsf(q), 28.0f, val);
    const float d = v[i] - __builtin_ldexpf(sign_of(q) ? -val : val, e);
    s[i] = d * d;
  }
  return tree16(s, 0) + tree16(s, 16);
}

template <bool kBf16, bool kRsf>
__global__ __launch_bounds__(kThreads) void mxfp6_encode_kernel(const uint8_t* __restrict__ W, uint32_t total,
                                                                uint2* __restrict__ codes,
                                                                uint8_t* __restrict__ bscales) {
  uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  float v[32];
  load_block<kBf16>(W + (size_t)g * (kBf16 ? 64 : 128), v);
  float ab = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) ab = fmaxf(ab, fabsf(v[i]));
  uint64_t bits[3] = {0ull, 0ull, 0ull};
  uint32_t byte = 0u;
  if (ab != 0.0f) {
    int e = floor_log2(ab) - 4;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    if constexpr (kRsf) {
      const int e0 = e;
      float best = mxfp6_block_error(v, e0);
#pragma unroll 1
      for (int t = 1; t < 3; ++t) {
        int ej = e0 + (t == 1 ? -1 : 1);
        ej = ej < -127 ? -127 : (ej > 127 ? 127 : ej);
        const float err = mxfp6_block_error(v, ej);
        if (err < best) {
          best = err;
          e = ej;
        }
      }
    }
    byte = (uint32_t)(e + 127);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float q = __builtin_ldexpf(v[i], -e);
      const uint64_t c = encode_mag<2, -2, 0x1fu>(fabsf(q)) | (sign_of(q) << 5);
      const int bit = 6 * i;                  // code i occupies bits 6i..6i+5 of the 192-bit block
      bits[bit >> 6] |= c << (bit & 63);
      if ((bit & 63) > 58) bits[(bit >> 6) + 1] |= c >> (64 - (bit & 63));
    }
  }
  uint2* dst = codes + (size_t)g * 3;
#pragma unroll
  for (int t = 0; t < 3; ++t) dst[t] = make_uint2((uint32_t)bits[t], (uint32_t)(bits[t] >> 32));
  bscales[g] = (uint8_t)byte;
}

inline uint32_t grid_for(uint32_t total) { return (total + kThreads - 1) / kThreads; }

}  // namespace

hipError_t launch_blockfp_quantize(int fmt, const void* W, bool bf16, int64_t N, int64_t K, uint8_t* codes,
                                   uint8_t* bscales, float* tscale, void* workspace, hipStream_t s, bool rsf) {
  const uint8_t* w = static_cast<const uint8_t*>(W);
  const int64_t esz = bf16 ? 2 : 4;
  if (fmt == TQ_FMT_NVFP4) {
    uint32_t* partial = static_cast<uint32_t*>(workspace);
    const size_t n16 = (size_t)(N * K * esz / 16);
    const size_t want = (n16 + kThreads - 1) / kThreads;
    size_t cap = (size_t)(4 * device_cu_count());
    cap = cap < kAmaxPartials ? cap : kAmaxPartials;
    const uint32_t parts = (uint32_t)(want < cap ? want : cap);
    if (bf16) hipLaunchKernelGGL(amax_kernel<true>, dim3(parts), dim3(kThreads), 0, s, w, n16, partial);
    else hipLaunchKernelGGL(amax_kernel<false>, dim3(parts), dim3(kThreads), 0, s, w, n16, partial);
    // Encode: a grid-stride launch of at most 16 workgroups per compute
    // unit, so the partials are reduced by a bounded number of workgroups.
    const int64_t blocks = N * K / 16;
    const int64_t per_launch = (int64_t)1 << 30;
    const uint32_t gcap = (uint32_t)(16 * device_cu_count());
    for (int64_t b0 = 0; b0 < blocks; b0 += per_launch) {
      const uint32_t total = (uint32_t)((blocks - b0 < per_launch) ? blocks - b0 : per_launch);
      const uint32_t grid = grid_for(total) < gcap ? grid_for(total) : gcap;
      const uint8_t* wb = w + b0 * 16 * esz;
      uint2* cb = reinterpret_cast<uint2*>(codes) + b0;
      float* ts = b0 == 0 ? tscale : nullptr;
#define TQ_NVFP4(B, R) \
  hipLaunchKernelGGL((nvfp4_encode_kernel<B, R>), dim3(grid), dim3(kThreads), 0, s, wb, total, partial, parts, ts, \
                     cb, bscales + b0)
      if (bf16) {
        if (rsf) TQ_NVFP4(true, true);
        else TQ_NVFP4(true, false);
      } else {
        if (rsf) TQ_NVFP4(false, true);
        else TQ_NVFP4(false, false);
      }
#undef TQ_NVFP4
    }
  } else {
    const int64_t blocks = N * K / 32;
    const int64_t per_launch = (int64_t)1 << 30;
    for (int64_t b0 = 0; b0 < blocks; b0 += per_launch) {
      const uint32_t total = (uint32_t)((blocks - b0 < per_launch) ? blocks - b0 : per_launch);
      const uint8_t* wb = w + b0 * 32 * esz;
      uint2* cb = reinterpret_cast<uint2*>(codes) + b0 * 3;
#define TQ_MXFP6(B, R) \
  hipLaunchKernelGGL((mxfp6_encode_kernel<B, R>), dim3(grid_for(total)), dim3(kThreads), 0, s, wb, total, cb, \
                     bscales + b0)
      if (bf16) {
        if (rsf) TQ_MXFP6(true, true);
        else TQ_MXFP6(true, false);
      } else {
        if (rsf) TQ_MXFP6(false, true);
        else TQ_MXFP6(false, false);
      }
#undef TQ_MXFP6
    }
  }
  return hipGetLastError();
}

}  // namespace tq
