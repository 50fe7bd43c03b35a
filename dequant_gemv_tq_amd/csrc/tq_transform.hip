// Per-block TQ4_1S transforms on gfx950: quantize (weights -> nibbles + fp16
// scales), rotate (activations -> rotated activations) and dequantize.
//
// TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160), "格式原理":
//   1. each 32-element block is rotated by a randomized Walsh-Hadamard
//      transform with sign flips;
//   2. every rotated value maps to the nearest of 16 Lloyd-Max N(0,1)
//      centroids;
//   3. elements 0-15 and 16-31 keep separate scales d0, d1.
// The decode-speed section's "rotate the activation once" is tq_rotate.
//
// One thread owns one block: the 32 values live in VGPRs, the FWHT is five
// register butterfly stages with no cross-lane traffic, and each thread
// writes 16 contiguous bytes of nibbles and one 32-bit scale pair, so
// consecutive lanes produce fully coalesced 16-byte and 4-byte stores.
//
// Bit-exact float32 order (shared definition with any CPU reference):
//   v = D w; u = FWHT32(v) in stages h = 1, 2, 4, 8, 16; w' = u * fl(1/sqrt 32);
//   per half: sq_i = w'_i * w'_i; ss = pairwise tree in index order;
//   rms = sqrt(ss * 0.0625) correctly rounded; d = fp16_rne_sat(rms);
//   idx = #{k : w' > fl(d * m_k)}.
// FMA contraction would change these roundings, so it is off in this file.
#pragma clang fp contract(off)

#include "tq_internal.hpp"
#include "tq_codes.hpp"

namespace tq {
namespace {

constexpr int kThreads = 256;

// kRsf: the RSF-lite scale search (quantizer-tool page, "RSF": search nearby
// multiples of the scale and keep the better lattice fit).  For each half,
// candidates d_j = fp16(dd * (1 + j/16)) are tried in the order j = 0, -1,
// +1, -2, +2, -3, +3, -4, +4; each re-chooses its indices with the same rule
// and scores e_i = w'_i - fl(d_j * c[idx_i]), E = pairwise tree of e_i^2 in
// float32; only a strictly smaller E replaces the current choice, so j = 0
// (the plain quantizer) wins ties and nothing gets worse.
template <bool kBf16, bool kRsf>
__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint8_t* __restrict__ W, int64_t ldw_bytes,
                                                            uint32_t nb, uint32_t total, uint32_t mask,
                                                            Codebook cb, uint4* __restrict__ packed,
                                                            uint32_t* __restrict__ scales) {
  __shared__ float lut[16];
  __shared__ uint2 cells[kCells];
  build_cells(cb, cells);
  if constexpr (kRsf) stage_centroids(cb, lut);
  __syncthreads();
  uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  uint32_t row = g / nb;
  uint32_t b = g - row * nb;
  const uint8_t* src = W + (int64_t)row * ldw_bytes + (int64_t)b * (kBf16 ? 64 : 128);

  float v[32];
  load_block<kBf16>(src, v);
  apply_signs(v, mask);
  fwht32(v);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = v[i] * kInvSqrt32;

  uint32_t words[4] = {0u, 0u, 0u, 0u};
  uint32_t dbits[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = v[16 * h + i] * v[16 * h + i];
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1) {
#pragma unroll
      for (int i = 0; i < w; ++i) s[i] = s[2 * i] + s[2 * i + 1];
    }
    float rms = __builtin_sqrtf(s[0] * 0.0625f);
    dbits[h] = f16_sat(rms);
    float dd = f16_bits_to_f32(dbits[h]);
    if constexpr (!kRsf) {
      const float r8 = 8.0f * __builtin_amdgcn_rcpf(dd);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        int e = 16 * h + i;
        words[e >> 3] |= nearest_index(v[e], dd, r8, cells) << (4 * (e & 7));
      }
    } else {
      constexpr int kOrder[9] = {0, -1, 1, -2, 2, -3, 3, -4, 4};
      float best = 0.f;
      uint32_t best_bits = 0u, best_w0 = 0u, best_w1 = 0u;
#pragma unroll 1
      for (int c = 0; c < 9; ++c) {
        const float mult = 1.0f + (float)kOrder[c] * 0.0625f;
        const uint32_t bits = f16_sat(dd * mult);                  // the float32 product is exact
        const float ddj = f16_bits_to_f32(bits);
        const float r8 = 8.0f * __builtin_amdgcn_rcpf(ddj);
        uint32_t w0 = 0u, w1 = 0u;
        float sq[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t idx = nearest_index(v[16 * h + i], ddj, r8, cells);
          if (i < 8) w0 |= idx << (4 * i);
          else w1 |= idx << (4 * (i - 8));
          const float e = v[16 * h + i] - ddj * lut[idx];
          sq[i] = e * e;
        }
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) {
#pragma unroll
          for (int i = 0; i < w; ++i) sq[i] = sq[2 * i] + sq[2 * i + 1];
        }
        if (c == 0 || sq[0] < best) {
          best = sq[0];
          best_bits = bits;
          best_w0 = w0;
          best_w1 = w1;
        }
      }
      dbits[h] = best_bits;
      words[2 * h] = best_w0;
      words[2 * h + 1] = best_w1;
    }
  }
  packed[g] = make_uint4(words[0], words[1], words[2], words[3]);
  scales[g] = dbits[0] | (dbits[1] << 16);
}

template <bool kInBf16, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void rotate_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes,
                                                          uint32_t nb, uint32_t total, uint32_t mask,
                                                          uint8_t* __restrict__ xr, int64_t ldr_bytes) {
  uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  uint32_t row = g / nb;
  uint32_t b = g - row * nb;
  float v[32];
  load_block<kInBf16>(x + (int64_t)row * ldx_bytes + (int64_t)b * (kInBf16 ? 64 : 128), v);
  apply_signs(v, mask);
  fwht32(v);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = v[i] * kInvSqrt32;
  uint8_t* dst = xr + (int64_t)row * ldr_bytes + (int64_t)b * (kOutBf16 ? 64 : 128);
  if constexpr (kOutBf16) {
    uint4* q = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = f32_to_bf16_rne(v[8 * t + 2 * u]) | (f32_to_bf16_rne(v[8 * t + 2 * u + 1]) << 16);
      q[t] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    float4* q = reinterpret_cast<float4*>(dst);
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = make_float4(v[4 * t], v[4 * t + 1], v[4 * t + 2], v[4 * t + 3]);
  }
}

// Dequantize: q_i = d_h * c[idx_i], then the inverse rotation
// w = fl(1/sqrt 32) * D * FWHT32(q)   (H32 is symmetric and H32^2 = 32 I).
// The sign flip rides on the scale multiply (fl(u * -s) = -fl(u * s)), with
// the signed scales formed on the scalar unit.  The bf16 output is rounded
// by v_cvt_pk_bf16_f32 (round to nearest even).  Each wavefront's 64 blocks
// pass through LDS on the way out, so that every store instruction writes
// 1 KiB of consecutive 16-byte chunks instead of 16 bytes every 64 (128 for
// float32 output).
typedef __bf16 bf16x2t __attribute__((ext_vector_type(2)));

template <bool kOutBf16>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint4* __restrict__ packed,
                                                              const uint32_t* __restrict__ scales,
                                                              uint32_t nb, uint32_t total, uint32_t mask,
                                                              Codebook cb, uint8_t* __restrict__ out,
                                                              int64_t ldo_bytes) {
  constexpr int kChunks = kOutBf16 ? 4 : 8;            // 16-byte chunks per block
  __shared__ float lut[16];
  __shared__ __attribute__((aligned(16))) uint4 stage[kThreads / 64][64 * kChunks];
  stage_centroids(cb, lut);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t gw = blockIdx.x * kThreads + wave * 64;         // first block of this wavefront
  if (gw >= total) return;                                       // wavefront-uniform
  const uint32_t g = gw + lane;
  const bool live = g < total;
  const uint32_t gc = live ? g : total - 1u;
  uint4 p = packed[gc];
  uint32_t sc = scales[gc];
  float d0 = f16_bits_to_f32(sc & 0xffffu);
  float d1 = f16_bits_to_f32(sc >> 16);
  uint32_t words[4] = {p.x, p.y, p.z, p.w};
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    uint32_t n = (words[e >> 3] >> (4 * (e & 7))) & 15u;
    v[e] = (e < 16 ? d0 : d1) * lut[n];
  }
  fwht32(v);
#pragma unroll
  for (int i = 0; i < 32; ++i)
    v[i] = v[i] * __uint_as_float(__float_as_uint(kInvSqrt32) ^ (((mask >> i) & 1u) << 31));
  uint4* const st = stage[wave];
  if constexpr (kOutBf16) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x2t h = {(__bf16)v[8 * t + 2 * u], (__bf16)v[8 * t + 2 * u + 1]};
        w[u] = __builtin_bit_cast(uint32_t, h);
      }
      st[lane * kChunks + t] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      st[lane * kChunks + t] = make_uint4(__float_as_uint(v[4 * t]), __float_as_uint(v[4 * t + 1]),
                                          __float_as_uint(v[4 * t + 2]), __float_as_uint(v[4 * t + 3]));
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0): this wavefront's LDS stores done
  __builtin_amdgcn_wave_barrier();
  // Chunk c of the wavefront is chunk c % kChunks of block gw + c / kChunks.
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const uint32_t c = (uint32_t)(lane + 64 * j);
    const uint32_t gb = gw + c / kChunks;
    if (gb < total) {
      const uint32_t row = gb / nb, b = gb - row * nb;
      uint8_t* dst = out + (int64_t)row * ldo_bytes + (int64_t)b * (16 * kChunks) + 16 * (c % kChunks);
      *reinterpret_cast<uint4*>(dst) = st[c];
    }
  }
}

inline uint32_t grid_for(uint32_t total) { return (total + kThreads - 1) / kThreads; }

}  // namespace

// The flat block index g = row * nb + b is kept in 32 bits; callers split
// larger tensors into row chunks so that each launch stays below 2^31 blocks.
hipError_t launch_quantize(const void* W, bool bf16, int64_t N, int64_t K, int64_t ldw, uint32_t mask,
                           uint8_t* packed, uint16_t* scales, hipStream_t s, bool rsf) {
  const Codebook& cb = host_codebook();
  const uint32_t nb = (uint32_t)(K / kBlock);
  const int64_t esz = bf16 ? 2 : 4;
  const int64_t rows_per_launch = ((int64_t)1 << 30) / nb;
  for (int64_t r0 = 0; r0 < N; r0 += rows_per_launch) {
    int64_t rows = (N - r0 < rows_per_launch) ? N - r0 : rows_per_launch;
    uint32_t total = (uint32_t)(rows * nb);
    const uint8_t* w = static_cast<const uint8_t*>(W) + r0 * ldw * esz;
    uint4* pk = reinterpret_cast<uint4*>(packed + r0 * (K / 2));
    uint32_t* sc = reinterpret_cast<uint32_t*>(scales + r0 * (K / 16));
#define TQ_QUANT(B_, R_)                                                                                   \
  hipLaunchKernelGGL((quantize_kernel<B_, R_>), dim3(grid_for(total)), dim3(kThreads), 0, s, w, ldw * esz, nb, \
                     total, mask, cb, pk, sc)
    if (bf16) {
      if (rsf) TQ_QUANT(true, true);
      else TQ_QUANT(true, false);
    } else {
      if (rsf) TQ_QUANT(false, true);
      else TQ_QUANT(false, false);
    }
#undef TQ_QUANT
  }
  return hipGetLastError();
}

hipError_t launch_rotate(const void* x, bool xbf16, int64_t M, int64_t K, int64_t ldx, uint32_t mask,
                         void* xr, bool rbf16, int64_t ldr, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  const int64_t rows_per_launch = ((int64_t)1 << 30) / nb;
  const int64_t xs = xbf16 ? 2 : 4, rs = rbf16 ? 2 : 4;
  for (int64_t r0 = 0; r0 < M; r0 += rows_per_launch) {
    int64_t rows = (M - r0 < rows_per_launch) ? M - r0 : rows_per_launch;
    uint32_t total = (uint32_t)(rows * nb);
    const uint8_t* xi = static_cast<const uint8_t*>(x) + r0 * ldx * xs;
    uint8_t* xo = static_cast<uint8_t*>(xr) + r0 * ldr * rs;
    dim3 grid(grid_for(total)), block(kThreads);
    if (xbf16 && rbf16)
      hipLaunchKernelGGL((rotate_kernel<true, true>), grid, block, 0, s, xi, ldx * xs, nb, total, mask, xo, ldr * rs);
    else if (xbf16)
      hipLaunchKernelGGL((rotate_kernel<true, false>), grid, block, 0, s, xi, ldx * xs, nb, total, mask, xo, ldr * rs);
    else if (rbf16)
      hipLaunchKernelGGL((rotate_kernel<false, true>), grid, block, 0, s, xi, ldx * xs, nb, total, mask, xo, ldr * rs);
    else
      hipLaunchKernelGGL((rotate_kernel<false, false>), grid, block, 0, s, xi, ldx * xs, nb, total, mask, xo, ldr * rs);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                             void* out, bool bf16, int64_t ldo, hipStream_t s) {
  const Codebook& cb = host_codebook();
  const uint32_t nb = (uint32_t)(K / kBlock);
  const int64_t esz = bf16 ? 2 : 4;
  const int64_t rows_per_launch = ((int64_t)1 << 30) / nb;
  for (int64_t r0 = 0; r0 < N; r0 += rows_per_launch) {
    int64_t rows = (N - r0 < rows_per_launch) ? N - r0 : rows_per_launch;
    uint32_t total = (uint32_t)(rows * nb);
    const uint4* pk = reinterpret_cast<const uint4*>(packed + r0 * (K / 2));
    const uint32_t* sc = reinterpret_cast<const uint32_t*>(scales + r0 * (K / 16));
    uint8_t* o = static_cast<uint8_t*>(out) + r0 * ldo * esz;
    if (bf16)
      hipLaunchKernelGGL(dequantize_kernel<true>, dim3(grid_for(total)), dim3(kThreads), 0, s, pk, sc, nb, total,
                         mask, cb, o, ldo * esz);
    else
      hipLaunchKernelGGL(dequantize_kernel<false>, dim3(grid_for(total)), dim3(kThreads), 0, s, pk, sc, nb, total,
                         mask, cb, o, ldo * esz);
  }
  return hipGetLastError();
}

}  // namespace tq
