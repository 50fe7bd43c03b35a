// Small-batch fused TQ4_1S GEMM on gfx950: Y[m, n] = sum_k X'[m, k] Q[n, k]
// with Q = d * c[idx] in the rotated domain and X' the pre-rotated
// activations (the same identity as the GEMV: rotating the activation once
// turns dequantization into a centroid lookup times a scale; TQ4 page
// "企业官网建设流程全解析", hotelren.com/news/5458160, decode-speed section).
//
// For M >= 16 the contraction is dense enough for the matrix cores:
// v_mfma_f32_16x16x32_bf16 computes a 16(m) x 16(n) tile over 32 k.
//   * B operand (weights): lane l holds row n = l % 16 of the n-tile and the
//     k-slot group g = l / 16.  One 16-byte load gives a lane the 32 nibbles
//     of block b0 + g of its row; dword s of that load feeds MFMA step s, so
//     every weight is loaded once and dequantized once (lookup, scale, round
//     to bf16) straight into the operand registers -- no LDS staging.
//   * A operand (activations): the same (g, s) k-assignment, i.e. lane l
//     loads 8 consecutive bf16 of X'[m = l % 16] at element 32 (b0 + g) + 8 s.
//     An MFMA only pairs A and B slots of the same lane group, so any k
//     permutation shared by A and B gives the same sum.
//   * Output: lane l, register r holds D[4 (l / 16) + r][l % 16].
//   * A workgroup is 4 wavefronts on one 16-row n-tile; wavefront w takes
//     every 4th group of 4 blocks along K (split-K inside the workgroup) and
//     the four partial tiles are summed through LDS, so even N = 4096 gives
//     256 workgroups.
// Arithmetic intensity stays below the bf16 ridge for M <= 64 (about 3.2 M
// flop per byte of packed weight), so HBM remains the bound.
//
// Precision: with bf16 activations both operands carry a 2^-9 relative
// rounding, so |dy| is about 2^-9 * ||w o x||_2, inside 1e-3 * sum|w x| once K
// is in the hundreds.  With float32 activations each operand is split into
// bf16 hi + lo (hi by truncation, lo = bf16(v - hi), exact residual) and three
// MFMAs (hi*hi + hi*lo + lo*hi) keep about 16 significant bits per product,
// which holds the bound at any K.
#include "tq_internal.hpp"

namespace tq {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;

// Split 8 float32 values into bf16 hi (truncation) and lo (RNE of the exact residual).
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t h = __float_as_uint(v[t]) & 0xffff0000u;
    hi[t] = (short)(h >> 16);
    lo[t] = (short)f32_to_bf16_rne(v[t] - __uint_as_float(h));
  }
}

template <int MT, bool kF32X>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(const uint4* __restrict__ packed,
                                                        const uint32_t* __restrict__ scales, uint32_t N,
                                                        uint32_t nb, const void* __restrict__ Xv, int64_t ldx,
                                                        uint32_t M, float* __restrict__ Y, int64_t ldy,
                                                        Codebook cb) {
  __shared__ float lut[16];
  __shared__ f32x4 part[kWaves - 1][MT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  stage_centroids(cb, lut);
  __syncthreads();

  const uint32_t n0 = blockIdx.x * 16u;
  const uint32_t row = n0 + nl;
  const bool row_ok = row < N;

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (uint32_t b0 = 4u * wave; b0 < nb; b0 += 4u * kWaves) {
    const uint32_t b = b0 + g;
    const bool ok = b < nb;
    uint4 p = make_uint4(0u, 0u, 0u, 0u);
    uint32_t sc = 0u;
    if (ok && row_ok) {
      p = packed[(size_t)row * nb + b];
      sc = scales[(size_t)row * nb + b];
    }
    const float d0 = f16_bits_to_f32(sc & 0xffffu);
    const float d1 = f16_bits_to_f32(sc >> 16);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float d = s < 2 ? d0 : d1;
      float wv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) wv[t] = d * lut[(w[s] >> (4 * t)) & 15u];
      if constexpr (!kF32X) {
        const uint16_t* X = static_cast<const uint16_t*>(Xv);
        bf16x8 B;
#pragma unroll
        for (int t = 0; t < 8; ++t) B[t] = (short)f32_to_bf16_rne(wv[t]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint32_t m = mt * 16u + nl;
          bf16x8 A = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
          if (ok && m < M) A = *reinterpret_cast<const bf16x8*>(X + (size_t)m * ldx + (size_t)b * 32 + 8 * s);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[mt], 0, 0, 0);
        }
      } else {
        const float* X = static_cast<const float*>(Xv);
        bf16x8 Bh, Bl;
        split8(wv, Bh, Bl);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint32_t m = mt * 16u + nl;
          float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (ok && m < M) {
            const float4* src = reinterpret_cast<const float4*>(X + (size_t)m * ldx + (size_t)b * 32 + 8 * s);
            const float4 u0 = src[0], u1 = src[1];
            xv[0] = u0.x; xv[1] = u0.y; xv[2] = u0.z; xv[3] = u0.w;
            xv[4] = u1.x; xv[5] = u1.y; xv[6] = u1.z; xv[7] = u1.w;
          }
          bf16x8 Ah, Al;
          split8(xv, Ah, Al);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bh, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bl, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bh, acc[mt], 0, 0, 0);
        }
      }
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) part[wave - 1][mt][lane] = acc[mt];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 v = acc[mt];
#pragma unroll
      for (int w2 = 0; w2 < kWaves - 1; ++w2) v += part[w2][mt][lane];
      if (row_ok) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t m = mt * 16u + 4u * g + r;
          if (m < M) Y[(size_t)m * ldy + row] = v[r];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                       const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  if (M < 16) return launch_gemm_valu(packed, scales, N, K, M, xr, xbf16, ldx, y, ldy, s);
  const Codebook& cb = host_codebook();
  const uint32_t nb = (uint32_t)(K / kBlock);
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(scales);
  const uint8_t* X = static_cast<const uint8_t*>(xr);
  const int64_t xs = xbf16 ? 2 : 4;
  const dim3 grid((unsigned)((N + 15) / 16)), block(256);
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t mc = (M - m0 < 64) ? M - m0 : 64;
    const void* Xm = X + m0 * ldx * xs;
    float* Ym = y + m0 * ldy;
    const int mt = (int)((mc + 15) / 16);
#define TQ_LAUNCH_MFMA(MT_, F32_)                                                                                  \
  hipLaunchKernelGGL((gemm_mfma_kernel<MT_, F32_>), grid, block, 0, s, pk, sc, (uint32_t)N, nb, Xm, ldx,          \
                     (uint32_t)mc, Ym, ldy, cb)
    if (xbf16) {
      switch (mt) {
        case 1: TQ_LAUNCH_MFMA(1, false); break;
        case 2: TQ_LAUNCH_MFMA(2, false); break;
        case 3: TQ_LAUNCH_MFMA(3, false); break;
        default: TQ_LAUNCH_MFMA(4, false); break;
      }
    } else {
      switch (mt) {
        case 1: TQ_LAUNCH_MFMA(1, true); break;
        case 2: TQ_LAUNCH_MFMA(2, true); break;
        case 3: TQ_LAUNCH_MFMA(3, true); break;
        default: TQ_LAUNCH_MFMA(4, true); break;
      }
    }
#undef TQ_LAUNCH_MFMA
  }
  return hipGetLastError();
}

}  // namespace tq
