// Fused batch-1 TQ4_1S GEMV on gfx950: y = W_deq x computed in the rotated
// domain, y_n = sum_b [ d0 * sum_{i<16} c[idx_i] x'_i + d1 * sum_{i>=16} c[idx_i] x'_i ].
//
// TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160), decode-speed
// section (paragraph on why CUDA differs): rotating the activation once
// removes the per-block inverse transform, so dequantization is a centroid
// lookup times a scale; amortizing the rotation over several rows (the Metal
// kernel's NR0 = 8) and keeping the fused kernel free of threadgroup-memory
// pressure (it fixed a 27B decode regression) are what made it fast.
//
// MI355X design
//   * The decode GEMV is HBM-bound: 0.625 B per weight (16 B of nibbles +
//     4 B of fp16 scales per 32 weights).  Each lane owns J fixed K-blocks
//     (b = lane + j*T) and keeps their 32*J rotated activations in VGPRs for
//     the whole kernel -- the register equivalent of NR0 -- so x' is read
//     once per workgroup, not once per row.
//   * Per row, a lane issues one 16-byte load of nibbles and one 4-byte load
//     of scales per owned block; consecutive lanes read consecutive blocks,
//     so every wavefront load is a contiguous 1 KiB (256 B for scales).  R
//     rows are loaded before any is consumed to keep ~R KiB per wavefront in
//     flight.
//   * The 16-entry codebook sits in 64 B of LDS; a wavefront's lookups hit 16
//     distinct banks at most, so they are conflict-free.
//   * Partial sums are reduced across the wavefront with cross-lane shuffles
//     and across the workgroup's wavefronts through a few bytes of LDS.
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kMaxThreads = 1024;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// One block against MC activations: the 32 weights are looked up once
// (c[idx], unscaled) and multiplied into every activation row; the two half
// sums of each row take their scale at the end.
template <int MC>
__device__ __forceinline__ void block_dot(const uint4& p, uint32_t sc, const float (&x)[MC][32], const float* lut,
                                          float (&acc)[MC]) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
  float a[MC][2];
#pragma unroll
  for (int m = 0; m < MC; ++m) a[m][0] = a[m][1] = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float c = lut[(w[q] >> (4 * t)) & 15u];
#pragma unroll
      for (int m = 0; m < MC; ++m) a[m][q >> 1] = __builtin_fmaf(c, x[m][8 * q + t], a[m][q >> 1]);
    }
  }
  const float d0 = f16_bits_to_f32(sc & 0xffffu);
  const float d1 = f16_bits_to_f32(sc >> 16);
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] += __builtin_fmaf(d0, a[m][0], d1 * a[m][1]);
}

// kMode: 0 = x' fp32, 1 = x' bf16, 2 = raw fp32 x, 3 = raw bf16 x (rotated here).
// Computes MC activation rows (row stride ldx bytes) against all N weight rows.
template <int MC>
constexpr int max_threads() { return MC == 1 ? kMaxThreads : kMaxThreads / 2; }

template <int J, int R, int MC, int kMode>
__global__ __launch_bounds__(max_threads<MC>()) void gemv_kernel(const uint4* __restrict__ packed,
                                                           const uint32_t* __restrict__ scales,
                                                           uint32_t N, uint32_t nb, uint32_t mask,
                                                           const uint8_t* __restrict__ x, int64_t ldx,
                                                           Codebook cb, float* __restrict__ y, int64_t ldy) {
  __shared__ float lut[16];
  __shared__ float red[R * MC][kMaxThreads / 64];
  const int T = blockDim.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = T >> 6;
  if (tid < 16) lut[tid] = cb.c[tid];

  float xr[J][MC][32];
  bool valid[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t b = tid + j * T;
    valid[j] = b < nb;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      if (valid[j]) {
        const uint8_t* row = x + m * ldx;
        if constexpr (kMode == 1 || kMode == 3) {
          load_block<true>(row + (size_t)b * 64, xr[j][m]);
        } else {
          load_block<false>(row + (size_t)b * 128, xr[j][m]);
        }
        if constexpr (kMode >= 2) {
          apply_signs(xr[j][m], mask);
          fwht32(xr[j][m]);
#pragma unroll
          for (int i = 0; i < 32; ++i) xr[j][m][i] = xr[j][m][i] * kInvSqrt32;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) xr[j][m][i] = 0.f;
      }
    }
  }
  __syncthreads();

  for (uint32_t row0 = blockIdx.x * R; row0 < N; row0 += gridDim.x * R) {
    uint4 p[R][J];
    uint32_t s[R][J];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t b = tid + j * T;
        if (valid[j] && row0 + r < N) {
          const size_t g = (size_t)(row0 + r) * nb + b;
          p[r][j] = packed[g];
          s[r][j] = scales[g];
        } else {
          p[r][j] = make_uint4(0u, 0u, 0u, 0u);
          s[r][j] = 0u;
        }
      }
    }
    float acc[R][MC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int m = 0; m < MC; ++m) acc[r][m] = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) block_dot<MC>(p[r][j], s[r][j], xr[j], lut, acc[r]);
#pragma unroll
      for (int m = 0; m < MC; ++m) acc[r][m] = wave_sum(acc[r][m]);
    }
    if (nwaves == 1) {
      if (lane < R * MC) {
        const int r = lane / MC, m = lane % MC;
        float v = 0.f;
#pragma unroll
        for (int rr = 0; rr < R; ++rr)
#pragma unroll
          for (int mm = 0; mm < MC; ++mm) v = (rr == r && mm == m) ? acc[rr][mm] : v;
        if (row0 + r < N) y[m * ldy + row0 + r] = v;
      }
    } else {
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < MC; ++m) red[r * MC + m][wave] = acc[r][m];
      }
      __syncthreads();
      if (tid < R * MC) {
        const int r = tid / MC, m = tid % MC;
        if (row0 + r < N) {
          float v = 0.f;
          for (int w = 0; w < nwaves; ++w) v += red[tid][w];
          y[m * ldy + row0 + r] = v;
        }
      }
      __syncthreads();
    }
  }
}

template <int J, int R, int MC>
void launch_jm(const uint4* pk, const uint32_t* sc, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x,
               int64_t ldx, int mode, float* y, int64_t ldy, int T, hipStream_t s) {
  const Codebook& cb = host_codebook();
  uint32_t tiles = (N + R - 1) / R;
  uint32_t grid = tiles < (1u << 30) ? tiles : (1u << 30);
  switch (mode) {
    case 0: hipLaunchKernelGGL((gemv_kernel<J, R, MC, 0>), dim3(grid), dim3(T), 0, s, pk, sc, N, nb, mask, x, ldx, cb, y, ldy); break;
    case 1: hipLaunchKernelGGL((gemv_kernel<J, R, MC, 1>), dim3(grid), dim3(T), 0, s, pk, sc, N, nb, mask, x, ldx, cb, y, ldy); break;
    case 2: hipLaunchKernelGGL((gemv_kernel<J, R, MC, 2>), dim3(grid), dim3(T), 0, s, pk, sc, N, nb, mask, x, ldx, cb, y, ldy); break;
    default: hipLaunchKernelGGL((gemv_kernel<J, R, MC, 3>), dim3(grid), dim3(T), 0, s, pk, sc, N, nb, mask, x, ldx, cb, y, ldy); break;
  }
}

// Blocks per lane J and threads T for a given K: T*J >= nb, T a multiple of
// 64 and at most max_threads (1024 for one activation row, 512 -- a 256-VGPR
// budget -- when several rows share the registers).
void shape_for(uint32_t nb, int max_t, int& J, int& T) {
  J = (int)((nb + max_t - 1) / max_t);
  const uint32_t per = (nb + J - 1) / J;
  T = (int)((per + 63) / 64 * 64);
}

template <int MC>
void launch_mc(const uint4* pk, const uint32_t* sc, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x,
               int64_t ldx, int mode, float* y, int64_t ldy, hipStream_t s) {
  int J, T;
  shape_for(nb, max_threads<MC>(), J, T);
  constexpr int R = MC == 1 ? 4 : 2;
  switch (J) {
    case 1: launch_jm<1, R, MC>(pk, sc, N, nb, mask, x, ldx, mode, y, ldy, T, s); break;
    case 2: launch_jm<2, R, MC>(pk, sc, N, nb, mask, x, ldx, mode, y, ldy, T, s); break;
    case 3: launch_jm<3, R, MC>(pk, sc, N, nb, mask, x, ldx, mode, y, ldy, T, s); break;
    default: launch_jm<4, R, MC>(pk, sc, N, nb, mask, x, ldx, mode, y, ldy, T, s); break;
  }
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                       const void* x, bool xbf16, bool rotated, float* y, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  const int mode = rotated ? (xbf16 ? 1 : 0) : (xbf16 ? 3 : 2);
  launch_mc<1>(reinterpret_cast<const uint4*>(packed), reinterpret_cast<const uint32_t*>(scales), (uint32_t)N, nb,
               mask, static_cast<const uint8_t*>(x), 0, mode, y, 0, s);
  return hipGetLastError();
}

// VALU path of tq_gemm for M < 16: activation rows in chunks held in
// registers (fp32), one launch per chunk; the chunk is 4 rows when a lane
// owns one K-block, 2 when it owns two, else 1 (32 VGPRs per row per block).
hipError_t launch_gemm_valu(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                            const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  int J, T;
  shape_for(nb, max_threads<2>(), J, T);
  const int64_t max_mc = J == 1 ? 4 : (J == 2 ? 2 : 1);
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(scales);
  const int mode = xbf16 ? 1 : 0;
  const int64_t xs = xbf16 ? 2 : 4;
  const uint8_t* xb = static_cast<const uint8_t*>(xr);
  for (int64_t m0 = 0; m0 < M;) {
    const int64_t left = M - m0;
    const uint8_t* xm = xb + m0 * ldx * xs;
    float* ym = y + m0 * ldy;
    if (left >= 4 && max_mc >= 4) {
      launch_mc<4>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, s);
      m0 += 4;
    } else if (left >= 2 && max_mc >= 2) {
      launch_mc<2>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, s);
      m0 += 2;
    } else {
      launch_mc<1>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, s);
      m0 += 1;
    }
  }
  return hipGetLastError();
}

}  // namespace tq
