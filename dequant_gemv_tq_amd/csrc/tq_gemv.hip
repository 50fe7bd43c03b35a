// Fused TQ4_1S GEMV (and the VALU small-batch GEMM) on gfx950:
//   y[m, n] = sum_b [ d0 * sum_{i<16} c[idx_i] x'_m,i + d1 * sum_{i>=16} c[idx_i] x'_m,i ]
// computed in the rotated domain with float32 accumulation.
//
// TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160), decode-speed
// section (paragraph on why CUDA differs): the activation is rotated once so
// dequantization becomes a centroid lookup times a scale; the rotation is
// amortized over many rows (the Metal kernel's NR0 = 8) and the fused
// kernel must not let on-chip memory pressure starve occupancy (the cause of
// a 27B decode regression).
//
// MI355X design (HBM-bound: 0.625 B per weight; ~3 VALU lane-ops per weight
// are available at 8 TB/s, so the decode must cost well under that):
//   * Pair lookup table.  A byte of packed nibbles holds two indices; a
//     256-entry table of (c[lo], c[hi]) float pairs turns it into two
//     weights with one ds_read_b64.  The table is replicated 32 times and
//     entry e of copy l%32 sits at LDS byte (e << 8) | 8 (l % 32), so the 16
//     lanes an LDS cycle serves always hit 16 distinct bank pairs (no
//     conflicts), and the address is ONE v_perm_b32 that drops byte k of
//     the packed word next to the lane offset.  Per two weights: 1 v_perm,
//     1 ds_read_b64, 2 FMAs -- 1.5 VALU ops per weight, exact float32.
//   * Registers hold the rotated activation of the K-blocks a lane owns
//     (b = lane_k + j * TK) for the whole kernel; the rotation (when the
//     activation arrives unrotated) is done once per workgroup in the
//     prologue.
//   * Persistent workgroups walk row tiles with the next tile's 16-byte
//     nibble loads and 4-byte scale loads issued before the current tile is
//     computed (two tiles in flight per wavefront).
//   * A wavefront ends a tile with R*MC partial sums per lane; a transposed
//     butterfly (v_permlane32_swap, v_permlane16_swap, DPP) halves the set
//     at every cross-lane step, ~2.5 VALU ops per row instead of ~11.
//   * Several wavefronts along K (TK = 64 * WK lanes per row slot) combine
//     through a small double-buffered LDS array, one barrier per tile.
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kCopies = 32;                       // LUT copies: one per lane of a 32-lane group
constexpr int kLutBytes = 256 * kCopies * 8;      // 64 KiB

template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kHalfMirror = 0x141;  // lane i <-> 7 - i within each 8

__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Reduce V (1, 2, 4 or 8) values per lane across the 64 lanes.  On return
// v[0] of lane l holds the wavefront total of value number
//   V = 8: (l >> 3) & 7,   V = 4: (l >> 4) & 3,   V = 2: (l >> 5) & 1,   V = 1: 0.
// permlane32_swap(a, b) -> ([a_lo, b_lo], [a_hi, b_hi]) and permlane16_swap
// does the same per 16-lane row, so a swap plus an add folds two values and
// two lane halves at once.
template <int V>
__device__ __forceinline__ void wave_reduce(float (&v)[V], int lane) {
  if constexpr (V == 1) {
    float a = v[0], b = v[0];
    swap32(a, b);
    v[0] = a + b;
    a = v[0];
    b = v[0];
    swap16(a, b);
    v[0] = a + b;
  } else {
#pragma unroll
    for (int r = 0; r < V / 2; ++r) {          // lanes 0-31 keep value r, 32-63 keep r + V/2
      float a = v[r], b = v[r + V / 2];
      swap32(a, b);
      v[r] = a + b;
    }
    if constexpr (V == 2) {
      float a = v[0], b = v[0];
      swap16(a, b);
      v[0] = a + b;
    } else {
#pragma unroll
      for (int r = 0; r < V / 4; ++r) {        // 16-lane rows 0,2 keep r, rows 1,3 keep r + V/4
        float a = v[r], b = v[r + V / 4];
        swap16(a, b);
        v[r] = a + b;
      }
    }
  }
  if constexpr (V == 8) {
    const bool hi = (lane >> 3) & 1;           // lanes 8-15 of each row keep value 1
    const float keep = hi ? v[1] : v[0];
    const float give = hi ? v[0] : v[1];
    v[0] = keep + dpp<kRowRor8>(give);
    v[0] += dpp<kHalfMirror>(v[0]);
  } else {
    v[0] += dpp<kRowRor8>(v[0]);
    v[0] += dpp<kRowRor4>(v[0]);
  }
  v[0] += dpp<kQuadXor2>(v[0]);
  v[0] += dpp<kQuadXor1>(v[0]);
}

template <int MC>
__device__ __forceinline__ void decode_block(const uint4& p, uint32_t sc, const float (&x)[MC][32],
                                             const uint8_t* lut, uint32_t laneoff, float (&acc)[MC]) {
  const uint32_t w[4] = {p.x, p.y, p.z, p.w};
  // All 16 pair lookups of the block are issued before the first FMA so the
  // LDS latency is paid once per block, not once per byte.
  float2 c[16];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t addr = __builtin_amdgcn_perm(w[q], laneoff, 0x0C0C0000u | ((4u + k) << 8));
      c[4 * q + k] = *reinterpret_cast<const float2*>(lut + addr);
    }
  float a[MC][2];
#pragma unroll
  for (int m = 0; m < MC; ++m) a[m][0] = a[m][1] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      a[m][i >> 3] = __builtin_fmaf(c[i].x, x[m][2 * i], a[m][i >> 3]);
      a[m][i >> 3] = __builtin_fmaf(c[i].y, x[m][2 * i + 1], a[m][i >> 3]);
    }
  }
  const float d0 = f16_bits_to_f32(sc & 0xffffu);
  const float d1 = f16_bits_to_f32(sc >> 16);
#pragma unroll
  for (int m = 0; m < MC; ++m) acc[m] = __builtin_fmaf(d0, a[m][0], __builtin_fmaf(d1, a[m][1], acc[m]));
}

// kMode: 0 = x' fp32, 1 = x' bf16, 2 = raw fp32 x, 3 = raw bf16 x (rotated in the prologue).
// kPrefetch: keep the next tile's loads in flight while the current one is
// computed (two register sets), otherwise rely on other wavefronts.
template <int J, int R, int MC, int kMode, int kMaxT, bool kPrefetch>
__global__ __launch_bounds__(kMaxT) void gemv_kernel(const uint4* __restrict__ packed,
                                                     const uint32_t* __restrict__ scales, uint32_t N, uint32_t nb,
                                                     uint32_t mask, const uint8_t* __restrict__ x, int64_t ldx,
                                                     Codebook cb, float* __restrict__ y, int64_t ldy, int TK,
                                                     uint32_t tiles) {
  constexpr int V = R * MC;
  static_assert(V == 1 || V == 2 || V == 4 || V == 8, "R * MC must be 1, 2, 4 or 8");
  constexpr bool kXbf16 = kMode == 1 || kMode == 3;
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  __shared__ float red[2][kMaxT / 64][V];
  __shared__ float c16[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int slot = tid / TK;                  // row slot of this thread
  const int lk = tid - slot * TK;             // lane index along K
  const int wk = lk >> 6;                     // wavefront index along K within the slot
  const int WK = TK >> 6;
  const int S = blockDim.x / TK;
  const uint32_t laneoff = (uint32_t)(lane & (kCopies - 1)) * 8u;

  // Loads are branch-free: indices are clamped into the tensor, so a lane
  // past the last block or row reads valid memory whose contribution is
  // discarded (x' is zero past the last block; rows past N are not written).
  uint4 pa[R][J], pb[kPrefetch ? R : 1][kPrefetch ? J : 1];
  uint32_t sa[R][J], sb[kPrefetch ? R : 1][kPrefetch ? J : 1];
  auto load_tile = [&](uint32_t t, auto& p, auto& s) {
    const uint32_t row0 = (t * S + slot) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = min(row0 + r, N - 1);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t b = min((uint32_t)(lk + j * TK), nb - 1);
        const size_t g = (size_t)row * nb + b;
        p[r][j] = packed[g];
        s[r][j] = scales[g];
      }
    }
  };

  // The first tile's weights and the activation are requested before
  // anything else so that their latency overlaps the table fill.
  const uint32_t G = gridDim.x;
  uint32_t t = blockIdx.x;
  load_tile(t, pa, sa);

  float xr[J][MC][32];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t b = min((uint32_t)(lk + j * TK), nb - 1);
#pragma unroll
    for (int m = 0; m < MC; ++m) load_block<kXbf16>(x + m * ldx + (size_t)b * (kXbf16 ? 64 : 128), xr[j][m]);
  }

  // Pair table: entry e, copy c -> (c[e & 15], c[e >> 4]).  Item i writes
  // copies 2 (i % 16) and 2 (i % 16) + 1 of entry i / 16 with one 16-byte
  // store, so consecutive lanes fill consecutive bytes of a 256-byte table
  // row (no bank conflicts; a lane stride of 256 B would put every lane of a
  // wavefront on one bank).
  stage_centroids(cb, c16);
  __syncthreads();
  for (int i = tid; i < 256 * (kCopies / 2); i += blockDim.x) {
    const int e = i >> 4, c = 2 * (i & 15);
    const float lo = c16[e & 15], hi = c16[e >> 4];
    *reinterpret_cast<float4*>(lut + (e << 8) + c * 8) = make_float4(lo, hi, lo, hi);
  }

  // Unrotated activations are rotated per lane while the first tile's loads
  // are in flight: x' = FWHT32(D x); the 1/sqrt(32) is applied once to each
  // finished row sum instead of to every element.
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool inside = (uint32_t)(lk + j * TK) < nb;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      if constexpr (kMode >= 2) {
        apply_signs(xr[j][m], mask);
        fwht32(xr[j][m]);
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) xr[j][m][i] = inside ? xr[j][m][i] : 0.f;
    }
  }
  __syncthreads();
  constexpr float kOutScale = kMode >= 2 ? kInvSqrt32 : 1.0f;

  int parity = 0;
  auto do_tile = [&](uint32_t tt, const auto& p, const auto& s) {
    float v[V];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float acc[MC];
#pragma unroll
      for (int m = 0; m < MC; ++m) acc[m] = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) decode_block<MC>(p[r][j], s[r][j], xr[j], lut, laneoff, acc);
#pragma unroll
      for (int m = 0; m < MC; ++m) v[r * MC + m] = acc[m];
    }
    wave_reduce<V>(v, lane);
    const uint32_t row0 = (tt * S + slot) * R;
    const bool writer = (lane & (64 / V - 1)) == 0;
    const int vi = lane / (64 / V);
    if (WK == 1) {
      if (writer) {
        const uint32_t row = row0 + vi / MC;
        if (row < N) y[(vi % MC) * ldy + row] = v[0] * kOutScale;
      }
    } else {
      if (writer) red[parity][slot * WK + wk][vi] = v[0];
      __syncthreads();
      if (tid < S * V) {
        const int s2 = tid / V, v2 = tid % V;
        const uint32_t row = (tt * S + s2) * R + v2 / MC;
        if (row < N) {
          float sum = 0.f;
          for (int w = 0; w < WK; ++w) sum += red[parity][s2 * WK + w][v2];
          y[(v2 % MC) * ldy + row] = sum * kOutScale;
        }
      }
      parity ^= 1;
    }
  };

  if constexpr (kPrefetch) {
    // Two tiles in flight per wavefront: ping-pong between register sets (no
    // copies, which would force a wait on the loads still in flight).
    // The prefetch is skipped (uniform branch) past the last tile: a wave
    // cannot retire while loads it issued are still in flight.
    while (t < tiles) {
      if (t + G < tiles) load_tile(t + G, pb, sb);
      __builtin_amdgcn_sched_barrier(0);      // keep the prefetch ahead of this tile's math
      do_tile(t, pa, sa);
      t += G;
      if (t >= tiles) break;
      if (t + G < tiles) load_tile(t + G, pa, sa);
      __builtin_amdgcn_sched_barrier(0);
      do_tile(t, pb, sb);
      t += G;
    }
  } else {
    while (true) {
      do_tile(t, pa, sa);
      t += G;
      if (t >= tiles) break;
      load_tile(t, pa, sa);
    }
  }
}

// ---------------------------------------------------------------------------
// launch configuration
// ---------------------------------------------------------------------------

struct Plan {
  int J;        // K-blocks per lane
  int TK;       // lanes per row slot (multiple of 64)
  int threads;  // workgroup size
};

// Lanes along K cover nb blocks with J per lane; row slots fill the workgroup
// up to max_t threads.
Plan plan_for(uint32_t nb, int max_t, int J) {
  Plan p;
  p.J = J;
  const uint32_t per = (nb + p.J - 1) / p.J;
  p.TK = (int)((per + 63) / 64 * 64);
  const int slots = max_t / p.TK > 0 ? max_t / p.TK : 1;
  p.threads = slots * p.TK;
  return p;
}

// Smallest J (blocks per lane) that fits nb into max_t lanes.
int min_j(uint32_t nb, int max_t) {
  int J = 1;
  while ((uint32_t)max_t * J < nb) ++J;
  return J;
}

// Persistent grid: enough resident wavefronts per CU for the VGPR budget of
// these kernels (about 16), one workgroup per CU for 1024-thread workgroups.
uint32_t grid_cap(int threads) {
  const int waves = threads / 64;
  const int per_cu = waves >= 16 ? 1 : 16 / waves;
  return (uint32_t)(device_cu_count() * per_cu);
}

template <int J, int R, int MC, int kMaxT, bool kPrefetch>
void launch_cfg(const uint4* pk, const uint32_t* sc, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x,
                int64_t ldx, int mode, float* y, int64_t ldy, const Plan& pl, hipStream_t s) {
  const Codebook& cb = host_codebook();
  const int S = pl.threads / pl.TK;
  const uint32_t rows_per_tile = (uint32_t)(S * R);
  const uint32_t tiles = (N + rows_per_tile - 1) / rows_per_tile;
  const uint32_t cap = grid_cap(pl.threads);
  const uint32_t grid = tiles < cap ? tiles : cap;
#define TQ_GEMV_LAUNCH(M_)                                                                                     \
  hipLaunchKernelGGL((gemv_kernel<J, R, MC, M_, kMaxT, kPrefetch>), dim3(grid), dim3(pl.threads), 0, s, pk, sc, N, \
                     nb, mask, x, ldx, cb, y, ldy, pl.TK, tiles)
  switch (mode) {
    case 0: TQ_GEMV_LAUNCH(0); break;
    case 1: TQ_GEMV_LAUNCH(1); break;
    case 2: TQ_GEMV_LAUNCH(2); break;
    default: TQ_GEMV_LAUNCH(3); break;
  }
#undef TQ_GEMV_LAUNCH
}

// GEMV configuration for one activation row.
struct GemvConfig {
  int J;          // K-blocks per lane (1..4)
  int R;          // rows per wavefront per tile (2 or 4)
  int max_t;      // workgroup size bound (1024 or 512)
  bool prefetch;  // second register set for the next tile
};

// Measured on MI355X over the decode shapes (K = 4096..28672): one K-block
// per lane, two rows per wavefront per tile and the register prefetch are
// the fastest choice for every shape; K > 32768 takes more blocks per lane
// (and no prefetch, which would spill).
GemvConfig choose_gemv_config(uint32_t nb, uint32_t N) {
  (void)N;
  GemvConfig c;
  c.max_t = 1024;
  c.J = min_j(nb, c.max_t);
  c.R = 2;
  c.prefetch = true;
  return c;
}

template <int J>
void launch_gemv_j(const uint4* pk, const uint32_t* sc, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x,
                   int mode, float* y, const GemvConfig& c, hipStream_t s) {
  const Plan pl = plan_for(nb, c.max_t, J);
  // The second register set only fits without spills at one block per lane.
  launch_cfg<J, 2, 1, 1024, J == 1>(pk, sc, N, nb, mask, x, 0, mode, y, 0, pl, s);
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                       const void* x, bool xbf16, bool rotated, float* y, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  const int mode = rotated ? (xbf16 ? 1 : 0) : (xbf16 ? 3 : 2);
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(scales);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const GemvConfig c = choose_gemv_config(nb, (uint32_t)N);
  switch (c.J) {
    case 1: launch_gemv_j<1>(pk, sc, (uint32_t)N, nb, mask, xb, mode, y, c, s); break;
    case 2: launch_gemv_j<2>(pk, sc, (uint32_t)N, nb, mask, xb, mode, y, c, s); break;
    case 3: launch_gemv_j<3>(pk, sc, (uint32_t)N, nb, mask, xb, mode, y, c, s); break;
    default: launch_gemv_j<4>(pk, sc, (uint32_t)N, nb, mask, xb, mode, y, c, s); break;
  }
  return hipGetLastError();
}

// VALU path of tq_gemm for M < 16: chunks of MC = 4, 2 or 1 activation rows
// held in registers (float32, 32 VGPRs per row per owned block), one launch
// per chunk; workgroups of at most 256 threads leave 256 VGPRs per lane.
hipError_t launch_gemm_valu(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                            const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / kBlock);
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(scales);
  const int mode = xbf16 ? 1 : 0;
  const int64_t xs = xbf16 ? 2 : 4;
  const uint8_t* xb = static_cast<const uint8_t*>(xr);
  for (int64_t m0 = 0; m0 < M;) {
    const int64_t left = M - m0;
    const uint8_t* xm = xb + m0 * ldx * xs;
    float* ym = y + m0 * ldy;
    if (left >= 4 && nb <= 256) {
      const Plan pl = plan_for(nb, 256, 1);
      launch_cfg<1, 2, 4, 256, false>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, pl, s);
      m0 += 4;
    } else if (left >= 2 && nb <= 512) {
      const Plan pl = plan_for(nb, 512, 1);
      launch_cfg<1, 2, 2, 512, false>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, pl, s);
      m0 += 2;
    } else {
      const Plan pl = plan_for(nb, 1024, min_j(nb, 1024));
      switch (pl.J) {
        case 1: launch_cfg<1, 2, 1, 1024, false>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, pl, s); break;
        case 2: launch_cfg<2, 2, 1, 1024, false>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, pl, s); break;
        case 3: launch_cfg<3, 2, 1, 1024, false>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, pl, s); break;
        default: launch_cfg<4, 2, 1, 1024, false>(pk, sc, (uint32_t)N, nb, 0u, xm, ldx * xs, mode, ym, ldy, pl, s); break;
      }
      m0 += 1;
    }
  }
  return hipGetLastError();
}

}  // namespace tq
