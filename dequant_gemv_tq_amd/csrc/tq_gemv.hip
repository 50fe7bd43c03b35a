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
//   * Persistent workgroups walk row tiles.  A wavefront keeps two register
//     sets of tile loads (16-byte nibble loads, 4-byte scale loads) in
//     flight; only the first tile is requested before the activation has
//     arrived, because a larger first burst of weight requests delays the
//     activation, which every tile waits for.  Row addresses are
//     wavefront-uniform (scalar) plus a fixed 32-bit lane offset.
//   * The decode is VALU-bound in the steady state (counters: ~65% VALU busy
//     per SIMD over a whole gate|up launch, LDS waits ~3%), so per-tile
//     overhead matters: a lane keeps the partial sums of several tiles and
//     one transposed butterfly (v_permlane32_swap, v_permlane16_swap, DPP)
//     reduces them at once, ~3-5 VALU ops per row instead of ~10.
//   * Several wavefronts along K (TK = 64 * WK lanes per row slot) leave
//     their partial sums in an LDS ring that is combined every 32 tiles.
#include <map>
#include <mutex>
#include <tuple>
#include <type_traits>

#include "tq_internal.hpp"

namespace tq {
namespace {


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

// ---------------------------------------------------------------------------
// Weight formats.  Each holds its device pointers and provides the per-lane
// data of one 32-element block (Raw), its load, and the decode-and-multiply
// of one block against MC activation rows held in registers.
// ---------------------------------------------------------------------------

// TQ4_1S: 16 bytes of nibble indices and an fp16 scale pair per block;
// decoded through the replicated pair table (1 v_perm + 1 ds_read_b64 + 2
// FMAs per two weights).
struct FmtTQ4 {
  static constexpr bool kLut = true;
  struct Raw {
    uint4 p;
    uint32_t s;
  };
  const uint4* codes;
  const uint32_t* scales;
  __device__ __forceinline__ void prepare() {}
  // Block b of row `row` (wavefront-uniform): a scalar row base plus the
  // lane's 32-bit byte offset.
  __device__ __forceinline__ Raw load(uint32_t row, uint32_t nb, uint32_t b) const {
    const uint8_t* cr = reinterpret_cast<const uint8_t*>(codes) + (size_t)row * nb * 16u;
    const uint8_t* sr = reinterpret_cast<const uint8_t*>(scales) + (size_t)row * nb * 4u;
    return Raw{*reinterpret_cast<const uint4*>(cr + (b << 4)), *reinterpret_cast<const uint32_t*>(sr + (b << 2))};
  }
  template <int MC>
  __device__ __forceinline__ void decode(const Raw& r, const float (&x)[MC][32], const uint8_t* lut,
                                         uint32_t laneoff, float (&acc)[MC]) const {
    const uint32_t w[4] = {r.p.x, r.p.y, r.p.z, r.p.w};
    // All 16 pair lookups of the block are issued before the first FMA so
    // the LDS latency is paid once per block, not once per byte.
    float2 c[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) c[4 * q + k] = *reinterpret_cast<const float2*>(lut + pair_addr(w[q], laneoff, k));
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
    const float d0 = f16_bits_to_f32(r.s & 0xffffu);
    const float d1 = f16_bits_to_f32(r.s >> 16);
#pragma unroll
    for (int m = 0; m < MC; ++m) acc[m] = __builtin_fmaf(d0, a[m][0], __builtin_fmaf(d1, a[m][1], acc[m]));
  }
};

// NVFP4: 16 bytes of E2M1 codes (element 2j in the low nibble of byte j),
// two E4M3 block scales per 32 elements and one float32 tensor scale.  The
// codes are decoded by v_cvt_scalef32_pk_f32_fp4 (two per instruction, scale
// 1, exact); each 16-element half-sum is multiplied once by its effective
// scale fl(e4m3 * s_t), the value the oracle's dequantization uses.
struct FmtNVFP4 {
  static constexpr bool kLut = false;
  struct Raw {
    uint4 p;
    uint32_t s;
  };
  const uint4* codes;
  const uint16_t* scales;
  const float* tscale;
  float st;
  __device__ __forceinline__ void prepare() { st = *tscale; }
  __device__ __forceinline__ Raw load(uint32_t row, uint32_t nb, uint32_t b) const {
    const uint8_t* cr = reinterpret_cast<const uint8_t*>(codes) + (size_t)row * nb * 16u;
    const uint8_t* sr = reinterpret_cast<const uint8_t*>(scales) + (size_t)row * nb * 2u;
    return Raw{*reinterpret_cast<const uint4*>(cr + (b << 4)), *reinterpret_cast<const uint16_t*>(sr + (b << 1))};
  }
  template <int MC>
  __device__ __forceinline__ void decode(const Raw& r, const float (&x)[MC][32], const uint8_t*, uint32_t,
                                         float (&acc)[MC]) const {
    const uint32_t w[4] = {r.p.x, r.p.y, r.p.z, r.p.w};
    float a[MC][2];
#pragma unroll
    for (int m = 0; m < MC; ++m) a[m][0] = a[m][1] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // Byte k of word q holds elements 8 q + 2 k (low nibble) and 8 q + 2 k + 1.
      const decltype(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(0u, 1.0f, 0)) v[4] = {
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 0), __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 1),
          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 2), __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 3)};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = 4 * q + k;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
          a[m][i >> 3] = __builtin_fmaf(v[k][0], x[m][2 * i], a[m][i >> 3]);
          a[m][i >> 3] = __builtin_fmaf(v[k][1], x[m][2 * i + 1], a[m][i >> 3]);
        }
      }
    }
    const float e0 = e4m3_decode(r.s & 0xffu) * st;
    const float e1 = e4m3_decode((r.s >> 8) & 0xffu) * st;
#pragma unroll
    for (int m = 0; m < MC; ++m) acc[m] = __builtin_fmaf(e0, a[m][0], __builtin_fmaf(e1, a[m][1], acc[m]));
  }
};

// MXFP6: 24 bytes of E3M2 codes per block (element i at bits 6i..6i+5 of the
// little-endian 192-bit block) and one E8M0 scale 2^(byte - 127).  One
// v_cvt_scalef32_pk32_f32_bf6 decodes the whole block (scale 1, exact); the
// block sum is scaled by ldexp, exact for every byte.
struct FmtMXFP6 {
  static constexpr bool kLut = false;
  struct Raw {
    uint2 c[3];
    uint32_t s;
  };
  const uint2* codes;
  const uint8_t* scales;
  __device__ __forceinline__ void prepare() {}
  __device__ __forceinline__ Raw load(uint32_t row, uint32_t nb, uint32_t b) const {
    const uint8_t* cr = reinterpret_cast<const uint8_t*>(codes) + (size_t)row * nb * 24u;
    const uint2* src = reinterpret_cast<const uint2*>(cr + b * 24u);
    return Raw{{src[0], src[1], src[2]}, scales[(size_t)row * nb + b]};
  }
  template <int MC>
  __device__ __forceinline__ void decode(const Raw& r, const float (&x)[MC][32], const uint8_t*, uint32_t,
                                         float (&acc)[MC]) const {
    typedef unsigned u32x6 __attribute__((ext_vector_type(6)));
    const u32x6 bits = {r.c[0].x, r.c[0].y, r.c[1].x, r.c[1].y, r.c[2].x, r.c[2].y};
    const auto v = __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(bits, 1.0f);
    float a[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      a[m] = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) a[m] = __builtin_fmaf(v[i], x[m][i], a[m]);
      acc[m] += __builtin_ldexpf(a[m], (int)r.s - 127);
    }
  }
};

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Bit e of kHadPar[i & 7] (byte i & 7 of the constant) is the parity of
// (i & e): the sign pattern of Sylvester Hadamard entries H[i][8 b + e].
constexpr unsigned long long kHadPar = 0x963C5AF066CCAA00ull;

// x' = H D x for the 64 blocks of one wavefront (lane l owns block l of the
// wavefront's range) on the matrix cores.  (H D)[i][k] = (-1)^(popcount(i & k)
// + mask_k) is +-1, exact in bf16, and so is a bf16 activation, so every
// product is exact and only the float32 accumulation rounds.  Per 32 blocks
// and half block h, one v_mfma_f32_32x32x16_bf16: the A operand is the
// matrix (lane l: row i = l % 32, columns k = 16 h + 8 (l / 32) + e), the B
// operand eight consecutive activation elements (lane l: block l % 32 of the
// tile, elements k = 16 h + 8 (l / 32) + e), xq[T][h] for tile T.  Lane l,
// register r of tile T's result holds element 8 (r / 4) + 4 (l / 32) + r % 4
// of block 32 T + l % 32; one permlane32 swap per register pair gives each
// lane the other half of its own block, so v[i] = x'_i on return.
__device__ __forceinline__ void rotate_blocks_mfma(const uint4 (&xq)[2][2], uint32_t mask, int lane,
                                                   float (&v)[32]) {
  const uint32_t i = (uint32_t)lane & 31u, kb = 8u * ((uint32_t)lane >> 5);
  const uint32_t par = (uint32_t)(kHadPar >> (8u * (i & 7u))) & 0xffu;
  bf16x8 A[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t base = 16u * (uint32_t)h + kb;                  // bits 3 and 4 only
    const uint32_t hi = (uint32_t)__builtin_popcount(i & base) & 1u;
    const uint32_t s8 = (par ^ (mask >> base) ^ (0u - hi)) & 0xffu;   // sign of element base + e at bit e
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      w[t] = 0x3F803F80u | (((s8 >> (2 * t)) & 1u) << 15) | (((s8 >> (2 * t + 1)) & 1u) << 31);
    A[h] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  f32x16 c[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    c[T] = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h)
      c[T] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[h], __builtin_bit_cast(bf16x8, xq[T][h]), c[T], 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float a = c[0][r], b = c[1][r];
    swap32(a, b);
    v[8 * (r / 4) + r % 4] = a;
    v[8 * (r / 4) + 4 + r % 4] = b;
  }
}

// One cross-lane stage of the 32-point FWHT when 8 consecutive lanes hold a
// block, 4 consecutive elements each: elements i and i + 4d sit in lanes
// l and l ^ d at the same position.  The lower lane forms a + b, the upper
// one a - b (a the lower lane's value), each with one rounding, exactly as
// the in-register butterfly does.
template <int D>
__device__ __forceinline__ void fwht_lane_stage(float (&v)[4], int lane) {
  const float sgn = (lane & D) ? -1.f : 1.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float p;
    if constexpr (D == 1) p = dpp<kQuadXor1>(v[e]);
    else if constexpr (D == 2) p = dpp<kQuadXor2>(v[e]);
    else p = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[e]), 0x101F));   // lane ^ 4 in 32
    v[e] = __builtin_fmaf(sgn, v[e], p);
  }
}

// Stage the activation of one GEMV in LDS as fp32 x' (rotated when kMode >=
// 2), once per workgroup.  Consecutive threads load consecutive 4-element
// groups, P groups per thread (coalesced: one request per cache line per
// workgroup instead of one per lane), all issued up front; the loads of a
// thread's unused groups are clamped to the tensor and discarded.  Once they
// arrive, the groups are rotated cooperatively (8 lanes per block, the
// butterfly stages in the same order as the per-lane transform) and block
// b, 16-byte chunk q is stored at float offset 32 b + 4 (q ^ (b % 8)):
// lanes that later read consecutive blocks then hit distinct banks.  The
// 1/sqrt(32) factor is left to the row sums.
template <int kMode, int P>
struct ActivationStage {
  static constexpr bool kBf16 = kMode == 1 || kMode == 3;
  uint32_t raw[P][kBf16 ? 2 : 4];

  __device__ __forceinline__ void load(const uint8_t* __restrict__ x, uint32_t K, int tid, int nthreads) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t e0 = min(4u * (uint32_t)(tid + p * nthreads), K - 4);
      if constexpr (kBf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(x + 2 * (size_t)e0);
        raw[p][0] = u.x; raw[p][1] = u.y;
      } else {
        const uint4 u = *reinterpret_cast<const uint4*>(x + 4 * (size_t)e0);
        raw[p][0] = u.x; raw[p][1] = u.y; raw[p][2] = u.z; raw[p][3] = u.w;
      }
    }
  }

  __device__ __forceinline__ void store(uint32_t K, uint32_t mask, float* xs, int tid, int nthreads) const {
    const int lane = tid & 63;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t e0 = 4u * (uint32_t)(tid + p * nthreads);
      if (e0 >= K) break;                // whole 8-lane groups leave together (K % 32 == 0)
      float v[4];
      if constexpr (kBf16) {
        v[0] = bf16_lo(raw[p][0]); v[1] = bf16_hi(raw[p][0]); v[2] = bf16_lo(raw[p][1]); v[3] = bf16_hi(raw[p][1]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(raw[p][e]);
      }
      if constexpr (kMode >= 2) {
        const uint32_t i0 = e0 & 31;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (((mask >> (i0 + e)) & 1u) << 31));
        float a = v[0], b = v[1];        // h = 1
        v[0] = a + b; v[1] = a - b;
        a = v[2]; b = v[3];
        v[2] = a + b; v[3] = a - b;
        a = v[0]; b = v[2];              // h = 2
        v[0] = a + b; v[2] = a - b;
        a = v[1]; b = v[3];
        v[1] = a + b; v[3] = a - b;
        fwht_lane_stage<1>(v, lane);     // h = 4
        fwht_lane_stage<2>(v, lane);     // h = 8
        fwht_lane_stage<4>(v, lane);     // h = 16
      }
      const uint32_t b = e0 >> 5, q = (e0 >> 2) & 7;
      *reinterpret_cast<float4*>(xs + 32 * b + 4 * (q ^ (b & 7))) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
};

// Largest K whose x' a workgroup stages in LDS next to the 64 KiB pair table.
constexpr int kStageFloats = 20480;
// Tiles whose cross-wavefront partial sums wait in LDS before being combined.
constexpr int kRing = 32;

// Work split of one launch, fixed on the host so that the prologue has no
// integer division: TK lanes per row slot (a multiple of 64), S slots per
// workgroup (S * TK threads), slot of wavefront w = (w * slot_mul) >> 8
// (exact for the at most 16 wavefronts of a workgroup), and workgroup g of G
// takes tiles g, g + G, ... : q + (g < r) of them.
struct GemvGrid {
  int TK;
  int S;
  uint32_t slot_mul;
  uint32_t G;
  uint32_t q;
  uint32_t r;
};

template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, F, I + 1>(static_cast<F&&>(f));
  }
}

// kMode: 0 = x' fp32, 1 = x' bf16, 2 = raw fp32 x, 3 = raw bf16 x (rotated in the prologue).
// kStage: stage x' in LDS once per workgroup with kStage groups of 4
// elements per thread (MC == 1, K <= kStageFloats); 0: every lane loads and
// rotates its own blocks.
// kDepth (1, 2 or 4): register sets of tile loads a wavefront keeps in
// flight; kEarly of them are requested at kernel start, the others once the
// wavefront has its part of the activation (a large first burst of weight
// requests delays the activation, which every tile waits for).
//
// Row sums are reduced across the wavefront in groups of V values (T tiles
// of R rows of MC activation rows, V = R MC T, usually 4): each lane keeps
// its V partial sums and one transposed butterfly reduces them all, about 3
// VALU operations per row instead of about 10 for a reduction of each row on
// its own.
template <typename Fmt, int J, int R, int MC, int kMode, int kMaxT, int kDepth, int kEarly, int kStage>
__global__ __launch_bounds__(kMaxT) void gemv_kernel(Fmt fmt, uint32_t N, uint32_t nb, uint32_t mask,
                                                     const uint8_t* __restrict__ x, int64_t ldx,
                                                     float* __restrict__ y, int64_t ldy, GemvGrid gg) {
  constexpr int RM = R * MC;                           // values per tile and lane
  static_assert(RM == 1 || RM == 2 || RM == 4 || RM == 8, "R * MC must be 1, 2, 4 or 8");
  // Tiles per reduction group: up to four rows' worth (one tile when a lane
  // owns several blocks), and no more than the register sets can hold at
  // the end of the list (the remaining tiles of a workgroup are computed
  // from registers only).
  constexpr int kT0 = (RM >= 4 || J > 1) ? 1 : 4 / RM;   // J > 1: x' alone takes 32 J registers
  constexpr int T = kT0 < (kDepth >= 4 ? 4 : 2) ? kT0 : (kDepth >= 4 ? 4 : 2);
  constexpr int V = RM * T;                            // values per reduction group
  static_assert(kDepth == 1 || kDepth == 2 || kDepth == 4, "kDepth must be 1, 2 or 4");
  static_assert(kEarly >= 1 && kEarly <= kDepth, "1 <= kEarly <= kDepth");
  constexpr int U = kDepth > T ? kDepth : T;           // tiles per loop iteration (both powers of two)
  constexpr bool kXbf16 = kMode == 1 || kMode == 3;
  static_assert(!kStage || MC == 1, "staged activations serve one row");
  // One LDS allocation with the pair table at offset 0, so a table address
  // is the v_perm result itself (a base above 64 KiB would not fit the
  // ds_read immediate and cost an add per lookup), then the staged x' and
  // the cross-wavefront partial sums.
  constexpr int kXsBytes = kStage ? kStageFloats * 4 : 0;
  constexpr int kRedBytes = kRing * (kMaxT / 64) * RM * 4;
  constexpr int kTable = Fmt::kLut ? kLutBytes : 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kTable + kXsBytes + kRedBytes];
  uint8_t* const lut = smem;
  float* const xs = reinterpret_cast<float*>(smem + kTable);
  float (*const red)[kMaxT / 64][RM] = reinterpret_cast<float (*)[kMaxT / 64][RM]>(smem + kTable + kXsBytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // TK is a multiple of 64, so the row slot and the wavefront's place along
  // K are wavefront-uniform: readfirstlane lets the row addressing run on
  // the scalar unit.
  const int TK = gg.TK, S = gg.S, nthreads = S * TK;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = (int)(((uint32_t)wave * gg.slot_mul) >> 8);   // row slot of this thread
  const int lk = tid - slot * TK;             // lane index along K
  const int wk = lk >> 6;                     // wavefront index along K within the slot
  const int WK = TK >> 6;
  const uint32_t laneoff = (uint32_t)(lane & (kCopies - 1)) * 8u;

  // Loads are branch-free: indices are clamped into the tensor, so a lane
  // past the last block or row reads valid memory whose contribution is
  // discarded (x' is zero past the last block; rows past N are not written).
  // The row is wavefront-uniform and the lane's block offset is fixed, so a
  // load is a scalar base plus one 32-bit lane offset.
  using Raw = typename Fmt::Raw;
  Raw ps[kDepth][R][J];
  uint32_t boff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) boff[j] = min((uint32_t)(lk + j * TK), nb - 1);
  fmt.prepare();
  auto load_tile = [&](uint32_t t, Raw (&p)[R][J]) {
    const uint32_t row0 = (t * S + slot) * R;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = min(row0 + r, N - 1);
#pragma unroll
      for (int j = 0; j < J; ++j)   // several blocks per lane: offsets recomputed (registers are scarce)
        p[r][j] = fmt.load(row, nb, J == 1 ? boff[j] : min((uint32_t)(lk + j * TK), nb - 1));
    }
  };

  const uint32_t G = gg.G;
  uint32_t t = blockIdx.x;
  const uint32_t n = gg.q + (t < gg.r ? 1u : 0u);      // this workgroup's tile count
  const uint32_t last = t + (n - 1) * G;               // and its last tile

  // The activation and the first kEarly tiles' weights are requested before
  // anything else so that their latency overlaps the table fill.
  float xr[J][MC][32];
  ActivationStage<kMode, kStage ? kStage : 1> xst;
  // A raw bf16 activation row with one block per lane is rotated on the
  // matrix cores: lane l loads the 16 bytes of blocks 32 T + l % 32 of the
  // wavefront's range that the MFMA B operand takes (rotate_blocks_mfma).
  constexpr bool kRotMfma = kMode == 3 && J == 1 && MC == 1 && !kStage;
  uint4 xq[2][2];
  if constexpr (kStage) {
    xst.load(x, nb * 32, tid, nthreads);
  } else if constexpr (kRotMfma) {
    const uint32_t wbase = (uint32_t)(lk - lane);           // 64 wk: the wavefront's first block
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t blk = min(wbase + 32u * (uint32_t)T + ((uint32_t)lane & 31u), nb - 1);
        xq[T][h] = *reinterpret_cast<const uint4*>(x + (size_t)blk * 64 + 32 * h + 16 * (lane >> 5));
      }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
      for (int m = 0; m < MC; ++m) load_block<kXbf16>(x + m * ldx + (size_t)boff[j] * (kXbf16 ? 64 : 128), xr[j][m]);
    }
  }
  static_for<kEarly>([&](auto ic) { load_tile(min(t + (uint32_t)ic.value * G, last), ps[ic.value]); });

  if constexpr (Fmt::kLut) fill_pair_lut(lut, tid, nthreads);

  if constexpr (kStage) {
    xst.store(nb * 32, mask, xs, tid, nthreads);
    __builtin_amdgcn_sched_barrier(0);
    static_for<kDepth - kEarly>([&](auto ic) {
      load_tile(min(t + (uint32_t)(kEarly + ic.value) * G, last), ps[kEarly + ic.value]);
    });
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t b0 = (uint32_t)(lk + j * TK);
      const bool inside = b0 < nb;
      const uint32_t b = boff[j];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 u = *reinterpret_cast<const float4*>(xs + 32 * b + 4 * (q ^ (b & 7)));
        xr[j][0][4 * q + 0] = inside ? u.x : 0.f;
        xr[j][0][4 * q + 1] = inside ? u.y : 0.f;
        xr[j][0][4 * q + 2] = inside ? u.z : 0.f;
        xr[j][0][4 * q + 3] = inside ? u.w : 0.f;
      }
    }
  } else {
    if constexpr (Fmt::kLut) __syncthreads();   // the pair table: before this wavefront waits for its x
    // Unrotated activations are rotated per lane while the first tile's
    // loads are in flight: x' = FWHT32(D x); the 1/sqrt(32) is applied once
    // to each finished row sum instead of to every element.
    if constexpr (kRotMfma) {
      rotate_blocks_mfma(xq, mask, lane, xr[0][0]);
      const bool inside = (uint32_t)lk < nb;
#pragma unroll
      for (int i = 0; i < 32; ++i) xr[0][0][i] = inside ? xr[0][0][i] : 0.f;
    } else {
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
    }
    __builtin_amdgcn_sched_barrier(0);
    static_for<kDepth - kEarly>([&](auto ic) {
      load_tile(min(t + (uint32_t)(kEarly + ic.value) * G, last), ps[kEarly + ic.value]);
    });
    __builtin_amdgcn_sched_barrier(0);
  }
  constexpr float kOutScale = kMode >= 2 ? kInvSqrt32 : 1.0f;

  // Rows split over WK > 1 wavefronts: each wavefront leaves its partial
  // sums for tile number i (of this workgroup) in ring slot i % kRing and
  // runs on; the partials are combined and y written once per kRing tiles
  // and after the last tile.  Wavefronts thus never wait for each other per
  // tile (a per-tile barrier would pace every tile by the slowest of the
  // workgroup's loads).  The tile count is uniform over the workgroup, so
  // every wavefront reaches the same barriers.
  const uint32_t t0 = t;
  auto flush = [&](uint32_t first, uint32_t cnt) {
    __syncthreads();
    for (uint32_t e = tid; e < cnt * (uint32_t)(S * RM); e += (uint32_t)nthreads) {
      const uint32_t jl = e / (uint32_t)(S * RM), rem = e - jl * (uint32_t)(S * RM);
      const int s2 = (int)rem / RM, v2 = (int)rem % RM;
      const uint32_t li = first + jl;
      const uint32_t row = ((t0 + li * G) * S + s2) * R + v2 / MC;
      if (row < N) {
        float sum = 0.f;
        for (int w = 0; w < WK; ++w) sum += red[li % kRing][s2 * WK + w][v2];
        y[(v2 % MC) * ldy + row] = sum * kOutScale;
      }
    }
    __syncthreads();                        // the ring slots are rewritten next
  };

  // Tiles i .. i + U - 1 of this workgroup's list in one pass of the loop:
  // tile i + u is computed from register set u % kDepth (when it exists),
  // which is then reloaded with tile i + u + kDepth.  The reloads are
  // unconditional, with the tile index clamped to `last` (the clamped loads
  // at the end re-read the last tile, cache hits, and are discarded), so
  // every path into a use of a register set carries the same loads and the
  // compiler's wait counts stay exact.
  // Tiles i .. i + U - 1 of this workgroup's list in one pass of the loop:
  // tile i + u is computed from register set u % kDepth, which is then
  // reloaded with tile i + u + kDepth.  The reloads are unconditional, with
  // the tile index clamped to `last` (the clamped loads at the end re-read
  // the last tile, cache hits, and are discarded), so every path into a use
  // of a register set carries the same loads and the compiler's wait counts
  // stay exact.
  float acc[V];
  uint32_t i = 0;
  for (; i + U <= n; i += U) {
    static_for<U>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int set = u % kDepth, g = u % T;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float a[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) a[m] = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) fmt.template decode<MC>(ps[set][r][j], xr[j], lut, laneoff, a);
#pragma unroll
        for (int m = 0; m < MC; ++m) acc[(g * R + r) * MC + m] = a[m];
      }
      load_tile(min(t + (uint32_t)(u + kDepth) * G, last), ps[set]);
      __builtin_amdgcn_sched_barrier(0);     // keep the reload ahead of the next tile's math
      if constexpr (g == T - 1) {
        // v[0] of lane l now holds value vi of the group (V = 8: (l >> 3) & 7,
        // V = 4: (l >> 4) & 3): tile g0 + vi / RM, row (vi / MC) % R,
        // activation row vi % MC.
        wave_reduce<V>(acc, lane);
        const uint32_t g0 = i + (uint32_t)(u - (T - 1));   // first tile of the group
        const int vi = (lane / (64 / V)) & (V - 1);
        const uint32_t tile_i = g0 + (uint32_t)(vi / RM);
        const int rv = vi % RM;
        if ((lane & (64 / V - 1)) == 0) {
          const uint32_t row = ((t0 + tile_i * G) * S + slot) * R + rv / MC;
          if (WK == 1) {
            if (row < N) y[(rv % MC) * ldy + row] = acc[0] * kOutScale;
          } else {
            red[tile_i % kRing][slot * WK + wk][rv] = acc[0];
          }
        }
        if (WK > 1 && (g0 + (uint32_t)T) % kRing == 0) flush(g0 + (uint32_t)T - kRing, kRing);
      }
    });
    t += (uint32_t)U * G;
  }
  // The remaining tiles (fewer than U <= kDepth + 1, so all of them are in
  // registers already: set s holds tile i + s), each reduced on its own.
  static_assert(U <= kDepth + 1, "the tail must be in registers");
  static_for<U - 1>([&](auto sc) {
    constexpr int s2 = decltype(sc)::value;
    if (i + s2 < n) {
      float v[RM];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float a[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) a[m] = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) fmt.template decode<MC>(ps[s2][r][j], xr[j], lut, laneoff, a);
#pragma unroll
        for (int m = 0; m < MC; ++m) v[r * MC + m] = a[m];
      }
      wave_reduce<RM>(v, lane);
      const uint32_t ti = i + s2;
      const int vi = lane / (64 / RM);
      if ((lane & (64 / RM - 1)) == 0) {
        const uint32_t row = ((t + (uint32_t)s2 * G) * S + slot) * R + vi / MC;
        if (WK == 1) {
          if (row < N) y[(vi % MC) * ldy + row] = v[0] * kOutScale;
        } else {
          red[ti % kRing][slot * WK + wk][vi] = v[0];
        }
      }
      if (WK > 1 && (ti + 1) % kRing == 0) flush(ti + 1 - kRing, kRing);
    }
  });
  if (WK > 1 && n % kRing != 0) flush(n - n % kRing, n % kRing);
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

// Persistent grid of one instantiation: the workgroups all compute units hold
// at once, as the runtime's occupancy calculator gives them for its register
// and LDS use (a grid larger than that runs a second round of workgroups,
// each paying the prologue again).  Cached per kernel, size and device.
uint32_t resident_grid(const void* kernel, int threads) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int>, uint32_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kernel, threads, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int blocks = 0;
  uint32_t g = grid_cap(threads);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, threads, 0) == hipSuccess && blocks > 0)
    g = (uint32_t)(blocks * device_cu_count());
  cache.emplace(key, g);
  return g;
}

template <typename Fmt, int J, int R, int MC, int kMaxT, int kDepth, int kEarly, int kStage = 0>
void launch_cfg(const Fmt& fmt, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x, int64_t ldx, int mode,
                float* y, int64_t ldy, const Plan& pl, hipStream_t s) {
  const int S = pl.threads / pl.TK;
  const uint32_t rows_per_tile = (uint32_t)(S * R);
  const uint32_t tiles = (N + rows_per_tile - 1) / rows_per_tile;
  // As many workgroups as fit the chip, trimmed so that every workgroup gets
  // the same number of tiles or one fewer (a round of 1.5 tiles per CU would
  // leave half the chip idle for the second half of the launch).
  const void* kern = nullptr;
  switch (mode) {
    case 0: kern = (const void*)&gemv_kernel<Fmt, J, R, MC, 0, kMaxT, kDepth, kEarly, kStage>; break;
    case 1: kern = (const void*)&gemv_kernel<Fmt, J, R, MC, 1, kMaxT, kDepth, kEarly, kStage>; break;
    case 2: if constexpr (Fmt::kLut) kern = (const void*)&gemv_kernel<Fmt, J, R, MC, 2, kMaxT, kDepth, kEarly, kStage>; break;
    default: if constexpr (Fmt::kLut) kern = (const void*)&gemv_kernel<Fmt, J, R, MC, 3, kMaxT, kDepth, kEarly, kStage>; break;
  }
  if (!kern) return;                         // rotation modes exist for TQ4_1S only (the entry points check)
  const uint32_t cap = resident_grid(kern, pl.threads);
  const uint32_t per_wg = (tiles + cap - 1) / cap;
  const uint32_t grid = (tiles + per_wg - 1) / per_wg;
  GemvGrid gg;
  gg.TK = pl.TK;
  gg.S = S;
  gg.slot_mul = (256u * 64u + (uint32_t)pl.TK - 1u) / (uint32_t)pl.TK;   // ceil(256 / WK)
  gg.G = grid;
  gg.q = tiles / grid;
  gg.r = tiles % grid;
#define TQ_GEMV_LAUNCH(M_)                                                                                     \
  hipLaunchKernelGGL((gemv_kernel<Fmt, J, R, MC, M_, kMaxT, kDepth, kEarly, kStage>), dim3(grid), dim3(pl.threads), 0, s, \
                     fmt, N, nb, mask, x, ldx, y, ldy, gg)
  switch (mode) {
    case 0: TQ_GEMV_LAUNCH(0); break;
    case 1: TQ_GEMV_LAUNCH(1); break;
    case 2: if constexpr (Fmt::kLut) TQ_GEMV_LAUNCH(2); break;   // rotation: TQ4_1S only
    default: if constexpr (Fmt::kLut) TQ_GEMV_LAUNCH(3); break;
  }
#undef TQ_GEMV_LAUNCH
}

// Decode GEMV shape, measured on MI355X over the Llama-3-8B and 70B decode
// layers: x' staged in LDS (when a workgroup holds more than two row slots),
// the fewest K-blocks per lane that fit a row into a 1024-thread workgroup,
// and one row per wavefront per tile with two register sets of tile loads,
// only the first requested before the activation has arrived.  Graph-timed
// 32-layer Llama-3-8B step on two boxes: 1.215 / 1.206 ms with both sets
// requested at the start, 1.164 / 1.147 ms with one; four sets (one early)
// measured 1.317 / 1.140 ms -- deeper queues help on some boxes and cost 8%
// on others, so two are kept.  Matrices that one round of two-row tiles
// covers (Llama-3-8B o: one tile per workgroup) used to take two rows per
// wavefront and one register set; two one-row tiles, the first computed
// while the second arrives, run o in 5.17-5.23 instead of 5.58-5.62 us.
constexpr bool kGemvStage = true;
constexpr int kGemvMinJ = 1;

template <typename Fmt, int J, int R>
void launch_gemv_jr(const Fmt& fmt, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x, int mode, float* y,
                    const Plan& pl, hipStream_t s) {
  // Groups of 4 elements each thread stages (a power of two, at most 8).
  const uint32_t K = nb * 32, per = 4u * (uint32_t)pl.threads;
  const uint32_t passes = (K + per - 1) / per;
  constexpr int D = R == 1 ? 2 : 1;
  if constexpr (J <= 2) {
    // Staging shares one rotation of each block among the workgroup's row
    // slots; with one or two slots (K above 8192) every lane rotates its own
    // blocks instead, which saves the staging barrier and the LDS round trip
    // (Llama-3-8B down 11.2-11.5 -> 11.0 us, 5120 x 17408 16.3-16.6 -> 13.8-14.5 us).
    // The block-float formats rotate nothing and need no pair table, so
    // per-lane loads leave their workgroups with no barrier before the
    // first tile at all: 27B-shaped NVFP4 layer, o 6.4-6.6 -> 5.6 us,
    // 16-layer stream 0.800 -> 0.764-0.773 ms.
    const bool shared = pl.threads / pl.TK > 2;
    if (kGemvStage && Fmt::kLut && shared && K <= (uint32_t)kStageFloats && passes <= 8) {
      if (passes <= 1) launch_cfg<Fmt, J, R, 1, 1024, D, 1, 1>(fmt, N, nb, mask, x, 0, mode, y, 0, pl, s);
      else if (passes <= 2) launch_cfg<Fmt, J, R, 1, 1024, D, 1, 2>(fmt, N, nb, mask, x, 0, mode, y, 0, pl, s);
      else if (passes <= 4) launch_cfg<Fmt, J, R, 1, 1024, D, 1, 4>(fmt, N, nb, mask, x, 0, mode, y, 0, pl, s);
      else launch_cfg<Fmt, J, R, 1, 1024, D, 1, 8>(fmt, N, nb, mask, x, 0, mode, y, 0, pl, s);
      return;
    }
  }
  // Larger K: every lane loads (and rotates) its own blocks; the loads of the
  // next tiles only fit in registers (without spills) at one block per lane.
  constexpr int DJ = J == 1 ? D : 1;
  launch_cfg<Fmt, J, R, 1, 1024, DJ, 1>(fmt, N, nb, mask, x, 0, mode, y, 0, pl, s);
}

template <typename Fmt, int J>
void launch_gemv_j(const Fmt& fmt, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x, int mode, float* y,
                   hipStream_t s) {
  const Plan pl = plan_for(nb, 1024, J);
  launch_gemv_jr<Fmt, J, 1>(fmt, N, nb, mask, x, mode, y, pl, s);
}

template <typename Fmt>
void launch_gemv_fmt(const Fmt& fmt, uint32_t N, uint32_t nb, uint32_t mask, const uint8_t* x, int mode, float* y,
                     hipStream_t s) {
  const int J = min_j(nb, 1024) > kGemvMinJ ? min_j(nb, 1024) : kGemvMinJ;
  switch (J) {
    case 1: launch_gemv_j<Fmt, 1>(fmt, N, nb, mask, x, mode, y, s); break;
    case 2: launch_gemv_j<Fmt, 2>(fmt, N, nb, mask, x, mode, y, s); break;
    case 3: launch_gemv_j<Fmt, 3>(fmt, N, nb, mask, x, mode, y, s); break;
    default: launch_gemv_j<Fmt, 4>(fmt, N, nb, mask, x, mode, y, s); break;
  }
}

// VALU small-batch path for M < 16: chunks of MC = 4, 2 or 1 activation rows
// held in registers (float32, 32 VGPRs per row per owned block), one launch
// per chunk, each keeping the next tile's weights in flight.  Four rows fit
// 256-thread workgroups up to K = 8192, two rows 512- or 1024-thread
// workgroups up to K = 32768 (one row per wavefront per tile at 1024
// threads, where the register budget is 128).
template <typename Fmt>
void launch_gemm_valu_fmt(const Fmt& fmt, uint32_t N, uint32_t nb, int64_t M, const uint8_t* xb, int mode,
                          int64_t ldx_bytes, float* y, int64_t ldy, hipStream_t s) {
  for (int64_t m0 = 0; m0 < M;) {
    const int64_t left = M - m0;
    const uint8_t* xm = xb + m0 * ldx_bytes;
    float* ym = y + m0 * ldy;
    if (left >= 4 && nb <= 256) {
      const Plan pl = plan_for(nb, 256, 1);
      launch_cfg<Fmt, 1, 2, 4, 256, 2, 2>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s);
      m0 += 4;
    } else if (left >= 2 && nb <= 512) {
      const Plan pl = plan_for(nb, 512, 1);
      launch_cfg<Fmt, 1, 2, 2, 512, 2, 2>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s);
      m0 += 2;
    } else if (left >= 2 && nb <= 1024) {
      const Plan pl = plan_for(nb, 1024, 1);
      launch_cfg<Fmt, 1, 1, 2, 1024, 2, 2>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s);
      m0 += 2;
    } else {
      const Plan pl = plan_for(nb, 1024, min_j(nb, 1024));
      switch (pl.J) {
        case 1: launch_cfg<Fmt, 1, 2, 1, 1024, 2, 2>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s); break;
        case 2: launch_cfg<Fmt, 2, 2, 1, 1024, 1, 1>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s); break;
        case 3: launch_cfg<Fmt, 3, 2, 1, 1024, 1, 1>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s); break;
        default: launch_cfg<Fmt, 4, 2, 1, 1024, 1, 1>(fmt, N, nb, 0u, xm, ldx_bytes, mode, ym, ldy, pl, s); break;
      }
      m0 += 1;
    }
  }
}

FmtTQ4 tq4_format(const uint8_t* packed, const uint16_t* scales) {
  return FmtTQ4{reinterpret_cast<const uint4*>(packed), reinterpret_cast<const uint32_t*>(scales)};
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                       const void* x, bool xbf16, bool rotated, float* y, hipStream_t s) {
  const int mode = rotated ? (xbf16 ? 1 : 0) : (xbf16 ? 3 : 2);
  launch_gemv_fmt(tq4_format(packed, scales), (uint32_t)N, (uint32_t)(K / kBlock), mask,
                  static_cast<const uint8_t*>(x), mode, y, s);
  return hipGetLastError();
}

hipError_t launch_gemm_valu(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                            const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, hipStream_t s) {
  launch_gemm_valu_fmt(tq4_format(packed, scales), (uint32_t)N, (uint32_t)(K / kBlock), M,
                       static_cast<const uint8_t*>(xr), xbf16 ? 1 : 0, ldx * (xbf16 ? 2 : 4), y, ldy, s);
  return hipGetLastError();
}

// Block-float decode GEMV/GEMM (M < 16 per launch chunk, VALU) on the same
// kernels: the activation is used as given (no rotation).
hipError_t launch_blockfp_gemv(int fmt, const uint8_t* codes, const uint8_t* bscales, const float* tscale, int64_t N,
                               int64_t K, int64_t M, const void* x, bool xbf16, int64_t ldx, float* y, int64_t ldy,
                               hipStream_t s) {
  const uint32_t nb = (uint32_t)(K / 32);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const int mode = xbf16 ? 1 : 0;
  const int64_t ldx_bytes = ldx * (xbf16 ? 2 : 4);
  if (fmt == TQ_FMT_NVFP4) {
    const FmtNVFP4 f{reinterpret_cast<const uint4*>(codes), reinterpret_cast<const uint16_t*>(bscales), tscale, 0.f};
    if (M == 1) launch_gemv_fmt(f, (uint32_t)N, nb, 0u, xb, mode, y, s);
    else launch_gemm_valu_fmt(f, (uint32_t)N, nb, M, xb, mode, ldx_bytes, y, ldy, s);
  } else {
    const FmtMXFP6 f{reinterpret_cast<const uint2*>(codes), bscales};
    if (M == 1) launch_gemv_fmt(f, (uint32_t)N, nb, 0u, xb, mode, y, s);
    else launch_gemm_valu_fmt(f, (uint32_t)N, nb, M, xb, mode, ldx_bytes, y, ldy, s);
  }
  return hipGetLastError();
}

}  // namespace tq
