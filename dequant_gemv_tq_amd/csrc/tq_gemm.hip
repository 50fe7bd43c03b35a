// Small-batch fused TQ4_1S GEMM on gfx950: Y[m, n] = sum_k X'[m, k] Q[n, k]
// with Q = d * c[idx] in the rotated domain and X' the pre-rotated
// activations (the same identity as the GEMV: rotating the activation once
// turns dequantization into a centroid lookup times a scale; TQ4 page
// "企业官网建设流程全解析", hotelren.com/news/5458160, decode-speed section).
//
// For M >= 16 the contraction is dense enough for the matrix cores:
// v_mfma_f32_16x16x32_bf16 computes a 16(m) x 16(n) tile over 32 k.
//   * Operand layout.  Lane l has column n = l % 16 and k-slot group
//     g = l / 16.  MFMA step s (0-3) of a group of four blocks b0..b0+3
//     covers block b0 + s, and group g takes its elements 8 g .. 8 g + 7, so
//     an activation operand load of 16 rows reads 16 whole 64-byte block rows
//     (coalesced).  The weights arrive the other way round -- one 16-byte
//     load gives lane (n, g) all four dwords of block b0 + g of row n -- and
//     a 4 x 4 transpose of dwords across the lane groups (two
//     v_permlane32_swap and two v_permlane16_swap) hands dword g of block
//     b0 + s to group g for step s.  Output: lane l, register r holds
//     D[4 g + r][l % 16].
//   * Dequantization once per weight: a byte of two nibbles is looked up in
//     the replicated pair table (one v_perm + one ds_read_b64 per two
//     weights), multiplied by its fp16 scale in float32 and rounded to bf16
//     by v_cvt_pk_bf16_f32 -- about two VALU ops per weight for any M.
//   * Operand reuse.  A wavefront covers RT tiles of 16 weight rows and MT
//     tiles of 16 activation rows: each activation operand is loaded once
//     per step and used for RT row tiles, each weight operand for MT
//     activation tiles.
//   * Split K inside the workgroup: wavefront w of 4 takes groups w, w + 4,
//     ... along K; the next group's weights and activations are requested
//     while the current one is computed (each register set is reloaded right
//     after its last use), and the four partial tiles are summed through LDS
//     (the pair table's space) at the end.
// Arithmetic intensity stays below the bf16 ridge for M <= 64 (about 3.2 M
// flop per byte of packed weight), so HBM remains the bound.
//
// Precision: with bf16 activations both operands carry up to 2^-8 relative
// rounding (the persistent kernel's weights 2^-8 + 2^-11: fp16 centroids), so
// each rotated-domain product q_k x'_k is off by at most 2^-7 + 2^-10 of its
// size; for dense activations the errors average out to about
// 2^-9 * ||w o x||_2, inside 1e-3 * sum|w x| once K is in the hundreds.  With
// float32 activations each operand is split into bf16 hi + lo (hi by
// truncation, lo = bf16(v - hi)) and three MFMAs (hi*hi + hi*lo + lo*hi) leave
// at most 2^-13 per product.  Both are bounds on sum_k |q_k x'_k|: a one-hot x,
// whose 32 rotated products cancel to one weight, can exceed 1e-3 * sum|w x|.
#include <algorithm>
#include <type_traits>

#include "tq_internal.hpp"

namespace tq {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2v v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(bf16x8, u);
}

// Split 8 float32 values into bf16 hi (truncation) and lo (RNE of the exact residual).
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t a = __float_as_uint(v[2 * t]) & 0xffff0000u, b = __float_as_uint(v[2 * t + 1]) & 0xffff0000u;
    h[t] = (a >> 16) | b;
    l[t] = pack_bf16x2(v[2 * t] - __uint_as_float(a), v[2 * t + 1] - __uint_as_float(b));
  }
  hi = as_bf16x8(h[0], h[1], h[2], h[3]);
  lo = as_bf16x8(l[0], l[1], l[2], l[3]);
}

// The 8 weights of dword w (elements 8 s .. 8 s + 7 of a block) times scale d, as float32.
__device__ __forceinline__ void dequant8(uint32_t w, float d, const uint8_t* lut, uint32_t laneoff, float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float2 c = *reinterpret_cast<const float2*>(lut + pair_addr(w, laneoff, k));
    v[2 * k] = c.x * d;
    v[2 * k + 1] = c.y * d;
  }
}

// The persistent kernel's pair table holds fp16 pairs: entry e (the byte of
// two nibbles, low nibble = even element) is the dword f16(c[e % 16]) |
// f16(c[e / 16]) << 16, in 64 copies (entry e, copy l at byte 256 e + 4 l),
// so one ds_read_b32 per lane serves all 64 lanes without bank conflicts and
// reads half the bytes of the float32 table.  The centroids in fp16 carry
// 11 significant bits; their product with an fp16 scale is exact in float32
// and is rounded once, to the bf16 operand.
constexpr int kLut16Bytes = 256 * 64 * 4;

__device__ __forceinline__ void fill_pair_lut16(uint8_t* lut, int tid, int nthreads) {
  const int lane = tid & 63, g = lane >> 4;
  for (int w = tid >> 6; w < 16; w += nthreads >> 6) {
    const int wu = __builtin_amdgcn_readfirstlane(w);
    float hi = centroid(0);
#pragma unroll
    for (int k = 1; k < 16; ++k) hi = wu == k ? centroid(k) : hi;
    const uint32_t hb = (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)hi) << 16;
    uint8_t* base = lut + ((16 * wu + g) << 8) + 16 * (lane & 15);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float lo = g == 0   ? centroid(4 * u)
                       : g == 1 ? centroid(4 * u + 1)
                       : g == 2 ? centroid(4 * u + 2)
                                : centroid(4 * u + 3);
      const uint32_t v = hb | __builtin_bit_cast(unsigned short, (_Float16)lo);
      *reinterpret_cast<uint4*>(base + (u << 10)) = make_uint4(v, v, v, v);
    }
  }
}

// f(std::integral_constant<int, j>) for j = 0 .. N-1.
template <int N, typename F, int J = 0>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>{});
    static_for<N, F, J + 1>(static_cast<F&&>(f));
  }
}

// 4 x 4 transpose of dwords across the four 16-lane groups: on entry lane
// (n, g) holds dwords 0-3 of block b0 + g; on exit out[s] is dword g of block
// b0 + s.  permlane32_swap(a, b) leaves (a rows 0-1, b rows 0-1) in its
// first result and (a rows 2-3, b rows 2-3) in its second; permlane16_swap
// does the same for row pairs (0, 1) and (2, 3).
__device__ __forceinline__ void transpose_groups(const uint4& p, uint32_t (&out)[4]) {
  auto s32 = __builtin_amdgcn_permlane32_swap(p.x, p.z, false, false);   // j = 0: words 0 and 2
  auto t32 = __builtin_amdgcn_permlane32_swap(p.y, p.w, false, false);   // j = 1: words 1 and 3
  auto a = __builtin_amdgcn_permlane16_swap(s32[0], t32[0], false, false);
  auto b = __builtin_amdgcn_permlane16_swap(s32[1], t32[1], false, false);
  out[0] = a[0];
  out[1] = a[1];
  out[2] = b[0];
  out[3] = b[1];
}

template <bool kF32X>
struct AOperand;

// Activation operand loads are issued unconditionally from a clamped,
// in-bounds address (row min(m, M - 1), element k of a block that exists)
// and the operand is zeroed afterwards when (m, block) lies outside X: a
// load under a lane condition becomes an exec-masked branch, after which the
// compiler can no longer count outstanding loads and waits for all of them.
template <>
struct AOperand<false> {                  // bf16 activations: one operand per (step, m tile)
  uint4 a;
  bool live;
  __device__ __forceinline__ void load(const uint8_t* X, int64_t ldx, uint32_t m, uint32_t M, uint32_t k, bool ok) {
    a = *reinterpret_cast<const uint4*>(X + ((size_t)min(m, M - 1u) * ldx + k) * 2);
    live = ok && m < M;
  }
  __device__ __forceinline__ uint4 value() const { return live ? a : make_uint4(0u, 0u, 0u, 0u); }
};

template <>
struct AOperand<true> {                   // float32 activations, split to bf16 hi/lo at use
  float raw[8];
  bool live;
  __device__ __forceinline__ void load(const uint8_t* X, int64_t ldx, uint32_t m, uint32_t M, uint32_t k, bool ok) {
    const float4* src = reinterpret_cast<const float4*>(X + ((size_t)min(m, M - 1u) * ldx + k) * 4);
    const float4 u0 = src[0], u1 = src[1];
    raw[0] = u0.x; raw[1] = u0.y; raw[2] = u0.z; raw[3] = u0.w;
    raw[4] = u1.x; raw[5] = u1.y; raw[6] = u1.z; raw[7] = u1.w;
    live = ok && m < M;
  }
  __device__ __forceinline__ void value(float (&v)[8]) const {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = live ? raw[t] : 0.f;
  }
};

// MT activation tiles (M <= 16 MT), RT weight-row tiles per workgroup, WD
// groups of weights in flight per wavefront.
template <int MT, int RT, int WD, bool kF32X>
__global__ __launch_bounds__(kThreads, 2) void gemm_mfma_kernel(const uint4* __restrict__ packed,
                                                                const uint32_t* __restrict__ scales, uint32_t N,
                                                                uint32_t nb, const uint8_t* __restrict__ X,
                                                                int64_t ldx, uint32_t M, float* __restrict__ Y,
                                                                int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLutBytes];
  static_assert((kWaves - 1) * RT * MT * 64 * 16 <= kLutBytes, "partial tiles must fit the table's space");
  uint8_t* const lut = smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 15;
  const uint32_t g = (uint32_t)(lane >> 4);
  const uint32_t laneoff = (uint32_t)(lane & (kCopies - 1)) * 8u;

  const uint32_t n0 = blockIdx.x * (16u * RT);
  const uint32_t ngroups = (nb + 3u) / 4u;

  // Row addresses (clamped: rows past N read a valid row and are not written).
  const uint4* prow[RT];
  const uint32_t* srow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint32_t row = min(n0 + 16u * rt + (uint32_t)nl, N - 1u);
    prow[rt] = packed + (size_t)row * nb;
    srow[rt] = scales + (size_t)row * nb;
  }

  // The groups of this wavefront are q_i = wave + 4 i, i < nq.  Indices
  // past the last group are clamped to it: those loads re-read a group
  // already loaded and are discarded.
  const uint32_t nq = (uint32_t)wave < ngroups ? (ngroups - 1u - (uint32_t)wave) / 4u + 1u : 0u;
  auto grp = [&](uint32_t i) { return (uint32_t)wave + 4u * min(i, nq - 1u); };

  // Weights of group q for this lane: block 4 q + g of its row and that
  // block's scale pair (clamped: a block past nb belongs to a step that is
  // skipped).
  struct WSet {
    uint4 p[RT];
    uint32_t sc[RT];
  };
  WSet ws[WD];
  auto load_w = [&](WSet& w, uint32_t q) {
    const uint32_t b = min(4u * q + g, nb - 1u);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      w.p[rt] = prow[rt][b];
      w.sc[rt] = srow[rt][b];
    }
  };
  // Activation operands: AD register sets.  Loads complete in issue order
  // (one vmcnt counter), so a wait for an operand also waits for every
  // weight load issued before it; with AD == WD each set is refilled right
  // behind the weight set of the same group and every wait covers exactly
  // the group about to be computed.  (AD == 1 refills during the group
  // before, which leaves the weight prefetch only one group of lead.)
  constexpr int AD = MT <= 2 ? WD : 1;
  AOperand<kF32X> A[AD][4][MT];
  auto load_a = [&](int set, uint32_t q, int s) {
    const uint32_t b = 4u * q + (uint32_t)s;
    const bool ok = b < nb;
    const uint32_t bc = min(b, nb - 1u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) A[set][s][mt].load(X, ldx, mt * 16u + (uint32_t)nl, M, 32u * bc + 8u * g, ok);
  };

  if (nq > 0u) {
#pragma unroll
    for (int j = 0; j < WD; ++j) {
      load_w(ws[j], grp((uint32_t)j));
      if (j < AD) {
#pragma unroll
        for (int s = 0; s < 4; ++s) load_a(j, grp((uint32_t)j), s);
      }
    }
  }
  fill_pair_lut(lut, tid, kThreads);
  __syncthreads();

  f32x4 acc[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Group i with weight set w (set number j): compute, then (reload) refill
  // w with group i + WD; the activation operands of step s are refilled with
  // group i + AD as soon as step s has used them.
  auto body = [&](uint32_t i, WSet& w, auto jc, auto reload) {
    constexpr int ja = decltype(jc)::value % AD;
    const uint32_t q = grp(i), qn = grp(i + (uint32_t)AD);
    // Dword g of block b0 + s for step s, and the scale of its half.
    uint32_t wt[RT][4];
    float dd[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      transpose_groups(w.p[rt], wt[rt]);
      uint32_t sct[4];
      transpose_groups(make_uint4(w.sc[rt], w.sc[rt], w.sc[rt], w.sc[rt]), sct);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) dd[rt][s2] = f16_bits_to_f32(g < 2u ? (sct[s2] & 0xffffu) : (sct[s2] >> 16));
    }
    if constexpr (decltype(reload)::value) load_w(w, grp(i + (uint32_t)WD));
    const uint32_t nsteps = min(4u, nb - 4u * q);          // steps whose block exists (wavefront-uniform)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if ((uint32_t)s < nsteps) {   // a step past the last block contributes nothing
        bf16x8 Bh[RT], Bl[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float v[8];
          dequant8(wt[rt][s], dd[rt][s], lut, laneoff, v);
          if constexpr (!kF32X) {
            Bh[rt] = as_bf16x8(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7]));
          } else {
            split8(v, Bh[rt], Bl[rt]);
          }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (!kF32X) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, A[ja][s][mt].value());
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Bh[rt], acc[rt][mt], 0, 0, 0);
          } else {
            bf16x8 ah, al;
            float av[8];
            A[ja][s][mt].value(av);
            split8(av, ah, al);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, Bh[rt], acc[rt][mt], 0, 0, 0);
              acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, Bl[rt], acc[rt][mt], 0, 0, 0);
              acc[rt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, Bh[rt], acc[rt][mt], 0, 0, 0);
            }
          }
        }
      }
      load_a(ja, qn, s);   // step s's operands are consumed: request their next group's
    }
  };

  // A fixed trip count with the remainder after it (no conditional reloads
  // inside the loop), so the compiler's wait counts stay exact.
  uint32_t i = 0;
  for (; i + WD <= nq; i += WD) {
    static_for<WD>([&](auto jc) { body(i + (uint32_t)jc.value, ws[jc.value], jc, std::true_type{}); });
  }
  static_for<WD - 1>([&](auto jc) {
    if (i + (uint32_t)jc.value < nq) body(i + (uint32_t)jc.value, ws[jc.value], jc, std::false_type{});
  });

  // Sum the four wavefronts' partial tiles through the table's LDS space.
  __syncthreads();
  f32x4* part = reinterpret_cast<f32x4*>(smem);
  if (wave > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) part[(((wave - 1) * RT + rt) * MT + mt) * 64 + lane] = acc[rt][mt];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t row = n0 + 16u * rt + (uint32_t)nl;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 v = acc[rt][mt];
#pragma unroll
        for (int w2 = 0; w2 < kWaves - 1; ++w2) v += part[((w2 * RT + rt) * MT + mt) * 64 + lane];
        if (row < N) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t m = mt * 16u + 4u * g + r;
            if (m < M) Y[(size_t)m * ldy + row] = v[r];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Weight formats of the persistent kernel.  Lane (n, g) of a wavefront loads
// block 4 q + g of weight row n for group q (four 32-element blocks) and
// turns it into the bf16 B operands of the four MFMA steps of the group:
//   kByBlock = true:  step s covers block 4 q + s, lane group g its elements
//                     8 g .. 8 g + 7 (the raw dwords are transposed across
//                     the lane groups first);
//   kByBlock = false: step s covers elements 8 s .. 8 s + 7 of every lane
//                     group's own block (no transpose of the weights; the
//                     activation operands are transposed across the lane
//                     groups instead).
// kLut says whether the pair table is needed; kTensorScale whether the
// finished sums are multiplied by a float32 tensor scale.
// ---------------------------------------------------------------------------

// TQ4_1S: 16 bytes of nibbles and the fp16 scale pair per block; each weight
// is the fp16 centroid pair lookup times its fp16 scale, rounded to bf16.
struct GemmTQ4 {
  static constexpr bool kLut = true, kByBlock = true, kTensorScale = false;
  struct Raw {
    uint4 p;
    uint32_t sc;
  };
  struct Dec {
    uint32_t w[4], sc[4];
  };
  __device__ __forceinline__ static void load(Raw& r, const uint8_t* codes, const uint8_t* scales, size_t blk) {
    r.p = reinterpret_cast<const uint4*>(codes)[blk];
    r.sc = reinterpret_cast<const uint32_t*>(scales)[blk];
  }
  __device__ __forceinline__ static void prepare(const Raw& r, Dec& d) {
    transpose_groups(r.p, d.w);
    // Lane groups 0, 1 take elements 0..15 of every block (scale d0, the low
    // half), groups 2, 3 elements 16..31 (d1): the sender shifts d1 down for
    // them, so every receiver finds its scale in the low half.
    transpose_groups(make_uint4(r.sc, r.sc, r.sc >> 16, r.sc >> 16), d.sc);
  }
  __device__ __forceinline__ static bf16x8 operand(const Dec& d, int s, uint32_t, const uint8_t* lut,
                                                   uint32_t laneoff) {
    // c * d with d read as fp16 straight from its register (v_fma_mix_f32:
    // no separate conversion; + 0 keeps it a fused multiply-add, whose
    // single rounding equals that of the product).
    const float sc = (float)__builtin_bit_cast(_Float16, (unsigned short)(d.sc[s] & 0xffffu));
    float v[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = *reinterpret_cast<const uint32_t*>(lut + pair_addr(d.w[s], laneoff, k));
      v[2 * k] = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (unsigned short)(c & 0xffffu)), sc, 0.0f);
      v[2 * k + 1] = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (unsigned short)(c >> 16)), sc, 0.0f);
    }
    return as_bf16x8(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7]));
  }
};

// NVFP4: 16 bytes of E2M1 codes and two E4M3 scales per 32-element block.
// The scaled fp4 conversion applies only the exponent of its scale, so the
// codes are converted with scale 1 and multiplied by the E4M3 value in
// float32; e2m1 * e4m3 has at most 6 significant bits, so the bf16 operand
// is exact.  The tensor scale multiplies the finished sums.
struct GemmNVFP4 {
  static constexpr bool kLut = false, kByBlock = false, kTensorScale = true;
  struct Raw {
    uint4 p;
    uint32_t sc;
  };
  typedef Raw Dec;
  __device__ __forceinline__ static void load(Raw& r, const uint8_t* codes, const uint8_t* scales, size_t blk) {
    r.p = reinterpret_cast<const uint4*>(codes)[blk];
    r.sc = reinterpret_cast<const uint16_t*>(scales)[blk];
  }
  __device__ __forceinline__ static void prepare(const Raw& r, Dec& d) { d = r; }
  __device__ __forceinline__ static bf16x8 operand(const Dec& d, int s, uint32_t, const uint8_t*, uint32_t) {
    const uint32_t w = s == 0 ? d.p.x : s == 1 ? d.p.y : s == 2 ? d.p.z : d.p.w;
    const float sc = e4m3_decode((d.sc >> (8 * (s >> 1))) & 0xffu);
    const auto v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);   // byte k: elements 2k, 2k + 1
    const auto v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    return as_bf16x8(pack_bf16x2(v0[0] * sc, v0[1] * sc), pack_bf16x2(v1[0] * sc, v1[1] * sc),
                     pack_bf16x2(v2[0] * sc, v2[1] * sc), pack_bf16x2(v3[0] * sc, v3[1] * sc));
  }
};

// MXFP6: 24 bytes of E3M2 codes and one E8M0 scale per block.  One scaled
// conversion turns the block into 32 bf16 values times 2^(byte - 127): the
// scale is a power of two, which the conversion applies exactly.
struct GemmMXFP6 {
  static constexpr bool kLut = false, kByBlock = false, kTensorScale = false;
  struct Raw {
    uint4 a;
    uint2 b;
    uint32_t sc;
  };
  typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
  struct Dec {
    u32x16 v;
  };
  __device__ __forceinline__ static void load(Raw& r, const uint8_t* codes, const uint8_t* scales, size_t blk) {
    // 24 bytes at an 8-byte aligned offset: one 16-byte and one 8-byte load
    // (global loads need 4-byte alignment only).
    const uint8_t* c = codes + blk * 24;
    r.a = *reinterpret_cast<const uint4*>(c);
    r.b = *reinterpret_cast<const uint2*>(c + 16);
    r.sc = scales[blk];
  }
  __device__ __forceinline__ static void prepare(const Raw& r, Dec& d) {
    typedef unsigned u32x6 __attribute__((ext_vector_type(6)));
    const u32x6 bits = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y};
    // E8M0 byte b as the float32 2^(b - 127): the conversion reads the
    // exponent field.  The empty asm keeps the shift here, at the use: the
    // compiler otherwise computed it right after the next tile's load was
    // issued, which made the loop wait for that load.
    uint32_t sc = r.sc;
    asm volatile("" : "+v"(sc));
    d.v = __builtin_bit_cast(u32x16, __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(bits, __uint_as_float(sc << 23)));
  }
  __device__ __forceinline__ static bf16x8 operand(const Dec& d, int s, uint32_t, const uint8_t*, uint32_t) {
    return as_bf16x8(d.v[4 * s], d.v[4 * s + 1], d.v[4 * s + 2], d.v[4 * s + 3]);
  }
};

// ---------------------------------------------------------------------------
// Persistent small-batch kernel, bf16 activations, M <= 64: one 1024-thread
// workgroup per CU, shaped like the fused GEMV.  K is covered in passes of
// 16 * NQ groups of four blocks (NQ * 2048 elements): in a pass, wavefront w
// takes groups w, w + 16, ... of the pass and keeps their activation
// operands (MT tiles of 16 rows) in registers while the workgroup walks its
// 16-row weight tiles (tiles g, g + G, ...) with the next tile's weights in
// flight.  The sixteen partial 16 x 16 MT tiles of a weight tile wait in an
// LDS ring (64 KiB) that all 1024 threads reduce, in wavefront order, every
// few tiles.  With more than one pass the sums of the earlier passes wait in
// an LDS accumulator (32 KiB, one float per output of the workgroup; the
// host splits taller launches) and Y is written once, by the last pass: a
// global read of Y in the loop would also wait for the weight prefetch,
// since vector loads complete in issue order.
//
// Few row tiles and K in several passes: the passes are split over S sets
// of workgroups (one pass each), so every workgroup takes several tiles and
// reads the activations of one pass only.  Each set stores its sums to a
// workspace; once a workgroup has stored all of its tiles it counts them on
// per-tile counters, and the workgroup that brings a count to S adds the S
// stored sums in split order and writes Y (so Y does not depend on which
// set finishes last), then returns the counter to zero.  Each wavefront loads its own
// activation operands from X (no LDS staging, no workgroup barrier), then
// its first two weight tiles, and fills its part of the pair table while
// they are in flight.
// ---------------------------------------------------------------------------
constexpr int kWide = 16;
constexpr int kRingBytes = 65536;
constexpr int kAccFloats = 8192;      // outputs of one workgroup that the pass accumulator holds

template <class Fmt, int MT, int NQ>
__global__ __launch_bounds__(64 * kWide) void gemm_small_kernel(const uint8_t* __restrict__ codes,
                                                                const uint8_t* __restrict__ scales,
                                                                const float* __restrict__ tscale, uint32_t N,
                                                                uint32_t nb, const uint8_t* __restrict__ X,
                                                                int64_t ldx, uint32_t M, float* __restrict__ Y,
                                                                int64_t ldy, uint32_t G, uint32_t tq, uint32_t tr,
                                                                uint32_t S, float* __restrict__ part,
                                                                uint32_t* __restrict__ counters) {
  constexpr int kRing = kRingBytes / (kWide * 64 * 16 * MT);        // weight tiles per ring
  static_assert(kRing * 256 * MT == 64 * kWide, "one output per thread per flush");
  // LDS: pair table (TQ4_1S only) | partial-tile ring | pass accumulator.
  constexpr int kLutSpace = Fmt::kLut ? kLut16Bytes : 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLutSpace + kRingBytes + kAccFloats * 4];
  uint8_t* const lut = smem;
  f32x4 (*const ring)[kWide][MT][64] = reinterpret_cast<f32x4 (*)[kWide][MT][64]>(smem + kLutSpace);
  float* const accum = reinterpret_cast<float*>(smem + kLutSpace + kRingBytes);
  const float ts = Fmt::kTensorScale ? *tscale : 1.0f;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t g = (uint32_t)(lane >> 4);
  const uint32_t laneoff = (uint32_t)lane * 4u;          // this lane's copy in the fp16 pair table
  const uint32_t ngroups = (nb + 3u) / 4u;
  constexpr uint32_t kPassGroups = (uint32_t)(kWide * NQ);
  const uint32_t passes = (ngroups + kPassGroups - 1u) / kPassGroups;

  // Workgroups sG .. sG + G - 1 take the same tiles over split s of the
  // passes (S == 1: all of them).
  const uint32_t split = blockIdx.x / G;
  const uint32_t t0 = blockIdx.x - split * G;
  const uint32_t per_split = (passes + S - 1u) / S;
  const uint32_t pass_begin = split * per_split;
  const uint32_t pass_end = min(pass_begin + per_split, passes);
  const uint32_t T = (N + 15u) / 16u;                    // row tiles
  const uint32_t n = tq + (t0 < tr ? 1u : 0u);          // this workgroup's tiles
  const uint32_t last = t0 + (n - 1u) * G;

  uint4 A[NQ][4][MT];                      // this wavefront's activation operands of the pass
  struct WSet {
    typename Fmt::Raw r[NQ];
  };
  // Group j of this wavefront in pass `pass` (clamped: a group past the last
  // one is skipped at compute time).
  auto group_of = [&](uint32_t pass, int j) { return pass * kPassGroups + (uint32_t)wave + (uint32_t)(kWide * j); };
  // A group's weights are loaded in row-major lane order: lane 4 r + b reads
  // block 4 q + b of tile row r, so each row's four blocks are contiguous
  // over four neighbouring lanes.  (With lane = r + 16 b, the order the MFMA
  // operands use, neighbouring lanes read different rows and the loads of
  // the whole tile loop ran at about two thirds of the rate.)  One
  // ds_bpermute per loaded dword then hands block 4 q + g of row n to lane
  // n + 16 g: a fixed rotation of the 6-bit lane index by two places.
  const uint32_t lrow = (uint32_t)lane >> 2, lblk = (uint32_t)lane & 3u;
  const int perm_addr = 4 * (((lane & 15) << 2) | (lane >> 4));
  auto to_mfma_lanes = [&](const typename Fmt::Raw& r) {
    static_assert(sizeof(typename Fmt::Raw) % 4 == 0, "whole dwords");
    constexpr int kWords = (int)(sizeof(typename Fmt::Raw) / 4);
    uint32_t wd[kWords];
    __builtin_memcpy(wd, &r, sizeof(wd));
#pragma unroll
    for (int i = 0; i < kWords; ++i) wd[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)wd[i]);
    typename Fmt::Raw out;
    __builtin_memcpy(&out, wd, sizeof(wd));
    return out;
  };
  // The scheduling barriers keep each register set's loads together (the
  // compiler interleaved the two sets otherwise), so every path into the
  // loop carries the same load order and the wait for a set never covers
  // the set loaded after it.
  auto load_w = [&](WSet& w, uint32_t tile, uint32_t pass) {
    const uint32_t row = min(tile * 16u + lrow, N - 1u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const uint32_t b = min(4u * group_of(pass, j) + lblk, nb - 1u);
      Fmt::load(w.r[j], codes, scales, (size_t)row * nb + b);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Activation operands of a pass.  For group j and m tile mt, lane (n, g)
  // needs, for step s, eight elements of activation row 16 mt + n: by block
  // the elements 32 s + 8 g of the group, by element 32 g + 8 s.  Rows past
  // M are clamped to row M - 1 and elements past K to the last block: both
  // only feed outputs that are not written (an MFMA output row depends on
  // its own activation row alone) or steps that are skipped.  Each
  // wavefront loads only its own operands (an earlier version staged a
  // pass's activations for the whole workgroup through LDS in 64 KiB parts,
  // with two barriers per part).
  //
  // Two m tiles (kStageA): each 4 KiB piece (one m tile: 16 rows x 128
  // elements) is loaded with 256 contiguous bytes of a row per 16 lanes
  // (four rows per load) and passed through this wavefront's 4 KiB of the
  // partial-tile ring, which is idle until the pass's first tile; row n keeps
  // its 16-byte chunk c at position c ^ n, so both the stores (one row, 16
  // chunks) and the loads (16 rows, one chunk each) of 16 lanes fall on
  // distinct banks; one workgroup barrier per pass then frees the ring for
  // the tiles.  8B layer at M = 32: 76.3-76.9 -> 72.1 us.  With one or
  // four m tiles, or MXFP6's larger register sets, the round trip costs
  // registers the kernel does not have (it spilled and ran slower), and the
  // operands are loaded in row-major
  // lane order, lane 4 n + g reading elements 32 s + 8 g of row n (64
  // contiguous bytes per row over four lanes), and handed to lane n + 16 g
  // by the same ds_bpermute as the weights; the by-element order then swaps
  // s and g across the lane groups.
  constexpr bool kStageA = MT == 2 && !std::is_same<Fmt, GemmMXFP6>::value;   // MXFP6: spills
  constexpr uint32_t kPassK = 16u * NQ * 128u;               // elements of K per pass
  const uint32_t K = nb * 32u;
  auto load_a = [&](uint32_t pass) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kStageA) {
      const uint32_t rq = (uint32_t)lane >> 4, e8 = 8u * ((uint32_t)lane & 15u);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const uint32_t k = min(pass * kPassK + 128u * ((uint32_t)wave + (uint32_t)(kWide * j)) + e8, K - 8u);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t r = min((uint32_t)(16 * mt + 4 * i) + rq, M - 1u);
            A[j][i][mt] = *reinterpret_cast<const uint4*>(X + ((size_t)r * ldx + k) * 2);
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const uint32_t kg = pass * kPassK + 128u * ((uint32_t)wave + (uint32_t)(kWide * j));   // wavefront-uniform
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t k = min(kg + 32u * (uint32_t)s + 8u * lblk, K - 8u);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const uint32_t r = min((uint32_t)(16 * mt) + lrow, M - 1u);
            A[j][s][mt] = *reinterpret_cast<const uint4*>(X + ((size_t)r * ldx + k) * 2);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto place_a = [&]() {
    if constexpr (kStageA) {
      uint8_t* const st = smem + kLutSpace + (size_t)wave * 4096u;
      const uint32_t wn = (uint32_t)lane >> 4, wc = (uint32_t)lane & 15u;   // store: row 4 i + wn, chunk wc
      const uint32_t nl = (uint32_t)lane & 15u, gl = (uint32_t)lane >> 4;   // load: row nl, lane group gl
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t n = 4u * (uint32_t)i + wn;
            *reinterpret_cast<uint4*>(st + 256u * n + 16u * (wc ^ n)) = A[j][i][mt];
          }
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): the piece is in LDS
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t c = Fmt::kByBlock ? 4u * (uint32_t)s + gl : 4u * gl + (uint32_t)s;
            A[j][s][mt] = *reinterpret_cast<const uint4*>(st + 256u * nl + 16u * (c ^ nl));
          }
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): read before the next piece is stored
          __builtin_amdgcn_wave_barrier();
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            uint4& a = A[j][s][mt];
            a.x = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)a.x);
            a.y = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)a.y);
            a.z = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)a.z);
            a.w = (uint32_t)__builtin_amdgcn_ds_bpermute(perm_addr, (int)a.w);
          }
          if constexpr (!Fmt::kByBlock) {
            uint32_t t[4][4];
            transpose_groups(make_uint4(A[j][0][mt].x, A[j][1][mt].x, A[j][2][mt].x, A[j][3][mt].x), t[0]);
            transpose_groups(make_uint4(A[j][0][mt].y, A[j][1][mt].y, A[j][2][mt].y, A[j][3][mt].y), t[1]);
            transpose_groups(make_uint4(A[j][0][mt].z, A[j][1][mt].z, A[j][2][mt].z, A[j][3][mt].z), t[2]);
            transpose_groups(make_uint4(A[j][0][mt].w, A[j][1][mt].w, A[j][2][mt].w, A[j][3][mt].w), t[3]);
#pragma unroll
            for (int s = 0; s < 4; ++s) A[j][s][mt] = make_uint4(t[0][s], t[1][s], t[2][s], t[3][s]);
          }
        }
      }
    }
  };

  // Reduce `cnt` ring entries (tiles first .. first + cnt - 1 of this
  // workgroup's list): thread t owns output (slot t / (256 MT), m tile,
  // lane l, register r) and adds the sixteen wavefront parts in order.
  auto flush = [&](uint32_t first, uint32_t cnt, uint32_t pass) {
    __syncthreads();
    const uint32_t slot = (uint32_t)tid / (256u * MT);
    const uint32_t o = (uint32_t)tid % (256u * MT);
    const int mt = (int)(o / 256u), l = (int)((o % 256u) >> 2), r = (int)(o & 3u);
    if (slot < cnt) {
      float sum = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWide; ++w2) sum += ring[slot][w2][mt][l][r];
      float* const acc = accum + (first + slot) * (256u * MT) + o;   // several passes only
      if (pass > pass_begin) sum = *acc + sum;
      if (pass + 1 < pass_end) {
        *acc = sum;
      } else {
        const uint32_t tt = t0 + (first + slot) * G;
        const uint32_t row = tt * 16u + (uint32_t)(l & 15);
        const uint32_t m = (uint32_t)mt * 16u + 4u * (uint32_t)(l >> 4) + (uint32_t)r;
        if (S == 1u) {
          if (m < M && row < N) Y[(size_t)m * ldy + row] = Fmt::kTensorScale ? sum * ts : sum;
        } else {
          __hip_atomic_store(part + ((size_t)split * T + tt) * (256u * MT) + o, sum, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();                        // the ring is rewritten next
  };

  WSet pa, pb;
  for (uint32_t pass = pass_begin; pass < pass_end; ++pass) {
    // The pass's activation operands, then its first two weight tiles, in
    // the same order on every pass; the table is filled while they are in
    // flight.  Vector loads complete in issue order, so the wait for the
    // activations (at their first use) leaves the weights in flight.
    load_a(pass);
    load_w(pa, t0, pass);
    load_w(pb, min(t0 + G, last), pass);
    if constexpr (kStageA) {
      // Every wavefront's operands out of the ring (and the table complete)
      // before any tile writes to the ring; the weight loads stay in flight.
      if constexpr (Fmt::kLut) {
        if (pass == pass_begin) fill_pair_lut16(lut, tid, 64 * kWide);
      }
      place_a();
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_s_barrier();
    } else {
      if constexpr (Fmt::kLut) {
        if (pass == pass_begin) {
          fill_pair_lut16(lut, tid, 64 * kWide);
          __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wavefront's table stores; loads left in flight
          __builtin_amdgcn_s_barrier();         // the whole table
        }
      }
      place_a();
    }

    uint32_t ti = 0;                        // tiles of this pass done
    // Tile tt from register set w; w is refilled with tile `next` as soon
    // as its registers are consumed (not for the last tile of the pass).
    // kFull: every group of the pass exists and has four blocks, so the
    // steps need no guards and the compiler may overlap one step's table
    // reads with the previous step's arithmetic.
    auto do_tile = [&](WSet& w, uint32_t next, auto reload, auto full) {
      constexpr bool kFull = decltype(full)::value;
      f32x4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const uint32_t q = group_of(pass, j);
        if (kFull || q < ngroups) {          // wavefront-uniform
          typename Fmt::Dec dec;
          Fmt::prepare(to_mfma_lanes(w.r[j]), dec);
          // By block: steps past the last block are skipped.  By element:
          // every step touches all four blocks, and a lane whose block lies
          // past the last one contributes zero weights.
          const uint32_t nsteps = Fmt::kByBlock && !kFull ? min(4u, nb - 4u * q) : 4u;
          const bool live = kFull || Fmt::kByBlock || 4u * q + g < nb;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            if (kFull || (uint32_t)s < nsteps) {
              bf16x8 B = Fmt::operand(dec, s, g, lut, laneoff);
              if (!kFull && !Fmt::kByBlock && !live) B = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[j][s][mt]), B,
                                                                  acc[mt], 0, 0, 0);
            }
          }
        }
      }
      if constexpr (decltype(reload)::value) load_w(w, next, pass);
      const uint32_t slot = ti % (uint32_t)kRing;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ring[slot][wave][mt][lane] = acc[mt];
      ++ti;
      if (ti % (uint32_t)kRing == 0u) flush(ti - (uint32_t)kRing, (uint32_t)kRing, pass);
    };
    // Fixed trip count with clamped, unconditional prefetches (exact waits).
    auto run_tiles = [&](auto full) {
      uint32_t t = t0;
      uint32_t i = 0;
      for (; i + 2 <= n; i += 2) {
        do_tile(pa, min(t + 2 * G, last), std::true_type{}, full);
        t += G;
        do_tile(pb, min(t + 2 * G, last), std::true_type{}, full);
        t += G;
      }
      if (i < n) do_tile(pa, last, std::false_type{}, full);
    };
    // (With four 16-row tiles the guard-free copy of the loop costs registers
    // the kernel does not have: it spilled and ran slower.)
    if (MT <= 2 && (pass + 1u) * kPassGroups * 4u <= nb) run_tiles(std::true_type{});
    else run_tiles(std::false_type{});
    if (ti % (uint32_t)kRing != 0u) flush(ti - ti % (uint32_t)kRing, ti % (uint32_t)kRing, pass);
  }

  if (S > 1u) {
    // Every tile's sums of this split are stored: count the tiles, and add
    // up those whose count this workgroup completes, in split order.  The
    // sums are stored and loaded as device-scope atomics, which the L2
    // caches of the chip keep coherent without a cache writeback or
    // invalidation (a __threadfence() here cost more than the whole GEMM);
    // each wavefront waits for its stores to complete before the barrier,
    // and the counting atomics are issued after it.  The ring, no longer
    // needed, holds the per-tile "last split" flags.
    uint32_t* const flags = reinterpret_cast<uint32_t*>(&ring[0][0][0][0]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (uint32_t i = (uint32_t)tid; i < n; i += 64u * kWide)
      flags[i] = __hip_atomic_fetch_add(counters + t0 + i * G, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                         S - 1u ? 1u : 0u;
    __syncthreads();
    constexpr uint32_t kOut = 256u * MT;
    for (uint32_t e = (uint32_t)tid; e < n * kOut; e += 64u * kWide) {
      const uint32_t i = e / kOut, o = e - i * kOut;
      if (!flags[i]) continue;
      const uint32_t tt = t0 + i * G;
      // Eight loads in flight at a time, added in split order.
      float sum = 0.f;
      for (uint32_t s0 = 0; s0 < S; s0 += 8u) {
        float v[8];
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u)
          v[u] = __hip_atomic_load(part + ((size_t)min(s0 + u, S - 1u) * T + tt) * kOut + o, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (uint32_t u = 0; u < 8u; ++u)
          if (s0 + u < S) sum += v[u];
      }
      const uint32_t l = (o % 256u) >> 2;
      const uint32_t row = tt * 16u + (l & 15u);
      const uint32_t m = (o / 256u) * 16u + 4u * (l >> 4) + (o & 3u);
      if (m < M && row < N) Y[(size_t)m * ldy + row] = Fmt::kTensorScale ? sum * ts : sum;
      if (o == 0u) __hip_atomic_store(counters + tt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Workspace layout: a fixed region of per-tile counters (one launch that
// splits K covers at most kSplitTiles row tiles; taller matrices are
// launched in row chunks), then the sums of every split.  The counters sit
// at the same place for every shape, so the sums of one call never land
// where another call's counters are, and every call leaves them at zero.
constexpr uint32_t kSplitTiles = 16384;
constexpr size_t kCounterBytes = kSplitTiles * 4;

// Launch shape of the persistent kernel for Nc rows: S sets of workgroups
// (one pass of K each when the tiles are few, else one set over all
// passes), G workgroups per set with the tiles spread evenly.
struct SmallPlan {
  uint32_t S, G, tq, tr;
};
SmallPlan small_plan(uint32_t Nc, uint32_t nb, int NQ, uint32_t cap) {
  const uint32_t passes = ((nb + 3u) / 4u + kWide * NQ - 1u) / (kWide * NQ);
  const uint32_t tiles = (Nc + 15u) / 16u;
  SmallPlan p;
  // Fewer than four row tiles per compute unit and K in several passes:
  // each set takes one pass, so that a workgroup works through more tiles
  // per pass instead of paying a pass's operand loads and flushes for one.
  p.S = passes >= 2u && tiles < 4u * cap ? passes : 1u;
  const uint32_t wgs = std::max(1u, cap / p.S);
  const uint32_t per_wg = (tiles + wgs - 1u) / wgs;
  p.G = (tiles + per_wg - 1u) / per_wg;
  p.tq = tiles / p.G;
  p.tr = tiles % p.G;
  return p;
}

// Rows per launch: with several passes per workgroup its outputs (16 * 16 *
// MT per tile) must fit the pass accumulator, and with several sets the
// tiles must fit the counters.
uint64_t small_chunk_rows(uint32_t N, uint32_t nb, int MT, int NQ, uint32_t cap) {
  const uint32_t passes = ((nb + 3u) / 4u + kWide * NQ - 1u) / (kWide * NQ);
  uint64_t rows = N;
  if (passes > 1u) rows = std::min<uint64_t>(rows, 16ull * (kAccFloats / (256u * MT)) * cap);
  return std::min<uint64_t>(rows, 16ull * kSplitTiles);
}

size_t small_workspace(uint32_t N, uint32_t nb, int MT, int NQ, uint32_t cap) {
  size_t need = 0;
  const uint64_t chunk = small_chunk_rows(N, nb, MT, NQ, cap);
  for (uint64_t r0 = 0; r0 < N; r0 += chunk) {
    const uint32_t Nc = (uint32_t)std::min<uint64_t>(N - r0, chunk);
    const SmallPlan p = small_plan(Nc, nb, NQ, cap);
    if (p.S > 1u) need = std::max(need, kCounterBytes + (size_t)p.S * ((Nc + 15u) / 16u) * 256u * (size_t)MT * 4u);
  }
  return need;
}

// Bytes of codes and of scales per 32-element block.
template <class Fmt> constexpr size_t code_bytes() { return std::is_same<Fmt, GemmMXFP6>::value ? 24 : 16; }
template <class Fmt> constexpr size_t scale_bytes() {
  return std::is_same<Fmt, GemmTQ4>::value ? 4 : std::is_same<Fmt, GemmNVFP4>::value ? 2 : 1;
}

template <class Fmt, int MT, int NQ>
hipError_t launch_small(const uint8_t* pk, const uint8_t* sc, const float* ts, uint32_t N, uint32_t nb, const uint8_t* X,
                  int64_t ldx, uint32_t M, float* Y, int64_t ldy, void* ws, hipStream_t s) {
  const uint32_t cap = (uint32_t)device_cu_count();
  uint32_t* counters = static_cast<uint32_t*>(ws);
  float* part = ws ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kCounterBytes) : nullptr;
  const uint64_t chunk = small_chunk_rows(N, nb, MT, NQ, cap);
  for (uint64_t r0 = 0; r0 < N; r0 += chunk) {
    const uint32_t Nc = (uint32_t)std::min<uint64_t>(N - r0, chunk);
    const SmallPlan p = small_plan(Nc, nb, NQ, cap);
    if (p.S > 1u && !ws) return hipErrorInvalidValue;   // the entry points size and check it; never reached
    hipLaunchKernelGGL((gemm_small_kernel<Fmt, MT, NQ>), dim3(p.G * p.S), dim3(64 * kWide), 0, s,
                       pk + r0 * nb * code_bytes<Fmt>(), sc + r0 * nb * scale_bytes<Fmt>(), ts, Nc, nb, X, ldx, M,
                       Y + r0, ldy, p.G, p.tq, p.tr, p.S, part, counters);
  }
  return hipSuccess;
}

// The persistent kernel for one chunk of up to 64 rows: MT = 1 (two groups
// per wavefront and pass), 2 or 4 tiles of 16 activation rows.
template <class Fmt>
hipError_t launch_small_mt(int mt, const uint8_t* pk, const uint8_t* sc, const float* ts, uint32_t N, uint32_t nb,
                           const uint8_t* X, int64_t ldx, uint32_t M, float* Y, int64_t ldy, void* ws,
                           hipStream_t s) {
  if (mt == 1) return launch_small<Fmt, 1, 2>(pk, sc, ts, N, nb, X, ldx, M, Y, ldy, ws, s);
  if (mt == 2) return launch_small<Fmt, 2, 1>(pk, sc, ts, N, nb, X, ldx, M, Y, ldy, ws, s);
  return launch_small<Fmt, 4, 1>(pk, sc, ts, N, nb, X, ldx, M, Y, ldy, ws, s);
}

// Weight groups in flight per wavefront: three where the registers allow.
template <int MT, int RT, bool kF32X>
constexpr int gemm_depth() { return (kF32X ? 2 : 1) * MT * RT <= 4 ? 3 : 2; }
// Workgroups aimed for per compute unit when choosing the row tiles.
constexpr uint32_t kGemmWgPerCu = 2;

template <int MT, int RT, bool kF32X>
void launch_mfma(const uint4* pk, const uint32_t* sc, uint32_t N, uint32_t nb, const uint8_t* X, int64_t ldx,
                 uint32_t M, float* Y, int64_t ldy, hipStream_t s) {
  const dim3 grid((N + 16u * RT - 1) / (16u * RT)), block(kThreads);
  hipLaunchKernelGGL((gemm_mfma_kernel<MT, RT, gemm_depth<MT, RT, kF32X>(), kF32X>), grid, block, 0, s, pk, sc, N, nb, X, ldx, M,
                     Y, ldy);
}

// Weight-row tiles per workgroup: as many as keep about two workgroups per
// compute unit busy (each workgroup reads the whole activation block from
// L2, so fewer, taller workgroups cut that traffic).
template <int MT, bool kF32X>
void launch_mt(const uint4* pk, const uint32_t* sc, uint32_t N, uint32_t nb, const uint8_t* X, int64_t ldx,
               uint32_t M, float* Y, int64_t ldy, hipStream_t s) {
  const uint32_t target = kGemmWgPerCu * (uint32_t)device_cu_count();
  const uint32_t tiles16 = (N + 15u) / 16u;
  if (MT == 1 && !kF32X && tiles16 >= 4u * target) launch_mfma<1, 4, kF32X>(pk, sc, N, nb, X, ldx, M, Y, ldy, s);
  else if (tiles16 >= 2u * target) launch_mfma<MT, 2, kF32X>(pk, sc, N, nb, X, ldx, M, Y, ldy, s);
  else launch_mfma<MT, 1, kF32X>(pk, sc, N, nb, X, ldx, M, Y, ldy, s);
}

}  // namespace

// Activation rows up to which the GEMMs run the VALU kernel (float32 FMAs);
// larger bf16 batches take the MFMA kernel, whose split-K launches need the
// workspace.  The dispatch and the workspace size both read this.  Measured
// over a Llama-3-8B layer: 2 rows 45 us on the VALU kernel against 56 us
// for one padded 16-row MFMA tile; 3 rows 81 against 56 us, 4 rows 72
// against 57 us.
constexpr int kValuRows = 2;

// Workspace bytes of the persistent kernel for an [N, K] weight and M bf16
// activation rows (the largest of its 64-row launches); 0 when no launch
// splits K or the call runs another kernel.
size_t gemm_workspace_bytes(int64_t N, int64_t K, int64_t M, bool xbf16) {
  if (M <= kValuRows || !xbf16 || N <= 0 || K <= 0) return 0;
  const uint32_t nb = (uint32_t)(K / kBlock), cap = (uint32_t)device_cu_count();
  size_t need = 0;
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t mc = (M - m0 < 64) ? M - m0 : 64;
    const int mt = (int)((mc + 15) / 16);
    need = std::max(need, mt == 1 ? small_workspace((uint32_t)N, nb, 1, 2, cap)
                                  : small_workspace((uint32_t)N, nb, mt == 2 ? 2 : 4, 1, cap));
  }
  return need;
}

hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                       const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, void* ws, hipStream_t s) {
  // Up to two rows (or float32 activations below 16 rows) the VALU kernel
  // keeps the rows in registers; from three bf16 rows on, one padded 16-row
  // MFMA tile is faster (kValuRows).
  if (M <= kValuRows || (M < 16 && !xbf16)) return launch_gemm_valu(packed, scales, N, K, M, xr, xbf16, ldx, y, ldy, s);
  const uint32_t nb = (uint32_t)(K / kBlock);
  const uint4* pk = reinterpret_cast<const uint4*>(packed);
  const uint32_t* sc = reinterpret_cast<const uint32_t*>(scales);
  const uint8_t* X = static_cast<const uint8_t*>(xr);
  const int64_t xs = xbf16 ? 2 : 4;
  // At most 64 bf16 or 32 float32 activation rows per launch: the
  // persistent bf16 kernel keeps its operands in registers (up to four
  // 16-row tiles), and float32 activations take three MFMAs per product and
  // twice the operand registers.
  const int64_t chunk = xbf16 ? 64 : 32;
  for (int64_t m0 = 0; m0 < M; m0 += chunk) {
    const int64_t mc = (M - m0 < chunk) ? M - m0 : chunk;
    const uint8_t* Xm = X + m0 * ldx * xs;
    float* Ym = y + m0 * ldy;
    const int mt = (int)((mc + 15) / 16);
    const uint32_t n = (uint32_t)N, mm = (uint32_t)mc;
    if (xbf16) {
      const hipError_t e = launch_small_mt<GemmTQ4>(mt, packed, reinterpret_cast<const uint8_t*>(scales), nullptr, n,
                                                    nb, Xm, ldx, mm, Ym, ldy, ws, s);   // the persistent kernel
      if (e != hipSuccess) return e;
    } else {
      if (mt == 1) launch_mt<1, true>(pk, sc, n, nb, Xm, ldx, mm, Ym, ldy, s);
      else launch_mt<2, true>(pk, sc, n, nb, Xm, ldx, mm, Ym, ldy, s);
    }
  }
  return hipGetLastError();
}

hipError_t launch_blockfp_gemm(int fmt, const uint8_t* codes, const uint8_t* bscales, const float* tscale,
                               int64_t N, int64_t K, int64_t M, const void* x, bool xbf16, int64_t ldx, float* y,
                               int64_t ldy, void* ws, hipStream_t s) {
  // Up to two rows, and float32 activations, on the VALU kernel (rows in
  // registers, any M); from three bf16 rows on, 16-row MFMA tiles with
  // exactly converted bf16 weights.
  if (M <= kValuRows || !xbf16) return launch_blockfp_gemv(fmt, codes, bscales, tscale, N, K, M, x, xbf16, ldx, y, ldy, s);
  const uint32_t nb = (uint32_t)(K / kBlock);
  const uint8_t* X = static_cast<const uint8_t*>(x);
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t mc = (M - m0 < 64) ? M - m0 : 64;
    const uint8_t* Xm = X + m0 * ldx * 2;
    float* Ym = y + m0 * ldy;
    const int mt = (int)((mc + 15) / 16);
    const hipError_t e =
        fmt == TQ_FMT_NVFP4
            ? launch_small_mt<GemmNVFP4>(mt, codes, bscales, tscale, (uint32_t)N, nb, Xm, ldx, (uint32_t)mc, Ym, ldy,
                                         ws, s)
            : launch_small_mt<GemmMXFP6>(mt, codes, bscales, nullptr, (uint32_t)N, nb, Xm, ldx, (uint32_t)mc, Ym, ldy,
                                         ws, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace tq
