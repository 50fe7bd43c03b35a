// turbo4 KV cache on gfx950: q8_0 keys, PolarQuant values (norm, random-sign
// Hadamard rotation of the whole 128-element head vector, 16-centroid
// indices), and decode attention over them (TQ4 page: the paragraph after
// the "格式原理" list, on the PolarQuant steps and the structured rotation;
// "叠加压缩：权重 + KV 缓存", asymmetric q8_0-K / turbo4-V).
//
// Value encode, float32 in this order (contraction off):
//   ss = pairwise tree of w_i^2 (index order); n16 = fp16_sat(sqrt(ss));
//   u = FWHT_128(D w) unnormalised, stages h = 1 .. 64;
//   idx_i = #{k : u_i > fl(nn * m_k)}  (u_i / ||w|| is sqrt(128) times the
//   rotated unit vector's coordinate, close to N(0, 1)).
// Decode: v_hat = (nn / 128) D H c[idx].
//
// Attention keeps the values in the rotated domain: o = sum_t p_t v_hat_t =
// (1/128) D H (sum_t p_t nn_t c[idx_t]), so the split kernel accumulates
// z = sum_t p_t nn_t c[idx_t] with a centroid lookup per element, and the
// combine kernel applies D H / 128 once per head.  The query is quantized
// per 32-element block like the int8 GEMV's activation, so each key block's
// dot product is an exact integer (v_dot4_i32_i8).
#pragma clang fp contract(off)

#include <algorithm>

#include <mutex>

#include "tq_internal.hpp"
#include "tq_codes.hpp"

// Split partials of tq_attn_decode_noalloc (TQ_ATTN_NOALLOC_SCRATCH_BYTES).
static __device__ __align__(256) float scratch[TQ_ATTN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace tq {
namespace {

constexpr int kD = 128;                 // head dimension
constexpr int kChunk = 256;             // tokens per split workgroup
constexpr int kThreads = 256;
constexpr int kLanesPerVec = 8;         // encode: 16 elements per lane
constexpr float kLog2e = 1.44269504088896340736f;

struct Signs {
  uint32_t w[4];
};

// Sums over the 2, 4 and 8 lanes of an aligned 8-lane group with DPP: lane
// ^ 1 and lane ^ 2 by quad permutes, the other quad of the group by the
// half-row mirror (lane i <-> 7 - i).
__device__ __forceinline__ int dpp_xor1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_mirror8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}

// Float32 value shuffled from lane ^ m (within the wavefront).
__device__ __forceinline__ float xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Elements 16 l .. 16 l + 15 of a vector held by lane l of an 8-lane group:
// the unnormalised FWHT_128 in the oracle's stage order (in-lane stages h =
// 1, 2, 4, 8, then lanes l ^ 1, l ^ 2, l ^ 4 for h = 16, 32, 64).  For each
// pair (a, b) with a at the lower index the result is (a + b, a - b).
__device__ __forceinline__ void fwht128_group(float (&v)[16], int sub) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) {
    const bool upper = (sub & m) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = xor_f(v[i], m);
      v[i] = upper ? p - v[i] : v[i] + p;
    }
  }
}

// Sign of element 16 sub + i: bit (16 sub + i) of the 128-bit mask.
__device__ __forceinline__ bool sign_bit(const Signs& s, int sub, int i) {
  return (s.w[sub >> 1] >> (16 * (sub & 1) + i)) & 1u;
}

// --------------------------------------------------------------------------
// q8_0 rows: one thread per 32-element block.
// --------------------------------------------------------------------------
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void q8_rows_kernel(const uint8_t* __restrict__ X, uint32_t total,
                                                           uint4* __restrict__ codes, uint16_t* __restrict__ scales) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= total) return;
  float v[32];
  load_block<kBf16>(X + (size_t)g * (kBf16 ? 64 : 128), v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t d16 = f16_sat(amax / 127.0f);
  const float dd = f16_bits_to_f32(d16);
  const float r = __builtin_amdgcn_rcpf(dd);
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) word |= q8_code(v[4 * k + j], dd, r) << (8 * j);
    w[k] = word;
  }
  codes[2 * (size_t)g] = make_uint4(w[0], w[1], w[2], w[3]);
  codes[2 * (size_t)g + 1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[g] = (uint16_t)d16;
}

// --------------------------------------------------------------------------
// turbo4 value encode / decode: an 8-lane group per vector.
// --------------------------------------------------------------------------
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void turbo4_encode_kernel(const uint8_t* __restrict__ V, uint32_t nvec,
                                                                 Signs sg, Codebook cb,
                                                                 uint2* __restrict__ packed,
                                                                 uint16_t* __restrict__ norms) {
  __shared__ uint2 cells[kCells];
  build_cells(cb, cells);
  __syncthreads();
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t vec = tid / kLanesPerVec;
  const int sub = (int)(tid % kLanesPerVec);
  // Every lane of a group takes part in the shuffles; lanes past the last
  // vector work on a clamped one and store nothing.
  const uint32_t vv = min(vec, nvec - 1u);
  float w[16];
  if constexpr (kBf16) {
    const uint4* p = reinterpret_cast<const uint4*>(V + ((size_t)vv * kD + 16 * sub) * 2);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint4 u = p[t];
      const uint32_t x[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        w[8 * t + 2 * k] = bf16_lo(x[k]);
        w[8 * t + 2 * k + 1] = bf16_hi(x[k]);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(V + ((size_t)vv * kD + 16 * sub) * 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 u = p[t];
      w[4 * t] = u.x; w[4 * t + 1] = u.y; w[4 * t + 2] = u.z; w[4 * t + 3] = u.w;
    }
  }
  // Norm: the pairwise tree over 128 squares in index order (16 in the lane,
  // then lane pairs, quads, the group).
  float s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = w[i] * w[i];
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
#pragma unroll
    for (int i = 0; i < m; ++i) s[i] = s[2 * i] + s[2 * i + 1];
  }
  float ss = s[0];
  ss = ss + xor_f(ss, 1);
  ss = ss + xor_f(ss, 2);
  ss = ss + xor_f(ss, 4);
  const uint32_t n16 = f16_sat(__builtin_sqrtf(ss));
  const float nn = f16_bits_to_f32(n16);

#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = sign_bit(sg, sub, i) ? -w[i] : w[i];
  fwht128_group(w, sub);

  // idx = #{k : u > fl(nn m_k)}, by the cell table.
  const float r8 = 8.0f * __builtin_amdgcn_rcpf(nn);
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t idx = nearest_index(w[i], nn, r8, cells);
    if (i < 8) lo |= idx << (4 * i);
    else hi |= idx << (4 * (i - 8));
  }
  if (vec < nvec) {
    packed[(size_t)vec * 8 + sub] = make_uint2(lo, hi);
    if (sub == 0) norms[vec] = (uint16_t)n16;
  }
}

// v_hat = (nn / 128) D H c[idx], float32 out.
__global__ __launch_bounds__(kThreads) void turbo4_decode_kernel(const uint2* __restrict__ packed,
                                                                 const uint16_t* __restrict__ norms, uint32_t nvec,
                                                                 Signs sg, Codebook cb, float* __restrict__ out) {
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t vec = tid / kLanesPerVec;
  const int sub = (int)(tid % kLanesPerVec);
  const uint32_t vv = min(vec, nvec - 1u);
  const uint2 p = packed[(size_t)vv * 8 + sub];
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t word = i < 8 ? p.x : p.y;
    const uint32_t idx = (word >> (4 * (i & 7))) & 15u;
    float c = cb.c[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) c = idx == (uint32_t)k ? cb.c[k] : c;
    v[i] = c;
  }
  fwht128_group(v, sub);
  const float scale = f16_bits_to_f32_exact(norms[vv]) * (1.0f / kD);
  if (vec < nvec) {
    float4* o = reinterpret_cast<float4*>(out + (size_t)vec * kD + 16 * sub);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * t + j;
        const float x = v[i] * scale;
        r[j] = sign_bit(sg, sub, i) ? -x : x;
      }
      o[t] = make_float4(r[0], r[1], r[2], r[3]);
    }
  }
}

// --------------------------------------------------------------------------
// Decode attention, split over the cache: workgroup (split s, cache head g,
// sequence b) takes tokens [256 s, 256 s + 256) of sequence b and the G
// query heads that read cache head g.  The cache is head-major ([B, Hkv,
// T_max, ...]), so a workgroup streams contiguous key codes (32 KiB), key
// scales, value nibbles (16 KiB) and norms.  It writes, per head, the running
// maximum m (log2 domain), the sum l of 2^(s_t - m), and the rotated-domain
// sum z = sum_t 2^(s_t - m) nn_t c[idx_t] (128 floats) to the workspace.
// --------------------------------------------------------------------------
constexpr int kPart = kD + 2;           // floats per (sequence, head, split): m, l, z[128]
// Query heads per cache head from which the value sums run on the matrix
// cores (16 rows per MFMA whatever G is).  16 sequences x 4096 tokens, 32
// query heads, per layer: G = 4 45.3 -> 39.7 us, G = 8 42.1 -> 31.8 us;
// G = 2 55.4 against 55.8 us, and G = 1 83.6 -> 91.4 us, where most of the
// 16 rows are padding.
constexpr int kMfmaValueHeads = 4;
// And from which the key scores do (v_mfma_i32_16x16x32_i8, bit-identical
// scores): same layout, G = 8 31.9 -> 27.9 us per layer, but G = 4 39.6 ->
// 41.6 us; the B operand needs twice the key load instructions (8-byte
// pieces of four blocks per lane instead of 16-byte halves of one).
constexpr int kMfmaScoreHeads = 8;

template <int G, bool kBf16Q>
__global__ __launch_bounds__(kThreads) void attn_split_kernel(
    const uint8_t* __restrict__ Q, const int32_t* __restrict__ lengths, const uint4* __restrict__ kcodes,
    const uint16_t* __restrict__ kscales, const uint32_t* __restrict__ vpacked, const uint16_t* __restrict__ vnorms,
    uint32_t Tmax, uint32_t Hkv, uint32_t S, Codebook cb, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) int8_t qs[G][kD];       // quantized query
  __shared__ float dq[G][4];
  __shared__ float lut[16][32];                                    // centroid k, copy lane % 32
  __shared__ float sc[G][kChunk];                                  // scores, then 2^(s - m)
  __shared__ float red[4][G][kD];                                  // per-wavefront z partials
  __shared__ float stat[G][2];
  __shared__ __attribute__((aligned(8))) uint16_t ksl[G >= kMfmaScoreHeads ? kChunk * 4 : 1];   // key block scales

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int32_t Lraw = lengths[b];
  const uint32_t L = (uint32_t)min(max(Lraw, 0), (int32_t)Tmax);
  const uint32_t t0 = s * kChunk;
  if (t0 >= L) return;                     // the combine reads only the splits that hold tokens
  const uint32_t n = min((uint32_t)kChunk, L - t0);
  const uint32_t Hq = Hkv * G;
  const size_t kv0 = ((size_t)b * Hkv + g) * Tmax + t0;       // cache row of token t0 (head-major rows)

  // Every key load of the chunk is issued here, before anything waits (8
  // lanes per token, 16 bytes each, 32 tokens per workgroup pass); the
  // value loads (16 lanes per token, 4 bytes each, 16 tokens per pass) are
  // issued after the scores, so their registers are not held through the
  // score phase and they arrive during the softmax.  Tokens past the chunk
  // re-read its last token and are masked.
  const int sub = lane & 7, slot = lane >> 4, e16 = lane & 15;
  // Chunk base pointers (wavefront-uniform) and 32-bit lane offsets; a full
  // chunk (the common case) needs no clamping.
  const uint4* kb = kcodes + kv0 * 8;
  const uint16_t* ksb = kscales + kv0 * 4;
  const uint32_t* vbp = vpacked + kv0 * 16;
  const uint16_t* vnb = vnorms + kv0;
  const bool full = n == (uint32_t)kChunk;
  const uint32_t ck = (uint32_t)(wave * 8 + (lane >> 3)), cv = (uint32_t)(wave * 4 + slot);
  // Scores on the int8 matrix cores (G >= kMfmaScoreHeads): wavefront w takes
  // tokens 64 w + 16 tg + l % 16 (tg = 0 .. 3); lane l loads bytes 8 (l / 16)
  // .. + 7 of each of the token's four q8_0 blocks (the MFMA B operand), and
  // the chunk's block scales go through LDS (they are only 2-byte aligned).
  constexpr bool kMS = G >= kMfmaScoreHeads;
  constexpr int kKq = kMS ? 1 : kChunk / 32;
  uint4 kq[kKq];
  uint32_t kscl[kKq], vb[kChunk / 16], vnr[kChunk / 16];
  uint2 km[kMS ? 16 : 1];
  uint32_t ksr[kMS ? 4 : 1];
  if constexpr (kMS) {
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const uint32_t tl = min((uint32_t)(wave * 64 + tg * 16 + e16), n - 1u);
      const uint2* kr = reinterpret_cast<const uint2*>(kb + tl * 8);
#pragma unroll
      for (int bk = 0; bk < 4; ++bk) km[tg * 4 + bk] = kr[4 * bk + slot];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ksr[j] = ksb[min((uint32_t)(tid + kThreads * j), 4u * n - 1u)];
  } else if (full) {
#pragma unroll
    for (int it = 0; it < kChunk / 32; ++it) {
      const uint32_t tl = (uint32_t)(it * 32) + ck;
      kq[it] = kb[tl * 8 + sub];
      kscl[it] = ksb[tl * 4 + (sub >> 1)];
    }
  } else {
#pragma unroll
    for (int it = 0; it < kChunk / 32; ++it) {
      const uint32_t tl = min((uint32_t)(it * 32) + ck, n - 1u);
      kq[it] = kb[tl * 8 + sub];
      kscl[it] = ksb[tl * 4 + (sub >> 1)];
    }
  }
  auto load_values = [&]() {
    if (full) {
#pragma unroll
      for (int it = 0; it < kChunk / 16; ++it) {
        const uint32_t tl = (uint32_t)(it * 16) + cv;
        vb[it] = vbp[tl * 16 + e16];
        vnr[it] = vnb[tl];
      }
    } else {
#pragma unroll
      for (int it = 0; it < kChunk / 16; ++it) {
        const uint32_t tl = min((uint32_t)(it * 16) + cv, n - 1u);
        vb[it] = vbp[tl * 16 + e16];
        vnr[it] = vnb[tl];
      }
    }
  };

  // Query quantization: thread t < 16 G takes 8 elements of head t / 16;
  // four threads share a 32-element block.
  if (tid < 16 * G) {
    const int h = tid >> 4, e0 = (tid & 15) * 8;
    const size_t qoff = ((size_t)b * Hq + g * G + h) * kD + e0;
    float x[8];
    if constexpr (kBf16Q) {
      const uint4 u = *reinterpret_cast<const uint4*>(Q + qoff * 2);
      x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
      x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
    } else {
      const float4* p = reinterpret_cast<const float4*>(Q + qoff * 4);
      const float4 a = p[0], c = p[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, xor_f(amax, 1));
    amax = fmaxf(amax, xor_f(amax, 2));
    const float d = amax / 127.0f;
    const float dsafe = d > 0.f ? d : 1.0f;                 // the division runs unconditionally (no branch)
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float c = d > 0.f ? __builtin_rintf(x[i] / dsafe) : 0.f;
      c = fminf(fmaxf(c, -127.f), 127.f);
      const uint32_t byte = (uint32_t)(int32_t)c & 0xffu;
      if (i < 4) w0 |= byte << (8 * i);
      else w1 |= byte << (8 * (i - 4));
    }
    *reinterpret_cast<uint2*>(&qs[h][e0]) = make_uint2(w0, w1);
    if ((tid & 3) == 0) dq[h][(tid & 15) >> 2] = d;
  }
  for (int i = tid; i < 16 * 32; i += kThreads) lut[i >> 5][i & 31] = cb.c[i >> 5];
  if constexpr (kMS) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ksl[tid + kThreads * j] = (uint16_t)ksr[j];
  }
  __syncthreads();

  if constexpr (kMS) {
    // One v_mfma_i32_16x16x32_i8 per q8_0 block and 16 tokens: A = the
    // quantized query (row h = l % 16, zero past G; bytes 32 b + 8 (l / 16)
    // .. + 7), B = the keys; the exact integer dot of block b for head
    // 4 (l / 16) + r and token l % 16 lands in lane l, register r, and is
    // scaled and summed over the blocks as ((f0 + f1) + (f2 + f3)), the
    // order of the VALU version, so the scores are the same bit for bit.
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const float scale = kLog2e * 0.08838834764831845f;     // log2(e) / sqrt(128), float32
    const int hrow = lane & 15;
    long qa[4];
#pragma unroll
    for (int bk = 0; bk < 4; ++bk)
      qa[bk] = hrow < G ? *reinterpret_cast<const long*>(&qs[hrow < G ? hrow : 0][32 * bk + 8 * slot]) : 0l;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const uint32_t tl = (uint32_t)(wave * 64 + tg * 16 + e16);
      const uint2 sr = *reinterpret_cast<const uint2*>(&ksl[4 * tl]);
      const float dk[4] = {f16_bits_to_f32(sr.x & 0xffffu), f16_bits_to_f32(sr.x >> 16),
                           f16_bits_to_f32(sr.y & 0xffffu), f16_bits_to_f32(sr.y >> 16)};
      i32x4 c[4];
#pragma unroll
      for (int bk = 0; bk < 4; ++bk)
        c[bk] = __builtin_amdgcn_mfma_i32_16x16x32_i8(qa[bk], __builtin_bit_cast(long, km[tg * 4 + bk]),
                                                      i32x4{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * slot + r;
        if (h < G) {
          float f[4];
#pragma unroll
          for (int bk = 0; bk < 4; ++bk) f[bk] = (float)c[bk][r] * (dk[bk] * dq[h][bk]);
          sc[h][tl] = ((f[0] + f[1]) + (f[2] + f[3])) * scale;
        }
      }
    }
  } else {
    // Scores on the VALU: 8 lanes per token, 16 key bytes per lane (half a
    // q8_0 block).
    const float scale = kLog2e * 0.08838834764831845f;     // log2(e) / sqrt(128), float32
    uint4 qc[G];
    float dqs[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qc[h] = *reinterpret_cast<const uint4*>(&qs[h][16 * sub]);
      dqs[h] = dq[h][sub >> 1];
    }
#pragma unroll
    for (int it = 0; it < kChunk / 32; ++it) {
      const uint32_t tl = (uint32_t)(it * 32 + wave * 8 + (lane >> 3));
      const uint4 kc = kq[it];
      const float dk = f16_bits_to_f32(kscl[it]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        int isum = __builtin_amdgcn_sdot4((int)kc.x, (int)qc[h].x, 0, false);
        isum = __builtin_amdgcn_sdot4((int)kc.y, (int)qc[h].y, isum, false);
        isum = __builtin_amdgcn_sdot4((int)kc.z, (int)qc[h].z, isum, false);
        isum = __builtin_amdgcn_sdot4((int)kc.w, (int)qc[h].w, isum, false);
        isum += dpp_xor1(isum);                             // the whole 32-element block
        float f = (float)isum * (dk * dqs[h]);
        f = f + dpp_xor2(f);                                 // two blocks
        f = f + dpp_mirror8(f);                              // all four
        sc[h][tl] = f * scale;               // the token's 8 lanes store the same value; entries past n are unused
      }
    }
  }
  __syncthreads();

  load_values();                           // in flight during the softmax statistics

  // Softmax statistics per head: wavefront w takes heads w, w + 4.
  for (int h = wave; h < G; h += 4) {
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kChunk / 64; ++k) {
      const uint32_t i = (uint32_t)(lane + 64 * k);
      m = fmaxf(m, i < n ? sc[h][i] : -__builtin_inff());
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, xor_f(m, o));
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < kChunk / 64; ++k) {
      const uint32_t i = (uint32_t)(lane + 64 * k);
      const float e = i < n ? __builtin_amdgcn_exp2f(sc[h][i] - m) : 0.f;
      sc[h][i] = e;
      l += e;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += xor_f(l, o);
    if (lane == 0) {
      stat[h][0] = m;
      stat[h][1] = l;
    }
  }
  __syncthreads();

  // Values on the matrix cores (G >= kMfmaValueHeads): z[h][j] =
  // sum_t w[h][t] c[idx_t][j] with w = 2^(s_t - m) nn_t is a (heads x
  // tokens) by (tokens x 128) product, one
  // v_mfma_f32_16x16x16f16 per 16 tokens and 16 elements (heads padded to
  // 16 rows; the matrix cores cost the same for every G up to 16).  Lane l
  // keeps the value loads it has: word e16 = l % 16 (elements 8 e16 .. 8 e16
  // + 7) of tokens it * 16 + 4 wave + slot, slot = l / 16, it = 0 .. 15.  So
  // k-group q (q = 0 .. 3) takes, from lane l, its tokens it = 4 q + e as
  // k = 4 slot + e: the A operand (row h = l % 16, k = 4 (l / 16) + e) is
  // w[h] of those tokens and the B operand (column n = l % 16, the same k) is
  // centroid nibble dt of their words, so output column n of tile dt is
  // element 8 n + dt.  Both operands are fp16: a centroid carries 11
  // significant bits, and w is scaled by 2^sw so that the wavefront's
  // largest norm lands just below 2^15 (w = p nn 2^sw < 2^15, no overflow;
  // only weights more than 2^29 below the largest become fp16 subnormals);
  // the float32 sums are scaled back by 2^-sw (exact) before they are stored.
  if constexpr (G >= kMfmaValueHeads) {
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int copy = lane & 31;
    const int hrow = lane & 15;
    float nmax = 0.f;
#pragma unroll
    for (int it = 0; it < kChunk / 16; ++it) {
      const uint32_t tl = (uint32_t)(it * 16 + wave * 4 + slot);
      nmax = fmaxf(nmax, tl < n ? f16_bits_to_f32(vnr[it]) : 0.f);
    }
    nmax = fmaxf(nmax, xor_f(nmax, 16));
    nmax = fmaxf(nmax, xor_f(nmax, 32));
    int ex = 0;
    (void)__builtin_frexpf(nmax, &ex);                       // nmax < 2^ex (0 for nmax = 0)
    const int sw = nmax > 0.f ? 15 - ex : 0;
    const float up = __builtin_ldexpf(1.0f, sw), down = __builtin_ldexpf(1.0f, -sw);
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int it = 4 * q + e;
        const uint32_t tl = (uint32_t)(it * 16 + wave * 4 + slot);
        const uint32_t tc = min(tl, n - 1u);
        const float nn = tl < n ? f16_bits_to_f32(vnr[it]) : 0.f;
        const float w = hrow < G ? sc[hrow < G ? hrow : 0][tc] * nn * up : 0.f;
        a[e] = (_Float16)w;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        half4 bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = (_Float16)lut[__builtin_amdgcn_ubfe(vb[4 * q + e], 4 * dt, 4)][copy];
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bv, acc[dt], 0, 0, 0);
      }
    }
    // Lane l holds heads 4 (l / 16) + r, element 8 (l % 16) + dt.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * slot + r;
      if (h < G) {
        float4* dst = reinterpret_cast<float4*>(&red[wave][h][8 * e16]);
        dst[0] = make_float4(acc[0][r] * down, acc[1][r] * down, acc[2][r] * down, acc[3][r] * down);
        dst[1] = make_float4(acc[4][r] * down, acc[5][r] * down, acc[6][r] * down, acc[7][r] * down);
      }
    }
  } else {
    // Values on the VALU: 4 tokens per wavefront step, 16 lanes per token,
    // 8 elements (4 bytes of nibbles) per lane.
    const int copy = lane & 31;
    float z[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) z[h][i] = 0.f;
    // Branch-free: a token past the chunk reads the chunk's last score and
    // gets weight 0, so the compiler can schedule the lookups of later steps
    // early (a branch per step left every step's LDS latency exposed).
#pragma unroll
    for (int it = 0; it < kChunk / 16; ++it) {
      const uint32_t tl = (uint32_t)(it * 16 + wave * 4 + slot);
      const uint32_t tc = min(tl, n - 1u);
      const uint32_t bits = vb[it];
      const float nn = tl < n ? f16_bits_to_f32(vnr[it]) : 0.f;
      float c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = lut[__builtin_amdgcn_ubfe(bits, 4 * i, 4)][copy];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float wgt = sc[h][tc] * nn;
#pragma unroll
        for (int i = 0; i < 8; ++i) z[h][i] = __builtin_fmaf(wgt, c[i], z[h][i]);
      }
    }
    // Sum the four token slots of the wavefront, then the wavefronts.
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = z[h][i];
        v = v + xor_f(v, 16);
        v = v + xor_f(v, 32);
        z[h][i] = v;
      }
    if (slot == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float4* r = reinterpret_cast<float4*>(&red[wave][h][8 * e16]);
        r[0] = make_float4(z[h][0], z[h][1], z[h][2], z[h][3]);
        r[1] = make_float4(z[h][4], z[h][5], z[h][6], z[h][7]);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kD; i += kThreads) {
    const int h = i / kD, e = i % kD;
    const float v = (red[0][h][e] + red[1][h][e]) + (red[2][h][e] + red[3][h][e]);
    float* dst = part + (((size_t)b * Hq + g * G + h) * S + s) * kPart;
    dst[2 + e] = v;
    if (e == 0) {
      dst[0] = stat[h][0];
      dst[1] = stat[h][1];
    }
  }
}

// Combine the splits of (sequence b, head h) and rotate back:
// o = (1/128) D H (Z / L_total).  Thread i computes output element i: up to
// 16 splits it requests every split's maximum, sum and z_i at once (one
// round trip of loads) and merges them in split order, M = max_j m_j, then
// l and z_i weighted by 2^(m_j - M).  With more splits the 128 threads first
// reduce the (m_j, l_j) pairs together, then each reads its z_i 32 splits at
// a time.  H is then applied in butterflies: stride 64 through LDS (the two
// wavefronts), strides 32 .. 1 by shuffles.
__global__ __launch_bounds__(kD) void attn_combine_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ lengths, uint32_t Tmax,
                                                          uint32_t Hq, uint32_t S, Signs sg, float* __restrict__ out) {
  constexpr uint32_t kIn = 16;            // splits merged in one round trip of loads
  constexpr uint32_t kZ = 32;             // z values a thread requests at once beyond that
  __shared__ float zs[kD];
  __shared__ float red[2][2];
  const int i = threadIdx.x, lane = i & 63;
  const uint32_t h = blockIdx.x, b = blockIdx.y;
  const uint32_t L = (uint32_t)min(max(lengths[b], 0), (int32_t)Tmax);
  float* o = out + ((size_t)b * Hq + h) * kD;
  if (L == 0) {
    o[i] = 0.f;
    return;
  }
  const uint32_t ns = (L + kChunk - 1) / kChunk;
  const float* p = part + ((size_t)b * Hq + h) * S * kPart;
  float M = -__builtin_inff(), l = 0.f, z = 0.f;
  if (ns <= kIn) {
    float mv[kIn], lv[kIn], zv[kIn];
#pragma unroll
    for (uint32_t u = 0; u < kIn; ++u) {
      const float* q = p + (size_t)min(u, ns - 1u) * kPart;     // repeats of the last split: no effect on M
      mv[u] = q[0];
      lv[u] = q[1];
      zv[u] = q[2 + i];
    }
#pragma unroll
    for (uint32_t u = 0; u < kIn; ++u) M = fmaxf(M, mv[u]);
#pragma unroll
    for (uint32_t u = 0; u < kIn; ++u) {   // no branch: a branch per split would hold its load back
      const float w = u < ns ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f;
      l += lv[u] * w;
      z += zv[u] * w;
    }
  } else {
    // Thread t reduces splits t, t + 128, ... to (m_t, l_t); each wavefront
    // merges its threads' pairs and the two wavefronts meet in LDS.
    float mt = -__builtin_inff(), lt = 0.f;
    for (uint32_t j = i; j < ns; j += kD) {
      const float mj = p[(size_t)j * kPart], lj = p[(size_t)j * kPart + 1];
      const float mn = fmaxf(mt, mj);
      lt = lt * __builtin_amdgcn_exp2f(mt - mn) + lj * __builtin_amdgcn_exp2f(mj - mn);
      mt = mn;
    }
    float Mw = mt;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) Mw = fmaxf(Mw, xor_f(Mw, m));
    float lw = mt == -__builtin_inff() ? 0.f : lt * __builtin_amdgcn_exp2f(mt - Mw);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) lw += xor_f(lw, m);
    if (lane == 0) {
      red[i >> 6][0] = Mw;
      red[i >> 6][1] = lw;
    }
    __syncthreads();
    M = fmaxf(red[0][0], red[1][0]);       // finite: wavefront 0 holds split 0
    l = red[0][1] * __builtin_amdgcn_exp2f(red[0][0] - M) + red[1][1] * __builtin_amdgcn_exp2f(red[1][0] - M);
    for (uint32_t j0 = 0; j0 < ns; j0 += kZ) {
      float mv[kZ], zv[kZ];
#pragma unroll
      for (uint32_t u = 0; u < kZ; ++u) {
        const float* q = p + (size_t)min(j0 + u, ns - 1u) * kPart;
        mv[u] = q[0];
        zv[u] = q[2 + i];
      }
#pragma unroll
      for (uint32_t u = 0; u < kZ; ++u) z += zv[u] * (j0 + u < ns ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f);
    }
  }
  zs[i] = z / l;
  __syncthreads();
  // (a, b) at indices (j, j + s), j without bit s: a + b at j, a - b at j + s.
  const float pv = zs[i ^ 64];
  float v = zs[i];
  v = (i & 64) ? pv - v : v + pv;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float pm = xor_f(v, m);
    v = (lane & m) ? pm - v : v + pm;
  }
  const float r = v * (1.0f / kD);
  o[i] = ((sg.w[i >> 5] >> (i & 31)) & 1u) ? -r : r;
}

inline Signs signs_of(const uint32_t* w) { return Signs{{w[0], w[1], w[2], w[3]}}; }
inline uint32_t grid_for(uint64_t threads) { return (uint32_t)((threads + kThreads - 1) / kThreads); }

template <bool kBf16Q>
void launch_split(int G, dim3 grid, const uint8_t* q, const int32_t* len, const uint4* kc, const uint16_t* ks,
                  const uint32_t* vp, const uint16_t* vn, uint32_t Tmax, uint32_t Hkv, uint32_t S, const Codebook& cb,
                  float* part, hipStream_t s) {
#define TQ_SPLIT(GG)                                                                                         \
  hipLaunchKernelGGL((attn_split_kernel<GG, kBf16Q>), grid, dim3(kThreads), 0, s, q, len, kc, ks, vp, vn, Tmax, \
                     Hkv, S, cb, part)
  switch (G) {
    case 1: TQ_SPLIT(1); break;
    case 2: TQ_SPLIT(2); break;
    case 4: TQ_SPLIT(4); break;
    default: TQ_SPLIT(8); break;
  }
#undef TQ_SPLIT
}

}  // namespace

size_t attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Tmax) {
  const int64_t S = (Tmax + kChunk - 1) / kChunk;
  return (size_t)(B * Hq * S * kPart) * sizeof(float);
}

hipError_t launch_q8_rows(const void* X, bool bf16, int64_t nblocks, int8_t* codes, uint16_t* scales,
                          hipStream_t s) {
  const int64_t per_launch = (int64_t)1 << 30;
  const uint8_t* x = static_cast<const uint8_t*>(X);
  for (int64_t b0 = 0; b0 < nblocks; b0 += per_launch) {
    const uint32_t total = (uint32_t)std::min<int64_t>(nblocks - b0, per_launch);
    uint4* c = reinterpret_cast<uint4*>(codes) + 2 * b0;
    if (bf16)
      hipLaunchKernelGGL(q8_rows_kernel<true>, dim3(grid_for(total)), dim3(kThreads), 0, s, x + b0 * 64, total, c,
                         scales + b0);
    else
      hipLaunchKernelGGL(q8_rows_kernel<false>, dim3(grid_for(total)), dim3(kThreads), 0, s, x + b0 * 128, total, c,
                         scales + b0);
  }
  return hipGetLastError();
}

hipError_t launch_turbo4_encode(const void* V, bool bf16, int64_t nvec, const uint32_t* sign, uint8_t* packed,
                                uint16_t* norms, hipStream_t s) {
  const Codebook& cb = host_codebook();
  const int64_t per_launch = (int64_t)1 << 26;
  const uint8_t* v = static_cast<const uint8_t*>(V);
  for (int64_t v0 = 0; v0 < nvec; v0 += per_launch) {
    const uint32_t cnt = (uint32_t)std::min<int64_t>(nvec - v0, per_launch);
    const dim3 grid(grid_for((uint64_t)cnt * kLanesPerVec));
    uint2* p = reinterpret_cast<uint2*>(packed) + v0 * 8;
    if (bf16)
      hipLaunchKernelGGL(turbo4_encode_kernel<true>, grid, dim3(kThreads), 0, s, v + v0 * kD * 2, cnt,
                         signs_of(sign), cb, p, norms + v0);
    else
      hipLaunchKernelGGL(turbo4_encode_kernel<false>, grid, dim3(kThreads), 0, s, v + v0 * kD * 4, cnt,
                         signs_of(sign), cb, p, norms + v0);
  }
  return hipGetLastError();
}

hipError_t launch_turbo4_decode(const uint8_t* packed, const uint16_t* norms, int64_t nvec, const uint32_t* sign,
                                float* out, hipStream_t s) {
  const Codebook& cb = host_codebook();
  const int64_t per_launch = (int64_t)1 << 26;
  for (int64_t v0 = 0; v0 < nvec; v0 += per_launch) {
    const uint32_t cnt = (uint32_t)std::min<int64_t>(nvec - v0, per_launch);
    hipLaunchKernelGGL(turbo4_decode_kernel, dim3(grid_for((uint64_t)cnt * kLanesPerVec)), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint2*>(packed) + v0 * 8, norms + v0, cnt, signs_of(sign), cb,
                       out + v0 * kD);
  }
  return hipGetLastError();
}

hipError_t launch_attn_decode(const void* q, bool qbf16, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tmax,
                              const int32_t* lengths, const int8_t* kcodes, const uint16_t* kscales,
                              const uint8_t* vpacked, const uint16_t* vnorms, const uint32_t* sign, float* o,
                              void* workspace, hipStream_t s) {
  const uint32_t S = (uint32_t)((Tmax + kChunk - 1) / kChunk);
  const int G = (int)(Hq / Hkv);
  const dim3 grid(S, (uint32_t)Hkv, (uint32_t)B);
  float* part = static_cast<float*>(workspace);
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const uint4* kc = reinterpret_cast<const uint4*>(kcodes);
  const uint32_t* vp = reinterpret_cast<const uint32_t*>(vpacked);
  const Codebook& cb = host_codebook();
  if (qbf16)
    launch_split<true>(G, grid, qb, lengths, kc, kscales, vp, vnorms, (uint32_t)Tmax, (uint32_t)Hkv, S, cb, part, s);
  else
    launch_split<false>(G, grid, qb, lengths, kc, kscales, vp, vnorms, (uint32_t)Tmax, (uint32_t)Hkv, S, cb, part,
                        s);
  hipLaunchKernelGGL(attn_combine_kernel, dim3((uint32_t)Hq, (uint32_t)B), dim3(kD), 0, s, part, lengths,
                     (uint32_t)Tmax, (uint32_t)Hq, S, signs_of(sign), o);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Decode attention for callers that cannot allocate (code under graph
// capture, serving loops): the split partials go to a file-scope device
// array instead of a caller workspace.  Every device the library runs on
// holds its own copy until the process ends; calls on one device share it,
// so calls that overlap on one device race.  Nothing in it needs clearing:
// the combine kernel reads only the partials the split kernel wrote in the
// same call.
// --------------------------------------------------------------------------
namespace {
std::mutex g_scratch_mu;
float* g_scratch_dev[64] = {nullptr};    // device address of `scratch`, per device ordinal
}  // namespace

// The device address of `scratch` on the current device, looked up once per
// device with that device current (the host-side name is only a stand-in).
hipError_t attn_scratch_ptr(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_attn_decode_noalloc(const void* q, bool qbf16, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tmax,
                                      const int32_t* lengths, const int8_t* kcodes, const uint16_t* kscales,
                                      const uint8_t* vpacked, const uint16_t* vnorms, const uint32_t* sign, float* o,
                                      hipStream_t s) {
  float* ws = nullptr;
  const hipError_t e = attn_scratch_ptr(&ws);
  if (e != hipSuccess) return e;
  return launch_attn_decode(q, qbf16, B, Hq, Hkv, Tmax, lengths, kcodes, kscales, vpacked, vnorms, sign, o, ws, s);
}

}  // namespace tq
