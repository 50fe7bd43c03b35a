// Exact code selection shared by the quantizers (TQ4_1S weights, the turbo4
// value cache, the int8 transcode and the q8_0 key cache): the nearest
// Lloyd-Max centroid by a cell table, a saturating fp16 scale, and
// rint(fl(v / d)) without a division per element.  Each reproduces its
// float32 definition exactly.
#pragma once

#include "tq_internal.hpp"

namespace tq {

// Index of the nearest centroid, idx = #{k in 0..14 : w > fl(dd * m_k)}.
//
// A table of 42 cells over the normalised value t = w / dd replaces a
// comparison tree: cell c covers t in [(c - 21) / 8, (c - 20) / 8) (cell 0
// and cell 41 are open towards -inf and +inf).  Adjacent thresholds are at
// least 0.25 apart, so a cell holds at most one of them; the entry keeps
// how many thresholds lie below the cell and the next threshold at or above
// its lower edge (+inf past the last).  The index is then that count plus
// one exact float32 comparison of w with fl(dd * next), the same comparison
// the definition makes.  The cell itself only needs to be found
// approximately: every threshold other than m_7 = 0 sits at least 0.008
// from a cell edge, and m_7 is the "next" threshold of both cells that meet
// at 0, so a value that falls into a neighbouring cell through rounding of
// w * (8 / dd) still gets the same index.  dd = 0 makes 8 / dd = +inf: a
// nonzero w goes to an end cell, and w = +-0 gives NaN, which the clamp
// sends to cell 0 (index 0, as 0 > -0 is false).
constexpr int kCells = 42;

__device__ __forceinline__ void build_cells(const Codebook& cb, uint2* cells) {
  const int c = threadIdx.x;
  if (c < kCells) {
    const float edge = (float)(c - 21) * 0.125f;
    float next = __builtin_inff();
    uint32_t below = 15u;
#pragma unroll
    for (int k = 14; k >= 0; --k) {
      if (cb.m[k] >= edge) {
        next = cb.m[k];
        below = (uint32_t)k;
      }
    }
    cells[c] = make_uint2(__float_as_uint(next), below);
  }
}

// r8 = 8 / dd (any rounding of it is fine, see above).
__device__ __forceinline__ uint32_t nearest_index(float w, float dd, float r8, const uint2* cells) {
  const float t = fminf(fmaxf(__builtin_fmaf(w, r8, 21.0f), 0.0f), 41.5f);
  const uint2 e = cells[(uint32_t)t];
  return e.y + (w > dd * __uint_as_float(e.x) ? 1u : 0u);
}

// float32 -> fp16 bits of a non-negative value, round to nearest even,
// saturating at 65504 (hardware conversion; kernels run with IEEE rounding
// and fp16 denormals kept).
__device__ __forceinline__ uint32_t f16_sat(float x) { return f32_to_f16_bits(fminf(x, 65504.0f)); }

// clamp(rint(fl(v / dd)), -127, 127) as a byte, 0 when dd = 0, with r =
// rcp(dd).  q = v * r is within 3.1e-5 of fl(v / dd) for |q| <= 128 (rcp
// within 1 ulp, one product rounding, half an ulp of the quotient), so
// rint(q) is the answer unless q lies within 1e-4 of a half-integer; only
// those values take the correctly rounded division.
__device__ __forceinline__ uint32_t q8_code(float v, float dd, float r) {
  const float q = v * r;
  float t = __builtin_rintf(q);
  if (fabsf(fabsf(q - t) - 0.5f) < 1e-4f) t = __builtin_rintf(v / dd);
  t = dd > 0.f ? fminf(fmaxf(t, -127.f), 127.f) : 0.f;
  return (uint32_t)(int32_t)t & 0xffu;
}

}  // namespace tq
