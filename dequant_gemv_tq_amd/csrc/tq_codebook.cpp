// Host-side constants: the 16-level Lloyd-Max codebook for N(0,1) and the
// splitmix64 sign mask.
//
// TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160), "格式原理"
// item 2 and the paragraph after the list: rotated coordinates are quantized
// one by one to the nearest optimal N(0,1) centroid; the codebook comes from
// Lloyd's algorithm.  The normal law is symmetric, so the fixed point is
// symmetric and only the 8 positive centroids are iterated: the innermost
// positive cell starts at the boundary 0, every other boundary is the
// midpoint of its neighbours, and each centroid moves to the conditional
// mean of its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
#include <cmath>
#include <mutex>

#include "tq_internal.hpp"

namespace tq {
namespace {

double normal_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) * 0.39894228040143267794;   // 1/sqrt(2 pi)
}

// Upper-tail probability Q(x) = P(X > x) = erfc(x / sqrt 2) / 2, accurate for x >= 0.
double upper_tail(double x) { return 0.5 * std::erfc(x * 0.70710678118654752440); }

Codebook build_codebook() {
  constexpr int kPos = 8;
  double c[kPos];
  for (int k = 0; k < kPos; ++k) c[k] = 0.25 + 0.3 * k;      // any increasing positive start
  for (int it = 0; it < 1000000; ++it) {
    double lo[kPos], hi[kPos];
    for (int k = 0; k < kPos; ++k) {
      lo[k] = (k == 0) ? 0.0 : 0.5 * (c[k - 1] + c[k]);
      hi[k] = (k == kPos - 1) ? INFINITY : 0.5 * (c[k] + c[k + 1]);
    }
    double change = 0.0;
    for (int k = 0; k < kPos; ++k) {
      double mass = upper_tail(lo[k]) - upper_tail(hi[k]);
      double nc = (normal_pdf(lo[k]) - normal_pdf(hi[k])) / mass;
      change = std::fmax(change, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (change < 1e-15) break;
  }
  Codebook cb;
  for (int k = 0; k < kPos; ++k) {
    float f = (float)c[k];
    cb.c[8 + k] = f;
    cb.c[7 - k] = -f;
  }
  for (int k = 0; k < 15; ++k) cb.m[k] = (float)(((double)cb.c[k] + (double)cb.c[k + 1]) * 0.5);
  return cb;
}

}  // namespace

const Codebook& host_codebook() {
  static std::once_flag once;
  static Codebook cb;
  std::call_once(once, [] { cb = build_codebook(); });
  return cb;
}

int device_cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace tq

extern "C" tq_status tq_codebook(float centroids[16], float thresholds[15]) {
  const tq::Codebook& cb = tq::host_codebook();
  if (centroids)
    for (int k = 0; k < 16; ++k) centroids[k] = cb.c[k];
  if (thresholds)
    for (int k = 0; k < 15; ++k) thresholds[k] = cb.m[k];
  return TQ_OK;
}

extern "C" uint32_t tq_sign_mask_from_seed(uint64_t seed) {
  // splitmix64 (Steele, Lea and Flood, 2014): one step of the state by the
  // 64-bit golden-ratio increment, then the variant-13 finalizer.
  uint64_t z = seed + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (uint32_t)z;
}

extern "C" uint32_t tq_default_sign_mask(void) { return tq_sign_mask_from_seed(0); }
