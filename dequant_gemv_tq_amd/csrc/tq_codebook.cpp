// Host-side constants: the 16-level Lloyd-Max codebook for N(0,1) with its
// 15 decision thresholds, and the splitmix64 sign mask.
//
// TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160), "格式原理"
// item 2 and the paragraph after the list: rotated coordinates are quantized
// one by one to the nearest optimal N(0,1) centroid; the codebook comes from
// Lloyd's algorithm.  The centroids are the float32 constants of
// tq_internal.hpp; a threshold is the midpoint of two neighbouring float32
// centroids, formed in float64 and rounded once to float32.
#include <mutex>

#include "tq_internal.hpp"

namespace tq {
namespace {

Codebook build_codebook() {
  Codebook cb;
  for (int k = 0; k < 16; ++k) cb.c[k] = centroid(k);
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

extern "C" tq_status tq_kv_sign_from_seed(uint64_t seed, uint32_t out[4]) {
  if (!out) return TQ_EINVAL;
  // The first two splitmix64 outputs: bits 0..63, then 64..127.
  uint64_t state = seed;
  for (int k = 0; k < 2; ++k) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    out[2 * k] = (uint32_t)z;
    out[2 * k + 1] = (uint32_t)(z >> 32);
  }
  return TQ_OK;
}
