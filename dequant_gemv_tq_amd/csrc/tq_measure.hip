// Plain streaming read on gfx950: the read envelope the decode kernels are
// compared with.  TQ4 page ("企业官网建设流程全解析", hotelren.com/news/5458160),
// decode-speed section: batch-1 decode is bound by memory bandwidth, and how
// close a backend's kernel gets to it decides the speed, so the bytes a GEMV
// launch moves are also timed through a kernel that only reads them.
//
// A persistent grid of 1024-thread workgroups (one per compute unit, the
// GEMV's shape) walks the buffer with consecutive threads on consecutive 16
// bytes and two loads in flight per thread (more in flight measured slower
// on MI355X: 1 GiB at 6.2 TB/s with two, 5.9 with four, 5.8 with eight).
// The words are folded with XOR and each wavefront stores its fold, so the
// loads cannot be dropped and the output is 4 bytes per wavefront.
#include "tq_internal.hpp"

namespace tq {
namespace {

constexpr int kReadThreads = 1024;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ p, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + stride < n16; i += 2 * stride) {
    const uint4 a = p[i], b = p[i + stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
  }
  if (i < n16) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // One fold per wavefront, no workgroup barrier (a barrier would make the
  // measurement wait for the slowest wavefront of every workgroup).
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, s, 64);
  if ((threadIdx.x & 63) == 0) sink[(size_t)blockIdx.x * (kReadThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t want = (n16 + kReadThreads - 1) / kReadThreads;
  size_t grid = (size_t)device_cu_count();
  const size_t max_grid = TQ_STREAM_READ_SINK_WORDS / (kReadThreads / 64);
  grid = grid < max_grid ? grid : max_grid;
  grid = want < grid ? want : grid;
  hipLaunchKernelGGL(stream_read_kernel, dim3((uint32_t)grid), dim3(kReadThreads), 0, s,
                     static_cast<const uint4*>(p), n16, sink);
  return hipGetLastError();
}

}  // namespace tq
