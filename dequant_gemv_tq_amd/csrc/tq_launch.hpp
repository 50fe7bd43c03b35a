// Host launchers of the libtq kernels (one per operation), called by the C
// entry points in tq_api.cpp after argument validation.  Kept apart from the
// device helpers in tq_internal.hpp so that declaring a new launcher leaves
// the kernels' own sources unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// ---------------------------------------------------------------------------
// launchers (each returns hipGetLastError() after its launches)
// ---------------------------------------------------------------------------

hipError_t launch_quantize(const void* W, bool bf16, int64_t N, int64_t K, int64_t ldw, uint32_t mask,
                           uint8_t* packed, uint16_t* scales, hipStream_t s, bool rsf = false);
hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                             uint32_t mask, void* out, bool bf16, int64_t ldo, hipStream_t s);
hipError_t launch_rotate(const void* x, bool xbf16, int64_t M, int64_t K, int64_t ldx, uint32_t mask,
                         void* xr, bool rbf16, int64_t ldr, hipStream_t s);
hipError_t launch_gemv(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                       const void* x, bool xbf16, bool rotated, float* y, hipStream_t s);
hipError_t launch_gemm_valu(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                            const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                       const void* xr, bool xbf16, int64_t ldx, float* y, int64_t ldy, void* ws, hipStream_t s);
size_t gemm_workspace_bytes(int64_t N, int64_t K, int64_t M, bool xbf16);
hipError_t launch_blockfp_quantize(int fmt, const void* W, bool bf16, int64_t N, int64_t K,
                                   uint8_t* codes, uint8_t* bscales, float* tscale, void* workspace,
                                   hipStream_t s, bool rsf = false);
hipError_t launch_blockfp_gemv(int fmt, const uint8_t* codes, const uint8_t* bscales, const float* tscale, int64_t N,
                               int64_t K, int64_t M, const void* x, bool xbf16, int64_t ldx, float* y, int64_t ldy,
                               hipStream_t s);
hipError_t launch_transcode_q8(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t mask,
                               int8_t* codes, uint16_t* qscales, hipStream_t s);
hipError_t launch_q8_gemv(const int8_t* codes, const uint16_t* qscales, int64_t N, int64_t K, const void* x,
                          bool xbf16, float* y, hipStream_t s);
hipError_t launch_blockfp_gemm(int fmt, const uint8_t* codes, const uint8_t* bscales, const float* tscale,
                               int64_t N, int64_t K, int64_t M, const void* x, bool xbf16, int64_t ldx,
                               float* y, int64_t ldy, void* ws, hipStream_t s);

// plain streaming read (tq_measure.hip).
hipError_t launch_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t s);

// turbo4 KV cache (tq_kv.hip).
hipError_t launch_q8_rows(const void* X, bool bf16, int64_t nblocks, int8_t* codes, uint16_t* scales, hipStream_t s);
hipError_t launch_turbo4_encode(const void* V, bool bf16, int64_t nvec, const uint32_t* sign, uint8_t* packed,
                                uint16_t* norms, hipStream_t s);
hipError_t launch_turbo4_decode(const uint8_t* packed, const uint16_t* norms, int64_t nvec, const uint32_t* sign,
                                float* out, hipStream_t s);
size_t attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Tmax);
hipError_t launch_attn_decode(const void* q, bool qbf16, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tmax,
                              const int32_t* lengths, const int8_t* kcodes, const uint16_t* kscales,
                              const uint8_t* vpacked, const uint16_t* vnorms, const uint32_t* sign, float* o,
                              void* workspace, hipStream_t s);
hipError_t launch_attn_decode_noalloc(const void* q, bool qbf16, int64_t B, int64_t Hq, int64_t Hkv, int64_t Tmax,
                                      const int32_t* lengths, const int8_t* kcodes, const uint16_t* kscales,
                                      const uint8_t* vpacked, const uint16_t* vnorms, const uint32_t* sign, float* o,
                                      hipStream_t s);

}  // namespace tq
