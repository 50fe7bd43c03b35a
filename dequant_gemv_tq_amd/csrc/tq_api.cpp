// C ABI of libtq: argument validation and dispatch to the HIP launchers.
// Every check runs before anything is enqueued, so a call that returns an
// error has not touched the stream.
#include <cstdint>

#include "tq_internal.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t dtype_size(tq_dtype t) {
  switch (t) {
    case TQ_F32: return 4;
    case TQ_BF16: return 2;
    case TQ_F16: return 2;
  }
  return 0;
}

bool float_or_bf16(tq_dtype t) { return t == TQ_F32 || t == TQ_BF16; }

tq_status from_hip(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EDEVICE; }

// Common checks for a TQ4_1S weight pair.
tq_status check_weights(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K) {
  if (!packed || !scales) return TQ_EINVAL;
  if (N <= 0 || K <= 0) return TQ_EINVAL;
  if (K % tq::kBlock || K > ((int64_t)1 << 31)) return TQ_ESHAPE;
  if (!aligned(packed, 16) || !aligned(scales, 4)) return TQ_EALIGN;
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument (null pointer, non-positive size, bad flag or format)";
    case TQ_ESHAPE: return "unsupported shape (K not a multiple of the block, or a size limit exceeded)";
    case TQ_EALIGN: return "misaligned pointer or leading dimension";
    case TQ_EDTYPE: return "dtype not accepted by this call";
    case TQ_EDEVICE: return "HIP runtime error at launch";
  }
  return "unknown status";
}

tq_status tq_quantize(const void* W, tq_dtype wt, int64_t N, int64_t K, int64_t ldw, uint32_t sign_mask,
                      uint8_t* packed, uint16_t* scales, hipStream_t stream) {
  if (!W) return TQ_EINVAL;
  if (tq_status st = check_weights(packed, scales, N, K)) return st;
  if (ldw < K) return TQ_EINVAL;
  if (!float_or_bf16(wt)) return TQ_EDTYPE;
  if (!aligned(W, 16) || (ldw * dtype_size(wt)) % 16) return TQ_EALIGN;
  return from_hip(tq::launch_quantize(W, wt == TQ_BF16, N, K, ldw, sign_mask, packed, scales, stream));
}

tq_status tq_quantize_rsf(const void* W, tq_dtype wt, int64_t N, int64_t K, int64_t ldw, uint32_t sign_mask,
                          uint8_t* packed, uint16_t* scales, hipStream_t stream) {
  if (!W) return TQ_EINVAL;
  if (tq_status st = check_weights(packed, scales, N, K)) return st;
  if (ldw < K) return TQ_EINVAL;
  if (!float_or_bf16(wt)) return TQ_EDTYPE;
  if (!aligned(W, 16) || (ldw * dtype_size(wt)) % 16) return TQ_EALIGN;
  return from_hip(tq::launch_quantize(W, wt == TQ_BF16, N, K, ldw, sign_mask, packed, scales, stream, true));
}

tq_status tq_dequantize(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t sign_mask,
                        void* W_out, tq_dtype ot, int64_t ldo, hipStream_t stream) {
  if (!W_out) return TQ_EINVAL;
  if (tq_status st = check_weights(packed, scales, N, K)) return st;
  if (ldo < K) return TQ_EINVAL;
  if (!float_or_bf16(ot)) return TQ_EDTYPE;
  if (!aligned(W_out, 16) || (ldo * dtype_size(ot)) % 16) return TQ_EALIGN;
  return from_hip(tq::launch_dequantize(packed, scales, N, K, sign_mask, W_out, ot == TQ_BF16, ldo, stream));
}

tq_status tq_rotate(const void* x, tq_dtype xt, int64_t M, int64_t K, int64_t ldx, uint32_t sign_mask,
                    void* x_rot, tq_dtype rt, int64_t ldr, hipStream_t stream) {
  if (!x || !x_rot || M <= 0 || K <= 0) return TQ_EINVAL;
  if (K % tq::kBlock) return TQ_ESHAPE;
  if (ldx < K || ldr < K) return TQ_EINVAL;
  if (!float_or_bf16(xt) || !float_or_bf16(rt)) return TQ_EDTYPE;
  if (!aligned(x, 16) || !aligned(x_rot, 16) || (ldx * dtype_size(xt)) % 16 || (ldr * dtype_size(rt)) % 16)
    return TQ_EALIGN;
  return from_hip(tq::launch_rotate(x, xt == TQ_BF16, M, K, ldx, sign_mask, x_rot, rt == TQ_BF16, ldr, stream));
}

tq_status tq_gemv(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t sign_mask,
                  const void* x, tq_dtype xt, int x_is_rotated, float* y, hipStream_t stream) {
  if (!x || !y) return TQ_EINVAL;
  if (tq_status st = check_weights(packed, scales, N, K)) return st;
  if (K > 131072 || N > 0x7fffffff) return TQ_ESHAPE;
  if (!float_or_bf16(xt)) return TQ_EDTYPE;
  if (!aligned(x, 16) || !aligned(y, 4)) return TQ_EALIGN;
  return from_hip(tq::launch_gemv(packed, scales, N, K, sign_mask, x, xt == TQ_BF16, x_is_rotated != 0, y, stream));
}

tq_status tq_gemm(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                  const void* x_rot, tq_dtype xt, int64_t ldx, float* y, int64_t ldy, void* workspace,
                  size_t ws_bytes, hipStream_t stream) {
  if (!x_rot || !y || M <= 0) return TQ_EINVAL;
  if (tq_status st = check_weights(packed, scales, N, K)) return st;
  if (ldx < K || ldy < N) return TQ_EINVAL;
  if (M > 256 || K > 131072 || N > 0x7fffffff) return TQ_ESHAPE;
  if (!float_or_bf16(xt)) return TQ_EDTYPE;
  if (!aligned(x_rot, 16) || (ldx * dtype_size(xt)) % 16 || !aligned(y, 4)) return TQ_EALIGN;
  const size_t need = tq::gemm_workspace_bytes(N, K, M, xt == TQ_BF16);
  if (need && (!workspace || ws_bytes < need)) return TQ_EINVAL;
  if (need && !aligned(workspace, 256)) return TQ_EALIGN;
  return from_hip(tq::launch_gemm(packed, scales, N, K, M, x_rot, xt == TQ_BF16, ldx, y, ldy, workspace, stream));
}

static tq_status blockfp_quantize(tq_format f, const void* W, tq_dtype wt, int64_t N, int64_t K, uint8_t* codes,
                                  uint8_t* block_scales, float* tensor_scale, void* workspace, size_t ws_bytes,
                                  hipStream_t stream, bool rsf) {
  if (f != TQ_FMT_NVFP4 && f != TQ_FMT_MXFP6) return TQ_EINVAL;
  if (!W || !codes || !block_scales || N <= 0 || K <= 0) return TQ_EINVAL;
  if (f == TQ_FMT_NVFP4 && (!tensor_scale || !workspace || ws_bytes < TQ_NVFP4_WORKSPACE_BYTES)) return TQ_EINVAL;
  if (K % (f == TQ_FMT_NVFP4 ? 16 : 32)) return TQ_ESHAPE;
  if (N > 0x7fffffff) return TQ_ESHAPE;
  if (!float_or_bf16(wt)) return TQ_EDTYPE;
  if (!aligned(W, 16) || (K * dtype_size(wt)) % 16 || !aligned(codes, 8)) return TQ_EALIGN;
  if (f == TQ_FMT_NVFP4 && (!aligned(tensor_scale, 4) || !aligned(workspace, 4))) return TQ_EALIGN;
  return from_hip(tq::launch_blockfp_quantize((int)f, W, wt == TQ_BF16, N, K, codes, block_scales, tensor_scale,
                                              workspace, stream, rsf));
}

tq_status tq_blockfp_quantize(tq_format f, const void* W, tq_dtype wt, int64_t N, int64_t K, uint8_t* codes,
                              uint8_t* block_scales, float* tensor_scale, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  return blockfp_quantize(f, W, wt, N, K, codes, block_scales, tensor_scale, workspace, ws_bytes, stream, false);
}

tq_status tq_blockfp_quantize_rsf(tq_format f, const void* W, tq_dtype wt, int64_t N, int64_t K, uint8_t* codes,
                                  uint8_t* block_scales, float* tensor_scale, void* workspace, size_t ws_bytes,
                                  hipStream_t stream) {
  return blockfp_quantize(f, W, wt, N, K, codes, block_scales, tensor_scale, workspace, ws_bytes, stream, true);
}

size_t tq_workspace_bytes(int op, int64_t N, int64_t K, int64_t M) {
  switch (op) {
    case TQ_OP_QUANTIZE: case TQ_OP_DEQUANTIZE: case TQ_OP_ROTATE: case TQ_OP_GEMV:
    case TQ_OP_MXFP6_QUANTIZE: case TQ_OP_TRANSCODE_Q8: case TQ_OP_Q8_GEMV:
      return 0;
    case TQ_OP_GEMM: case TQ_OP_BLOCKFP_GEMM:
      if (N <= 0 || K <= 0 || M <= 0) return SIZE_MAX;
      return tq::gemm_workspace_bytes(N, K, M, true);
    case TQ_OP_NVFP4_QUANTIZE:
      return TQ_NVFP4_WORKSPACE_BYTES;
    case TQ_OP_ATTN_DECODE:
      if (N <= 0 || K <= 0 || M <= 0) return SIZE_MAX;
      return tq::attn_workspace_bytes(N, K, M);
  }
  return SIZE_MAX;
}

tq_status tq_blockfp_gemm(tq_format f, const uint8_t* codes, const uint8_t* block_scales, const float* tensor_scale,
                          int64_t N, int64_t K, int64_t M, const void* x, tq_dtype xt, int64_t ldx, float* y,
                          int64_t ldy, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (f != TQ_FMT_NVFP4 && f != TQ_FMT_MXFP6) return TQ_EINVAL;
  if (!codes || !block_scales || !x || !y || N <= 0 || K <= 0 || M <= 0) return TQ_EINVAL;
  if (f == TQ_FMT_NVFP4 && !tensor_scale) return TQ_EINVAL;
  if (ldx < K || ldy < N) return TQ_EINVAL;
  if (K % 32) return TQ_ESHAPE;
  if (M > 4096 || K > 32768 || N > 0x7fffffff) return TQ_ESHAPE;
  if (!float_or_bf16(xt)) return TQ_EDTYPE;
  if (!aligned(codes, f == TQ_FMT_NVFP4 ? 16 : 8) || !aligned(x, 16) || (ldx * dtype_size(xt)) % 16 || !aligned(y, 4))
    return TQ_EALIGN;
  if (f == TQ_FMT_NVFP4 && (!aligned(block_scales, 2) || !aligned(tensor_scale, 4))) return TQ_EALIGN;
  const size_t need = tq::gemm_workspace_bytes(N, K, M, xt == TQ_BF16);
  if (need && (!workspace || ws_bytes < need)) return TQ_EINVAL;
  if (need && !aligned(workspace, 256)) return TQ_EALIGN;
  return from_hip(tq::launch_blockfp_gemm((int)f, codes, block_scales, tensor_scale, N, K, M, x, xt == TQ_BF16, ldx,
                                          y, ldy, workspace, stream));
}

tq_status tq_transcode_q8(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, uint32_t sign_mask,
                          int8_t* codes, uint16_t* q8_scales, hipStream_t stream) {
  if (!codes || !q8_scales) return TQ_EINVAL;
  if (tq_status st = check_weights(packed, scales, N, K)) return st;
  if (!aligned(codes, 16) || !aligned(q8_scales, 2)) return TQ_EALIGN;
  return from_hip(tq::launch_transcode_q8(packed, scales, N, K, sign_mask, codes, q8_scales, stream));
}

tq_status tq_q8_gemv(const int8_t* codes, const uint16_t* q8_scales, int64_t N, int64_t K, const void* x,
                     tq_dtype xt, float* y, hipStream_t stream) {
  if (!codes || !q8_scales || !x || !y || N <= 0 || K <= 0) return TQ_EINVAL;
  if (K % tq::kBlock) return TQ_ESHAPE;
  if (K > 32768 || N > 0x7fffffff) return TQ_ESHAPE;
  if (!float_or_bf16(xt)) return TQ_EDTYPE;
  if (!aligned(codes, 16) || !aligned(q8_scales, 2) || !aligned(x, 16) || !aligned(y, 4)) return TQ_EALIGN;
  return from_hip(tq::launch_q8_gemv(codes, q8_scales, N, K, x, xt == TQ_BF16, y, stream));
}

tq_status tq_kv_quantize_k(const void* K, tq_dtype kt, int64_t n, int64_t d, int8_t* codes, uint16_t* scales,
                           hipStream_t stream) {
  if (!K || !codes || !scales || n <= 0 || d <= 0) return TQ_EINVAL;
  if (d % tq::kBlock) return TQ_ESHAPE;
  if (!float_or_bf16(kt)) return TQ_EDTYPE;
  if (!aligned(K, 16) || !aligned(codes, 16) || !aligned(scales, 2)) return TQ_EALIGN;
  return from_hip(tq::launch_q8_rows(K, kt == TQ_BF16, n * (d / tq::kBlock), codes, scales, stream));
}

tq_status tq_kv_quantize_v(const void* V, tq_dtype vt, int64_t n, int64_t d, const uint32_t sign[4],
                           uint8_t* packed, uint16_t* norms, hipStream_t stream) {
  if (!V || !sign || !packed || !norms || n <= 0 || d <= 0) return TQ_EINVAL;
  if (d != 128) return TQ_ESHAPE;
  if (!float_or_bf16(vt)) return TQ_EDTYPE;
  if (!aligned(V, 16) || !aligned(packed, 8) || !aligned(norms, 2)) return TQ_EALIGN;
  return from_hip(tq::launch_turbo4_encode(V, vt == TQ_BF16, n, sign, packed, norms, stream));
}

tq_status tq_kv_dequantize_v(const uint8_t* packed, const uint16_t* norms, int64_t n, int64_t d,
                             const uint32_t sign[4], float* out, hipStream_t stream) {
  if (!packed || !norms || !sign || !out || n <= 0 || d <= 0) return TQ_EINVAL;
  if (d != 128) return TQ_ESHAPE;
  if (!aligned(packed, 8) || !aligned(norms, 2) || !aligned(out, 16)) return TQ_EALIGN;
  return from_hip(tq::launch_turbo4_decode(packed, norms, n, sign, out, stream));
}

size_t tq_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t T_max) {
  if (B <= 0 || Hq <= 0 || T_max <= 0) return 0;
  return tq::attn_workspace_bytes(B, Hq, T_max);
}

tq_status tq_attn_decode(const void* q, tq_dtype qt, int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t T_max,
                         const int32_t* lengths, const int8_t* k_codes, const uint16_t* k_scales,
                         const uint8_t* v_packed, const uint16_t* v_norms, const uint32_t sign[4], float* o,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q || !lengths || !k_codes || !k_scales || !v_packed || !v_norms || !sign || !o || !workspace)
    return TQ_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || T_max <= 0) return TQ_EINVAL;
  if (d != 128 || Hq % Hkv) return TQ_ESHAPE;
  const int64_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ESHAPE;
  if (B > 65535 || Hkv > 65535 || Hq > 65535 || T_max > (int64_t)INT32_MAX) return TQ_ESHAPE;
  if (ws_bytes < tq::attn_workspace_bytes(B, Hq, T_max)) return TQ_EINVAL;
  if (!float_or_bf16(qt)) return TQ_EDTYPE;
  if (!aligned(q, 16) || !aligned(lengths, 4) || !aligned(k_codes, 16) || !aligned(k_scales, 2) ||
      !aligned(v_packed, 4) || !aligned(v_norms, 2) || !aligned(o, 4) || !aligned(workspace, 4))
    return TQ_EALIGN;
  return from_hip(tq::launch_attn_decode(q, qt == TQ_BF16, B, Hq, Hkv, T_max, lengths, k_codes, k_scales, v_packed,
                                         v_norms, sign, o, workspace, stream));
}

tq_status tq_attn_decode_noalloc(const void* q, tq_dtype qt, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                 int64_t T_max, const int32_t* lengths, const int8_t* k_codes,
                                 const uint16_t* k_scales, const uint8_t* v_packed, const uint16_t* v_norms,
                                 const uint32_t sign[4], float* o, hipStream_t stream) {
  if (!q || !lengths || !k_codes || !k_scales || !v_packed || !v_norms || !sign || !o) return TQ_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || T_max <= 0) return TQ_EINVAL;
  if (d != 128 || Hq % Hkv) return TQ_ESHAPE;
  const int64_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TQ_ESHAPE;
  if (B > 65535 || Hkv > 65535 || Hq > 65535 || T_max > (int64_t)INT32_MAX) return TQ_ESHAPE;
  if (tq::attn_workspace_bytes(B, Hq, T_max) > (size_t)TQ_ATTN_NOALLOC_SCRATCH_BYTES) return TQ_ESHAPE;
  if (!float_or_bf16(qt)) return TQ_EDTYPE;
  if (!aligned(q, 16) || !aligned(lengths, 4) || !aligned(k_codes, 16) || !aligned(k_scales, 2) ||
      !aligned(v_packed, 4) || !aligned(v_norms, 2) || !aligned(o, 4))
    return TQ_EALIGN;
  return from_hip(tq::launch_attn_decode_noalloc(q, qt == TQ_BF16, B, Hq, Hkv, T_max, lengths, k_codes, k_scales,
                                                 v_packed, v_norms, sign, o, stream));
}

tq_status tq_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!p || !sink || bytes == 0) return TQ_EINVAL;
  if (bytes % 16) return TQ_ESHAPE;
  if (!aligned(p, 16) || !aligned(sink, 4)) return TQ_EALIGN;
  return from_hip(tq::launch_stream_read(p, bytes, sink, stream));
}

}  // extern "C"
