/*
 * tq.h -- C ABI of libtq: TQ4_1S block quantization and fused
 * dequantize-times-activation GEMV/GEMM on AMD Instinct MI355X (gfx950),
 * plus NVFP4 / MXFP6 block formats.
 *
 * Sources (five web pages; cited by title and section):
 *   TQ4 page  -- "企业官网建设流程全解析" (hotelren.com/news/5458160), a
 *                summary of community results for TQ4_1S weight compression.
 *                Section "TQ4_1S 是什么", sub-list "格式原理" items 1-3 and the
 *                paragraph after it define the encoding; the decode-speed
 *                section ("解码速度：分硬件汇总", paragraph on why CUDA differs)
 *                describes rotating the activation once so that
 *                dequantization becomes a centroid lookup times a scale;
 *                "适用前提与边界" notes that the attention tensors of a layer
 *                share one in-place rotation.
 *   Quantizer-tool page -- "这是我的 llama.cpp NVFP4/MXFP6 GGUF 量化工具"
 *                (bittide.aicompass.dev): NVFP4 weight and tensor scales,
 *                MXFP6 ("目前能实现的部分功能", "MXFP6 的未来").
 *
 * Conventions for every call below
 *   - W is [N, K] row-major and y = W x; K is split into blocks of 32
 *     contiguous elements (16 for NVFP4).
 *   - Buffer pointers are DEVICE pointers unless marked [host].  The caller
 *     allocates and frees every buffer; the library never allocates device
 *     memory and keeps no state other than its host-side constant tables,
 *     built once on first use (thread-safe).
 *   - Inputs are never modified.  Outputs must not alias inputs.
 *   - All work is enqueued asynchronously on `stream` (NULL = the null
 *     stream); a call returns once its kernels are launched.
 *   - Arguments are validated before anything is launched; on any error
 *     nothing is enqueued.  TQ_EDEVICE reports a failed launch.
 *   - NaN or Inf inputs give unspecified (but memory-safe) outputs.
 *
 * TQ4_1S storage (one 32-element block of row n, block b):
 *   packed[n][16b .. 16b+15]   (uint8, K/2 bytes per row): byte j of the
 *                              block holds element 2j in its low nibble and
 *                              element 2j+1 in its high nibble; a nibble is
 *                              the index (0 = most negative) of one of the
 *                              16 Lloyd-Max centroids of N(0,1).
 *   scales[n][2b], [2b+1]      (fp16 bits, K/16 per row): d0 for elements
 *                              0-15 and d1 for elements 16-31 of the block.
 *   5.0 bits per weight.
 * Rotation: w' = (1/sqrt 32) * H32 * D * w per block, H32 the Sylvester
 * Hadamard matrix in natural order and D = diag(+-1) with D_i = -1 when bit
 * i of `sign_mask` is set.  The same mask must be used for the weights and
 * the activations they multiply.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 3

typedef enum tq_status {
  TQ_OK = 0,
  TQ_EINVAL = 1,      /* null pointer, non-positive size, bad flag or format   */
  TQ_ESHAPE = 2,      /* K not a multiple of the block, size beyond a limit    */
  TQ_EALIGN = 3,      /* a pointer or leading dimension breaks an alignment rule */
  TQ_EDTYPE = 4,      /* dtype not accepted by this call                         */
  TQ_EDEVICE = 5      /* the HIP runtime reported an error at launch             */
} tq_status;

typedef enum tq_dtype { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;

typedef enum tq_format { TQ_FMT_NVFP4 = 1, TQ_FMT_MXFP6 = 2 } tq_format;

/* Version of this ABI (TQ_ABI_VERSION). */
int tq_abi_version(void);

/* Static English text for a status code. */
const char* tq_status_str(int status);

/* [host] The 16 centroids (ascending) of the 16-level Lloyd-Max quantizer of
 * N(0,1) and the 15 decision thresholds m_k = float32((c_k + c_{k+1}) / 2),
 * as the kernels use them (TQ4 page, "格式原理" item 2 and the paragraph after
 * it: Lloyd's algorithm on the rotated-coordinate law).  The centroids are
 * the fixed point of Lloyd's iteration computed in double precision and
 * rounded once to float32; the library ships these float32 constants (the
 * kernels use them as immediates) and forms the thresholds from them.
 * Either pointer may be NULL.  Returns TQ_OK. */
tq_status tq_codebook(float centroids[16], float thresholds[15]);

/* [host] Sign mask from a seed: low 32 bits of the first splitmix64 output
 * (state advanced by the 64-bit golden-ratio constant 0x9E3779B97F4A7C15).
 * This is the reading taken of the TQ4 page's "golden-ratio sign flips"
 * ("格式原理" item 1). */
uint32_t tq_sign_mask_from_seed(uint64_t seed);

/* [host] tq_sign_mask_from_seed(0) = 0x7B1DCDAF, the default mask. */
uint32_t tq_default_sign_mask(void);

/* Quantize W to TQ4_1S (TQ4 page, "格式原理" items 1-3).
 *   W       [N, K] with row stride `ldw` elements; dtype `wt` = TQ_F32 or
 *           TQ_BF16.  16-byte aligned; ldw * sizeof(wt) a multiple of 16.
 *   packed  [N, K/2] uint8, 16-byte aligned (output).
 *   scales  [N, K/16] fp16 bits, 4-byte aligned (output).
 * Per block and half h: d_h = fp16(RMS of the 16 rotated values), rounded to
 * nearest even and saturated at 65504; index = number of thresholds
 * float32(d_h * m_k) the rotated value exceeds.  The float32 operation order
 * is fixed (see the oracle), so the output is bit-reproducible.
 * Errors: TQ_EINVAL (null, N or K <= 0, ldw < K), TQ_ESHAPE (K % 32, K > 2^31),
 * TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_quantize(const void* W, tq_dtype wt, int64_t N, int64_t K, int64_t ldw,
                      uint32_t sign_mask, uint8_t* packed, uint16_t* scales,
                      hipStream_t stream);

/* tq_quantize with the RSF-lite scale search (quantizer-tool page, "RSF":
 * refined scale fitting searches nearby multiples of a scale and keeps the
 * better lattice fit; here without importance weights).  For each half
 * block, candidates fp16(d * (1 + j/16)), j = -4..4, with d the plain scale,
 * re-choose the indices with the same rule and are scored by the float32
 * squared error of fl(d_j * c[idx]) against the rotated values (pairwise sum
 * in index order); the smallest wins, ties to the multiplier nearest 1.  The
 * output is ordinary TQ4_1S (same layout, every other call reads it) and
 * bit-exact against that definition.  Arguments, alignment and errors as
 * tq_quantize; about six times its arithmetic. */
tq_status tq_quantize_rsf(const void* W, tq_dtype wt, int64_t N, int64_t K, int64_t ldw,
                          uint32_t sign_mask, uint8_t* packed, uint16_t* scales, hipStream_t stream);

/* Dequantize TQ4_1S back to the original (unrotated) domain: per block
 * W_out = (1/sqrt 32) * D * H32 * (d_h * c[index]) (TQ4 page, paragraph after
 * "格式原理": the reference dequantizes by inverse rotation and rescaling).
 *   W_out   [N, K] with row stride `ldo`; `ot` = TQ_F32 or TQ_BF16 (RNE);
 *           16-byte aligned, ldo * sizeof(ot) a multiple of 16.
 * Errors as tq_quantize. */
tq_status tq_dequantize(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                        uint32_t sign_mask, void* W_out, tq_dtype ot, int64_t ldo,
                        hipStream_t stream);

/* Pre-rotate activations once: x_rot = (1/sqrt 32) * H32 * D * x per
 * 32-block (TQ4 page, decode-speed section: rotate the activation instead of
 * inverse-rotating every weight block).  The float32 order is the same
 * butterfly order as tq_quantize.
 *   x       [M, K], row stride ldx; `xt` = TQ_F32 or TQ_BF16; 16-byte aligned.
 *   x_rot   [M, K], row stride ldr; `rt` = TQ_F32 or TQ_BF16 (RNE).
 * Errors: TQ_EINVAL, TQ_ESHAPE (K % 32), TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_rotate(const void* x, tq_dtype xt, int64_t M, int64_t K, int64_t ldx,
                    uint32_t sign_mask, void* x_rot, tq_dtype rt, int64_t ldr,
                    hipStream_t stream);

/* Fused batch-1 GEMV y = W_deq x on TQ4_1S weights, computed in the rotated
 * domain: y_n = sum_b [ d0 * sum_{i<16} c[idx_i] x'_i + d1 * sum_{i>=16} ... ]
 * with float32 accumulation (TQ4 page, decode-speed section).
 *   x            [K]; if x_is_rotated != 0 it is x' from tq_rotate (TQ_F32,
 *                or TQ_BF16 as tq_rotate rounds it: the product is then
 *                exact for that rounded x'); otherwise it is the raw
 *                activation (TQ_F32 or TQ_BF16) and the kernel rotates it
 *                itself (sign_mask used; the +-1 products are exact and only
 *                the float32 sums of the rotation round, whether they run as
 *                butterflies or, for a bf16 x with K in (10240, 32768], on
 *                the matrix cores).
 *   y            [N] float32 (output).
 * Limits: K <= 131072.  Errors: TQ_EINVAL, TQ_ESHAPE, TQ_EALIGN (x 16-byte
 * aligned, y 4-byte aligned), TQ_EDTYPE. */
tq_status tq_gemv(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                  uint32_t sign_mask, const void* x, tq_dtype xt, int x_is_rotated,
                  float* y, hipStream_t stream);

/* Small-batch fused GEMM Y = X' Q^T with Q = d * c[idx] in the rotated
 * domain (the same identity as tq_gemv, M activations at once).
 *   x_rot   [M, K] pre-rotated activations (tq_rotate), row stride ldx,
 *           TQ_BF16 or TQ_F32, 16-byte aligned.
 *   y       [M, N] float32, row stride ldy (output).
 * M <= 2 (and float32 activations with M < 16) run a VALU kernel with
 * float32 FMAs.  Larger M runs bf16 MFMA in 16-row tiles with float32
 * accumulation, dequantizing each weight once: one pass for bf16
 * activations, three hi/lo-split passes for float32 activations.
 * Precision of the MFMA path: the products are formed in the rotated domain,
 * so what is guaranteed is a bound on sum_k |q_k x'_k| (q = d * c[idx]):
 * per product at most 2^-7 + 2^-10 of |q x'| with bf16 x' (x' rounds by up
 * to 2^-8; the weight, the fp16-rounded centroid times the scale rounded
 * once to bf16, by up to 2^-8 + 2^-11), at most 2^-13 with float32 x' (hi/lo
 * split without the lo*lo term), plus float32 accumulation over K.  The
 * original-domain bound 1e-3 * sum_k |W_deq[n,k] x_k| is only statistical:
 * it holds for dense activations (bf16 once K is in the hundreds, float32 at
 * any K) but not for one-hot or very sparse rows, whose 32 rotated products
 * per block cancel down to a single weight.  Callers with such activations
 * who need that bound pass float32 x' in launches of at most 15 rows, which
 * run float32 FMAs.
 * Workspace (bf16 activations, M >= 3): the MFMA kernel splits K into
 * several ranges when K is long (more than 4096 elements for launches of up
 * to 16 rows, 2048 for 17-64; M is launched 64 rows at a time) or when N
 * has few 16-row tiles per compute unit.  Each range's sums then go to the
 * workspace, and the last workgroup to finish a tile adds the ranges in
 * their fixed order, so y is the same on every run.  `workspace` is device
 * memory of at least tq_workspace_bytes(TQ_OP_GEMM, N, K, M) bytes,
 * 256-byte aligned, zero-filled before the first call that uses it; every
 * call leaves it fit for the next one.  Calls that share a workspace must
 * not run at the same time (one stream, or ordered streams).  When that
 * size is 0 the workspace may be NULL.
 * Limits: M <= 256, K <= 131072.  Errors: TQ_EINVAL (also: a workspace
 * missing or smaller than needed), TQ_ESHAPE, TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_gemm(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K, int64_t M,
                  const void* x_rot, tq_dtype xt, int64_t ldx, float* y, int64_t ldy,
                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of NVFP4 quantization: the amax pass leaves one partial
 * maximum per workgroup (at most 1024) for the encode pass. */
#define TQ_NVFP4_WORKSPACE_BYTES 4096

/* Operations for tq_workspace_bytes. */
typedef enum tq_op {
  TQ_OP_QUANTIZE = 1,          /* tq_quantize, tq_quantize_rsf: none            */
  TQ_OP_DEQUANTIZE = 2,        /* none                                          */
  TQ_OP_ROTATE = 3,            /* none                                          */
  TQ_OP_GEMV = 4,              /* none                                          */
  TQ_OP_GEMM = 5,              /* split-K sums and per-tile counters            */
  TQ_OP_NVFP4_QUANTIZE = 6,    /* tq_blockfp_quantize(_rsf) with TQ_FMT_NVFP4   */
  TQ_OP_MXFP6_QUANTIZE = 7,    /* tq_blockfp_quantize(_rsf) with TQ_FMT_MXFP6: none */
  TQ_OP_BLOCKFP_GEMM = 8,      /* as TQ_OP_GEMM                                 */
  TQ_OP_TRANSCODE_Q8 = 9,      /* none                                          */
  TQ_OP_Q8_GEMV = 10,          /* none                                          */
  TQ_OP_ATTN_DECODE = 11       /* N = B, K = Hq, M = T_max: as tq_attn_workspace_bytes */
} tq_op;

/* Device workspace bytes a call of `op` needs for an [N, K] weight and M
 * activation rows (TQ_OP_ATTN_DECODE: N = sequences, K = query heads, M =
 * T_max).  0 when the call takes no workspace; SIZE_MAX for an unknown op
 * or a non-positive size where one is used.  The caller allocates the
 * workspace (the library allocates nothing) and owns it again once the
 * stream has passed the call. */
size_t tq_workspace_bytes(int op, int64_t N, int64_t K, int64_t M);

/* Quantize W [N, K] (TQ_F32 or TQ_BF16, dense rows) to a block float format
 * (quantizer-tool page, "目前能实现的部分功能" / "MXFP6 的未来"):
 *   TQ_FMT_NVFP4: codes [N, K/2] (E2M1, element 2j in the low nibble of byte
 *     j), block_scales [N, K/16] (E4M3fn), *tensor_scale = amax|W| / 2688
 *     (one float32, device memory).  K % 16 == 0.  Two launches: an amax
 *     pass that leaves partial maxima in `workspace` (device, 4-byte
 *     aligned, ws_bytes >= tq_workspace_bytes(TQ_OP_NVFP4_QUANTIZE, N, K, 0)
 *     = TQ_NVFP4_WORKSPACE_BYTES; no initial contents needed), then the
 *     encode, which reduces them and writes the tensor scale.
 *   TQ_FMT_MXFP6: codes [N, 3K/4] (E3M2, 4 codes per little-endian 24-bit
 *     word), block_scales [N, K/32] (E8M0); tensor_scale and workspace
 *     ignored (may be NULL).  K % 32 == 0.  One launch.
 * Rounding is to nearest even with saturation; the sign of a value that
 * rounds to zero is kept.  W 16-byte aligned, codes 8-byte aligned.
 * Errors: TQ_EINVAL (also: NVFP4 without tensor_scale or workspace, or a
 * workspace smaller than needed), TQ_ESHAPE, TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_blockfp_quantize(tq_format f, const void* W, tq_dtype wt, int64_t N, int64_t K,
                              uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                              void* workspace, size_t ws_bytes, hipStream_t stream);

/* tq_blockfp_quantize with the RSF-lite block-scale search (quantizer-tool
 * page, "RSF": nearby multiples of a block scale are tried and the better
 * lattice fit kept; here without importance weights).
 *   TQ_FMT_NVFP4: per 16-element block, the E4M3 roundings of
 *     dec(sb) * (1 + j/16), j = 0, -1, +1, ..., -4, +4 (sb the plain scale);
 *     each re-encodes the block with the plain rule and is scored by the
 *     float32 squared error of fl(e2m1 * eff) against w (pairwise sum in
 *     index order).  The tensor scale is the plain one.
 *   TQ_FMT_MXFP6: per 32-element block, exponents e, e - 1, e + 1 (clamped
 *     to [-127, 127]) of the plain E8M0 scale, scored the same way over the
 *     32 elements.
 * The smallest error wins, ties to the earlier candidate (the plain scale
 * first), so the result is never worse than tq_blockfp_quantize's and is
 * bit-exact against that definition.  Output layout, arguments (the
 * workspace included), alignment and errors as tq_blockfp_quantize. */
tq_status tq_blockfp_quantize_rsf(tq_format f, const void* W, tq_dtype wt, int64_t N, int64_t K,
                                  uint8_t* codes, uint8_t* block_scales, float* tensor_scale,
                                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* Y[m, n] = sum_k W_deq[n, k] X[m, k] for a block-float weight (fused
 * decode, float32 accumulation; the activation is used as given, there is
 * no rotation).  Codes are decoded by gfx950's scaled-convert instructions.
 *   M <= 2, or float32 X (any M): VALU kernel.  E2M1 two at a time, E3M2 a
 *     whole 32-element block at a time, scale 1, exact; each 16- (NVFP4) or
 *     32-element (MXFP6) partial sum is multiplied once by its scale:
 *     float32(e4m3 * tensor_scale) for NVFP4, 2^(e8m0 - 127) (ldexp,
 *     exact) for MXFP6.
 *   M >= 3 with bf16 X: bf16 MFMA in 16-row tiles (up to 64 rows per
 *     launch), every weight converted once to an exact bf16 operand
 *     (e2m1 * e4m3 for NVFP4, the tensor scale applied to the finished sums;
 *     e3m2 * 2^(e8m0 - 127) for MXFP6), float32 accumulation.  Long K or
 *     few row tiles: K split into ranges through the workspace, with the
 *     contract of tq_gemm's (tq_workspace_bytes(TQ_OP_BLOCKFP_GEMM, N, K,
 *     M) bytes, 256-byte aligned, zero-filled before first use; the result
 *     does not vary by run).
 * X [M, K] row stride ldx, TQ_F32 or TQ_BF16, 16-byte aligned; Y [M, N]
 * float32, row stride ldy.  K % 32 == 0, K <= 32768, M <= 4096; NVFP4 codes
 * 16-byte aligned (MXFP6 codes 8-byte), NVFP4 block_scales 2-byte aligned.
 * Errors: TQ_EINVAL (also: a workspace missing or smaller than needed),
 * TQ_ESHAPE, TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_blockfp_gemm(tq_format f, const uint8_t* codes, const uint8_t* block_scales,
                          const float* tensor_scale, int64_t N, int64_t K, int64_t M,
                          const void* x, tq_dtype xt, int64_t ldx, float* y, int64_t ldy,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/* Load-time transcode of TQ4_1S weights to int8 blocks (TQ4 page, the note
 * under the decode-speed summary and the backend item of "适用前提与边界":
 * converting TQ4_1S to q8_0 when the model is loaded keeps the TQ4_1S file
 * size and decodes at the q8_0 path's speed).  Per 32-element block, in
 * float32: q_i = d_h * c[idx_i]; u = FWHT32(q); w_i = D_i * u_i / sqrt(32);
 * d = fp16(amax|w| / 127) (round to nearest even, saturating);
 * codes_i = clamp(rint(w_i / d), -127, 127) (ties to even; d = 0 -> 0).
 *   codes      [N, K] int8 row-major, 16-byte aligned (output).
 *   q8_scales  [N, K/32] fp16 bits, one per block, 2-byte aligned (output).
 * 1.0625 bytes per weight; the codes are bit-exact against the canonical
 * order above.  K % 32 == 0.  Errors: TQ_EINVAL, TQ_ESHAPE, TQ_EALIGN. */
tq_status tq_transcode_q8(const uint8_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                          uint32_t sign_mask, int8_t* codes, uint16_t* q8_scales,
                          hipStream_t stream);

/* Batch-1 GEMV on transcoded int8 weights: the activation x [K] (TQ_F32 or
 * TQ_BF16, not rotated, 16-byte aligned) is quantized per 32-element block
 * the same way (dx = amax|x| / 127 in float32, codes rint(x / dx)), and
 * y_n = sum_b d[n, b] dx[b] sum_i codes[n, b, i] xq[b, i] with exact integer
 * block sums (v_dot4_i32_i8) and float32 accumulation.
 *   y  [N] float32, 4-byte aligned (output).
 * K % 32 == 0, K <= 32768.  Errors: TQ_EINVAL, TQ_ESHAPE, TQ_EALIGN,
 * TQ_EDTYPE. */
tq_status tq_q8_gemv(const int8_t* codes, const uint16_t* q8_scales, int64_t N, int64_t K,
                     const void* x, tq_dtype xt, float* y, hipStream_t stream);

/* ------------------------------------------------------------------------
 * turbo4 KV cache: q8_0 keys, PolarQuant values, decode attention (TQ4
 * page: the paragraph after the "格式原理" list, on the reference code's
 * PolarQuant steps -- norm, structured rotation of random signs and a
 * Hadamard transform, nearest-centroid index, inverse rotation and rescale;
 * "叠加压缩：权重 + KV 缓存", where asymmetric q8_0-K / turbo4-V is the best
 * cache configuration).  Head dimension 128.
 * ------------------------------------------------------------------------ */

/* [host] The 128 rotation sign bits for a seed: out[w] holds bits 32 w ..
 * 32 w + 31; bits 0..63 are the first splitmix64 output, 64..127 the
 * second.  Bit i set flips element i.  Errors: TQ_EINVAL (out NULL). */
tq_status tq_kv_sign_from_seed(uint64_t seed, uint32_t out[4]);

/* Keys to q8_0: rows K [n, d] (TQ_F32 or TQ_BF16, dense, 16-byte aligned),
 * per 32-element block scale = fp16(amax / 127) (RNE, saturating), code =
 * clamp(rint(k / scale), -127, 127) (ties to even).
 *   codes  int8 [n, d], 16-byte aligned (output).
 *   scales fp16 bits [n, d/32], 2-byte aligned (output).
 * Errors: TQ_EINVAL, TQ_ESHAPE (d % 32), TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_kv_quantize_k(const void* K, tq_dtype kt, int64_t n, int64_t d, int8_t* codes,
                           uint16_t* scales, hipStream_t stream);

/* Values to turbo4: rows V [n, 128] (TQ_F32 or TQ_BF16, 16-byte aligned).
 * Per vector, float32 in this order: n16 = fp16(sqrt(pairwise sum of
 * squares)); u = FWHT_128(D v) (unnormalised, stages 1..64); index_i =
 * number of thresholds fl(nn * m_k) below u_i (m_k the codebook midpoints).
 *   sign   [host] 4 words from tq_kv_sign_from_seed (the caller's choice).
 *   packed uint8 [n, 64] (element 2j in the low nibble of byte j), 8-byte
 *          aligned (output);  norms fp16 bits [n], 2-byte aligned (output).
 * Bit-exact against that definition.  4.125 bits per element.
 * Errors: TQ_EINVAL, TQ_ESHAPE (d != 128), TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_kv_quantize_v(const void* V, tq_dtype vt, int64_t n, int64_t d, const uint32_t sign[4],
                           uint8_t* packed, uint16_t* norms, hipStream_t stream);

/* turbo4 values back to float32: out [n, 128] = (nn / 128) D H c[index]
 * (16-byte aligned).  Errors as tq_kv_quantize_v. */
tq_status tq_kv_dequantize_v(const uint8_t* packed, const uint16_t* norms, int64_t n, int64_t d,
                             const uint32_t sign[4], float* out, hipStream_t stream);

/* Bytes of workspace tq_attn_decode needs: B * Hq * ceil(T_max / 256) *
 * 130 floats (0 for non-positive arguments). */
size_t tq_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t T_max);

/* Decode attention for one new token per sequence over the quantized
 * cache:  o[b, h] = sum_t p_t v_hat[b, t, h / G],  p = softmax over t <
 * lengths[b] of s_t = q_hat . k_hat[b, t, h / G] / sqrt(128), G = Hq / Hkv.
 * The query is quantized per 32-element block (scale fl(amax / 127) in
 * float32, codes as tq_kv_quantize_k) so each key block's dot product is an
 * exact integer; values are summed in the rotated domain and rotated back
 * once per head.  With G >= 4 the value sums run on the matrix cores with
 * fp16 operands (the centroid, and the weight 2^(s - m) * norm scaled by a
 * power of two per wavefront so that it cannot overflow): each product
 * carries at most about 2^-11 relative error before the float32 sums.
 *   q        [B, Hq, 128] TQ_BF16 or TQ_F32, 16-byte aligned.
 *   lengths  int32 [B] device, each clamped to [0, T_max] (0 gives o = 0).
 *   k_codes  int8 [B, Hkv, T_max, 128], k_scales fp16 [B, Hkv, T_max, 4]
 *            (tq_kv_quantize_k rows in this order: head-major, so the
 *            tokens of one cache head are contiguous).
 *   v_packed uint8 [B, Hkv, T_max, 64], v_norms fp16 [B, Hkv, T_max]
 *            (tq_kv_quantize_v rows in this order).
 *   sign     [host] the words the values were encoded with.
 *   o        float32 [B, Hq, 128] (output).
 *   workspace device, >= tq_attn_workspace_bytes(B, Hq, T_max) bytes; the
 *            call owns it until the stream reaches the end of the call.
 * G must be 1, 2, 4 or 8; B, Hq, Hkv <= 65535; T_max <= 2^31 - 1 (the kernels
 * index tokens with 32-bit signed integers).
 * Errors: TQ_EINVAL (null, non-positive sizes, workspace too small),
 * TQ_ESHAPE, TQ_EALIGN, TQ_EDTYPE. */
tq_status tq_attn_decode(const void* q, tq_dtype qt, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                         int64_t T_max, const int32_t* lengths, const int8_t* k_codes,
                         const uint16_t* k_scales, const uint8_t* v_packed, const uint16_t* v_norms,
                         const uint32_t sign[4], float* o, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/* tq_attn_decode for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation, arguments, layout, limits and errors without the
 * workspace.  The split partials go to a device array inside the library
 * (TQ_ATTN_NOALLOC_SCRATCH_BYTES, held by every device the library runs on
 * until the process ends); a call whose tq_attn_workspace_bytes(B, Hq,
 * T_max) exceeds it is rejected with TQ_ESHAPE before anything launches.
 * Calls on one device share that array, so calls that overlap on one device
 * (other streams, other threads) race; calls in stream order do not.  The
 * call allocates nothing; its first call on a device looks up the array's
 * device address (TQ_EDEVICE if that fails). */
#define TQ_ATTN_NOALLOC_SCRATCH_BYTES (8u << 20)
tq_status tq_attn_decode_noalloc(const void* q, tq_dtype qt, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                                 int64_t T_max, const int32_t* lengths, const int8_t* k_codes,
                                 const uint16_t* k_scales, const uint8_t* v_packed, const uint16_t* v_norms,
                                 const uint32_t sign[4], float* o, hipStream_t stream);

/* Measurement helper: read `bytes` bytes at p (device, 16-byte aligned, bytes
 * a positive multiple of 16) through a plain streaming-read kernel with the
 * decode GEMV's launch shape (one 1024-thread workgroup per compute unit),
 * and store one XOR fold per wavefront in sink (device, at least
 * TQ_STREAM_READ_SINK_WORDS words; the folds carry no meaning beyond keeping
 * the loads).  Timing it on the bytes of a GEMV launch
 * gives the read envelope that launch is compared with (TQ4 page,
 * "解码速度：分硬件汇总": decode is bound by memory bandwidth).
 * Errors: TQ_EINVAL (null, zero bytes), TQ_ESHAPE (bytes % 16), TQ_EALIGN. */
#define TQ_STREAM_READ_SINK_WORDS 16384
tq_status tq_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
