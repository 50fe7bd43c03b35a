"""NVFP4 and MXFP6 block encodings, canonical float32 quantizers, float64 products.

Test infrastructure only (see the package docstring).

The pages name both formats without a recipe: NVFP4 is NVIDIA's 4-bit
float format brought in with Blackwell (llm-compressor page,
"NVFP4 + FP8 双格式支持"); the quantizer-tool page says its tool builds the
NVFP4 weight scales and the per-tensor ("input tensor") scales correctly
("目前能实现的部分功能") and that MXFP6 moves more bytes than NVFP4
("MXFP6 的未来").  The plainest public readings are used:

NVFP4 (16-element blocks of E2M1 values, an E4M3fn scale per block, one
float32 scale per tensor):

  s_t   = float32(amax|W| / 2688)          (2688 = 6 * 448: E2M1 max * E4M3 max)
  r_b   = float32(amax_b / float32(6 * s_t))
  sb    = E4M3fn_RNE_satfinite(r_b)
  eff_b = float32(dec(sb) * s_t)
  code  = E2M1_RNE_satfinite(float32(w / eff_b)); eff_b = 0 -> +0 codes
  w_deq = e2m1(code) * dec(sb) * s_t        (exact in float64)
  A tensor whose amax is 0 has s_t = 0, every scale byte 0 and every code 0.
  Packing: element 2j in the low nibble of byte j; scales [N, K/16].

MXFP6 (OCP MX: 32-element blocks of E3M2 values, one E8M0 scale per block):

  e     = floor(log2 amax_b) - 4, clamped to [-127, 127]   (4 = emax of E3M2)
  byte  = e + 127; amax_b = 0 -> byte 0 and +0 codes
  code  = E3M2_RNE_satfinite(w * 2^-e)      (the scaling is exact)
  w_deq = e3m2(code) * 2^(byte - 127)
  Packing: 4 codes per 3 bytes; element 4j+t occupies bits 6t..6t+5 of the
  little-endian 24-bit word made of bytes 3j, 3j+1, 3j+2.  Codes [N, 3K/4],
  scales [N, K/32].
"""

import numpy as np

from .minifloat import E2M1, E3M2, E4M3FN, e8m0_decode

NVFP4_BLOCK = 16
MXFP6_BLOCK = 32
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E3M2_EMAX = 4


# ----------------------------------------------------------------------------
# NVFP4
# ----------------------------------------------------------------------------

def nvfp4_tensor_scale(W: np.ndarray) -> np.float32:
    amax = np.float32(np.max(np.abs(np.asarray(W, dtype=np.float32))))
    return np.float32(amax / np.float32(E2M1_MAX * E4M3_MAX))


def nvfp4_quantize_o32(W: np.ndarray):
    """Canonical NVFP4 encoder.  W: [N, K] float32-exact values, K % 16 == 0.

    Returns (codes uint8 [N, K/2], block_scales uint8 [N, K/16], tensor_scale float32).
    """
    W = np.asarray(W, dtype=np.float32)
    n, k = W.shape
    if k % NVFP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    s_t = nvfp4_tensor_scale(W)
    blocks = W.reshape(n, k // NVFP4_BLOCK, NVFP4_BLOCK)
    if s_t == 0:
        return (np.zeros((n, k // 2), np.uint8), np.zeros((n, k // NVFP4_BLOCK), np.uint8), s_t)
    amax_b = np.max(np.abs(blocks), axis=-1)
    six_st = np.float32(np.float32(E2M1_MAX) * s_t)
    r = (amax_b / six_st).astype(np.float32)
    sb = E4M3FN.encode(r.astype(np.float64))
    eff = (E4M3FN.decode(sb).astype(np.float32) * s_t).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (blocks / eff[..., None]).astype(np.float32)
    codes = E2M1.encode(q.astype(np.float64))
    codes = np.where(eff[..., None] == 0, 0, codes).astype(np.uint8).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb.astype(np.uint8), s_t


def nvfp4_dequantize_o64(codes: np.ndarray, block_scales: np.ndarray, tensor_scale) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    c = np.empty((n, k), dtype=np.int64)
    c[:, 0::2] = codes & 0x0F
    c[:, 1::2] = codes >> 4
    vals = E2M1.decode(c)
    s = E4M3FN.decode(np.asarray(block_scales)) * float(np.float32(tensor_scale))
    return vals * np.repeat(s, NVFP4_BLOCK, axis=1)


# ----------------------------------------------------------------------------
# MXFP6
# ----------------------------------------------------------------------------

def mxfp6_scale_exponent(amax_b: np.ndarray) -> np.ndarray:
    """floor(log2 amax) - 4 from the exact binary exponent, clamped to [-127, 127]."""
    a = np.asarray(amax_b, dtype=np.float64)
    mant, ex = np.frexp(a)            # a = mant * 2^ex, mant in [0.5, 1)
    fl = ex.astype(np.int64) - 1       # floor(log2 a) for a > 0
    e = np.clip(fl - E3M2_EMAX, -127, 127)
    return np.where(a > 0, e, -127)


def pack6(codes: np.ndarray) -> np.ndarray:
    """[N, K] 6-bit codes -> [N, 3K/4] bytes (4 codes per little-endian 24-bit word)."""
    c = np.asarray(codes, dtype=np.uint32)
    n, k = c.shape
    g = c.reshape(n, k // 4, 4)
    word = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
    out = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF], axis=-1)
    return out.reshape(n, 3 * k // 4).astype(np.uint8)


def unpack6(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint32)
    n, kb = p.shape
    g = p.reshape(n, kb // 3, 3)
    word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    c = np.stack([(word >> (6 * t)) & 0x3F for t in range(4)], axis=-1)
    return c.reshape(n, kb // 3 * 4).astype(np.uint8)


def mxfp6_quantize_o32(W: np.ndarray):
    """Canonical MXFP6 encoder.  W: [N, K] float32-exact, K % 32 == 0.

    Returns (codes uint8 [N, 3K/4], scales uint8 [N, K/32]).
    """
    W = np.asarray(W, dtype=np.float32)
    n, k = W.shape
    if k % MXFP6_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = W.reshape(n, k // MXFP6_BLOCK, MXFP6_BLOCK).astype(np.float64)
    amax_b = np.max(np.abs(blocks), axis=-1)
    e = mxfp6_scale_exponent(amax_b)
    scaled = np.ldexp(blocks, (-e)[..., None])                # exact power-of-two scaling
    codes = E3M2.encode(scaled)
    codes = np.where((amax_b == 0)[..., None], 0, codes).astype(np.uint8)
    scale_bytes = np.where(amax_b == 0, 0, e + 127).astype(np.uint8)
    return pack6(codes.reshape(n, k)), scale_bytes


def mxfp6_dequantize_o64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = unpack6(codes)
    vals = E3M2.decode(c.astype(np.int64))
    s = e8m0_decode(np.asarray(scales))
    return vals * np.repeat(s, MXFP6_BLOCK, axis=1)


# ----------------------------------------------------------------------------
# products
# ----------------------------------------------------------------------------

def gemm_deq_o64(W_deq: np.ndarray, X: np.ndarray):
    """Y = X W_deq^T in float64 and the tolerance scale A = |X| |W_deq|^T."""
    Xa = np.atleast_2d(np.asarray(X, dtype=np.float64))
    return Xa @ W_deq.T, np.abs(Xa) @ np.abs(W_deq).T


def bytes_per_weight(fmt: str) -> float:
    """Stored bytes per weight: NVFP4 0.5 + 1/16 (fp32 tensor scale ignored), MXFP6 0.75 + 1/32."""
    return {"nvfp4": 0.5 + 1.0 / 16, "mxfp6": 0.75 + 1.0 / 32}[fmt]

