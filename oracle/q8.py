"""Load-time transcode of TQ4_1S weights to an int8 block format, and the int8 GEMV.

Test infrastructure only (see the package docstring).

What the TQ4 page says (section "解码速度：分硬件汇总", the note under the
decode-speed summary and the paragraph on why CUDA differs; section
"适用前提与边界", backend item): a community contribution converts TQ4_1S
tensors to q8_0 when the model is loaded, which sidesteps the fused-kernel
bottleneck on CUDA: the file keeps the TQ4_1S size and decode runs at the
speed of the backend's own q8_0 path.

The pages print no recipe for q8_0 or for the conversion.  Readings taken
(each also listed in the design notes):

* q8_0 is read as its usual meaning: 32-element blocks of int8 codes with one
  fp16 scale, value = scale * code, scale = block amax / 127.  It is restated
  here from that definition.  The layout is this library's own: codes int8
  [N, K] row-major, scales fp16 bits [N, K/32], 1.0625 bytes per weight.
  Compatibility with GGUF's interleaved q8_0 blocks is not claimed.
* The values converted are the TQ4_1S dequantized weights in a canonical
  float32 order, so that another implementation can reproduce the codes bit
  for bit:

    q_i = float32(d_h) * c[idx_i]                 (one rounding)
    u   = FWHT32(q), the quantizer's butterfly order
    w_i = D_i * (u_i * float32(1/sqrt 32))        (one rounding; the flip is exact)
    amax = max_i |w_i|
    d    = fp16_sat(amax / 127)                   (float32 division, RNE to fp16)
    dd   = float32(d)
    code_i = clamp(rint(w_i / dd), -127, 127)      (float32 division, ties to even;
                                                    dd = 0 -> code 0)

* The int8 GEMV quantizes the activation per 32-element block the same way
  (dx = float32(amax_x / 127) kept in float32, code = clamp(rint(x / dx),
  -127, 127)), so every block's dot product is an exact integer sum:
  y_n = sum_b dd[n, b] * dx[b] * sum_i code_w[n, b, i] * code_x[b, i].
  (An int8 dot-product GEMV is what a q8_0 decode path runs; the pages do not
  say how the activation is handled, and this is the plainest reading.)
"""

import numpy as np

from . import codebook
from .tq4_1s import (BLOCK, HALF, S32, fp16_bits_to_f32, fp16_sat, fwht32_f32, unpack_nibbles)

Q8_MAX = 127


def dequantize_o32_blocks(packed: np.ndarray, scales: np.ndarray, sign_mask: int, centroids32=None) -> np.ndarray:
    """TQ4_1S weights in the canonical float32 order above, float32 [N, K/32, 32]."""
    c32 = codebook.tq4_codebook_f32() if centroids32 is None else np.asarray(centroids32, np.float32)
    idx = unpack_nibbles(packed)
    n, k = idx.shape
    nb = k // BLOCK
    d = fp16_bits_to_f32(scales).reshape(n, nb, 2)                    # float32 d0, d1
    dh = np.repeat(d, HALF, axis=2)                                   # [n, nb, 32]
    q = (dh * c32[idx].reshape(n, nb, BLOCK)).astype(np.float32)
    u = fwht32_f32(q)
    w = (u * S32).astype(np.float32)
    flip = ((int(sign_mask) >> np.arange(BLOCK)) & 1).astype(bool)
    return np.where(flip, -w, w).astype(np.float32)


def _codes(v: np.ndarray, dd: np.ndarray) -> np.ndarray:
    """clamp(rint(v / dd), -127, 127) in float32 (dd broadcast over the last axis; dd = 0 -> 0)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(dd[..., None] > 0, v / np.where(dd > 0, dd, np.float32(1))[..., None], np.float32(0))
    t = t.astype(np.float32)
    return np.clip(np.rint(t), -Q8_MAX, Q8_MAX).astype(np.int8)


def transcode_q8_o32(packed: np.ndarray, scales: np.ndarray, sign_mask: int, centroids32=None):
    """TQ4_1S -> int8 codes [N, K] and fp16 scale bits [N, K/32] (canonical float32 order)."""
    w = dequantize_o32_blocks(packed, scales, sign_mask, centroids32)   # [n, nb, 32]
    amax = np.abs(w).max(axis=-1)                                      # exact
    d16 = fp16_sat((amax / np.float32(Q8_MAX)).astype(np.float32))     # [n, nb]
    dd = d16.astype(np.float32)
    codes = _codes(w, dd)
    n, nb, _ = w.shape
    return codes.reshape(n, nb * BLOCK), d16.view(np.uint16).copy()


def quantize_act_q8(x: np.ndarray):
    """Activation [K] or [M, K] (float32-exact values) -> int8 codes (same shape) and float32 scales [..., K/32]."""
    xa = np.asarray(x, dtype=np.float32)
    shp = xa.shape
    if shp[-1] % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = xa.reshape(shp[:-1] + (shp[-1] // BLOCK, BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    dx = (amax / np.float32(Q8_MAX)).astype(np.float32)
    return _codes(blocks, dx).reshape(shp), dx


def q8_dequantize_o64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """dd * code, float64 [N, K]."""
    c = np.asarray(codes, dtype=np.float64)
    n, k = c.shape
    dd = fp16_bits_to_f32(scales).astype(np.float64).reshape(n, k // BLOCK)
    return (c.reshape(n, k // BLOCK, BLOCK) * dd[..., None]).reshape(n, k)


def q8_gemv_o64(codes: np.ndarray, scales: np.ndarray, x: np.ndarray):
    """int8 GEMV of the transcoded weights with the activation quantized by :func:`quantize_act_q8`.

    Returns (y [N], A [N]) in float64: y_n = sum_b dd[n,b] dx[b] sum_i code_w code_x
    (exact integer block sums), A_n = sum_b |dd dx| sum_i |code_w code_x|, the
    scale the parity bound |dy| <= 1e-3 * A is stated against.
    """
    qx, dx = quantize_act_q8(x)
    cw = np.asarray(codes, dtype=np.int64)
    n, k = cw.shape
    nb = k // BLOCK
    cw = cw.reshape(n, nb, BLOCK)
    cx = qx.astype(np.int64).reshape(nb, BLOCK)
    isum = (cw * cx).sum(axis=-1)                                      # exact integers [n, nb]
    asum = np.abs(cw * cx).sum(axis=-1)
    dd = fp16_bits_to_f32(scales).astype(np.float64).reshape(n, nb)
    s = dd * dx.astype(np.float64)[None, :]
    return (s * isum).sum(axis=1), (np.abs(s) * asum).sum(axis=1)
