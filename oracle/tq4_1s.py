"""TQ4_1S block encoding: rotation, quantization, dequantization, GEMV/GEMM.

Test infrastructure only (see the package docstring).

What the TQ4 page fixes ("格式原理", items 1-3 and the paragraph after):

1. each 32-element block of a weight row gets a randomized Walsh-Hadamard
   rotation with sign flips (the same rotation family as TurboQuant's KV
   cache; the sign source is described as golden-ratio sign flips);
2. every rotated coordinate is mapped independently to the nearest of the 16
   Lloyd-Max centroids of N(0,1);
3. elements 0-15 and 16-31 of a block keep separate scales d0 and d1;
   16 centroids, plain nibble packing and no correction term.

The decode-speed section adds that the activation can be rotated once
instead (the transform is orthogonal), after which dequantization is a
centroid lookup times a scale.

Readings taken where the pages are silent (each also listed in the design
notes):

* R = (1/sqrt 32) * H32 * D, H32 the Sylvester Hadamard matrix in natural
  order, D = diag(+-1) from a 32-bit ``sign_mask`` (bit i set -> D_i = -1).
  One mask serves every block, tensor and activation.  Its default is the low
  32 bits of the first splitmix64 output for seed 0 (splitmix64 steps its
  state by the 64-bit golden-ratio constant 0x9E3779B97F4A7C15).
* The scale of a half block is its RMS in the rotated domain, rounded to
  fp16 (round-to-nearest-even, saturating at 65504, subnormals kept).
* The index is the nearest centroid to w'/d, taken as the count of float32
  thresholds float32(d * m_k) that w' exceeds strictly (ties -> lower index).
* Layout: ``packed[n, j]`` (uint8, K/2 per row) holds element 2j in its low
  nibble and element 2j+1 in its high nibble; ``scales[n, 2b + h]`` holds the
  fp16 bits of d_h of block b.

The canonical float32 quantizer (:func:`quantize_o32`) fixes the order of
every float32 operation so that another implementation can reproduce its
bytes exactly:

  v   = D w                                  (exact)
  u   = FWHT32(v), butterfly stages h = 1, 2, 4, 8, 16, each
        (v_i, v_{i+h}) <- (v_i + v_{i+h}, v_i - v_{i+h})
  w'  = u * float32(1/sqrt 32)               (one rounding)
  per half: sq_i = w'_i * w'_i; ss = pairwise tree in index order;
            rms = sqrt(ss * 0.0625); d = fp16_sat(rms); dd = float32(d)
  idx = #{k : w' > float32(dd * m_k)}
"""

import math

import numpy as np

from . import codebook

BLOCK = 32
HALF = 16
S32 = np.float32(1.0 / math.sqrt(32.0))  # 0x3E3504F3
FP16_MAX = 65504.0

_MASK64 = (1 << 64) - 1
GOLDEN64 = 0x9E3779B97F4A7C15


# ----------------------------------------------------------------------------
# sign vector D
# ----------------------------------------------------------------------------

def splitmix64(seed: int, count: int = 1) -> list:
    """The first ``count`` outputs of splitmix64 (Steele, Lea, Flood 2014) from ``seed``.

    state += 0x9E3779B97F4A7C15; z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9; z = (z ^ (z >> 27)) * 0x94D049BB133111EB;
    output z ^ (z >> 31)   (all arithmetic mod 2^64).
    """
    out = []
    state = seed & _MASK64
    for _ in range(count):
        state = (state + GOLDEN64) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_mask_from_seed(seed: int) -> int:
    """Low 32 bits of the first splitmix64 output for ``seed``."""
    return splitmix64(seed, 1)[0] & 0xFFFFFFFF


DEFAULT_SIGN_MASK = sign_mask_from_seed(0)


def sign_vector(sign_mask: int) -> np.ndarray:
    """D as a float64 vector of +-1: entry i is -1 when bit i of ``sign_mask`` is set."""
    bits = (int(sign_mask) >> np.arange(BLOCK)) & 1
    return np.where(bits == 1, -1.0, 1.0)


# ----------------------------------------------------------------------------
# Hadamard rotation
# ----------------------------------------------------------------------------

def hadamard(n: int = BLOCK) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (power of two), float64.

    H_1 = [1];  H_2m = [[H_m, H_m], [H_m, -H_m]].
    """
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_f64(blocks: np.ndarray, sign_mask: int) -> np.ndarray:
    """w' = (1/sqrt 32) H32 D w for every 32-vector along the last axis (float64)."""
    b = np.asarray(blocks, dtype=np.float64)
    d = sign_vector(sign_mask)
    return (b * d) @ hadamard().T / math.sqrt(BLOCK)


def inverse_rotate_f64(blocks: np.ndarray, sign_mask: int) -> np.ndarray:
    """w = (1/sqrt 32) D H32 w' (the inverse of :func:`rotate_f64`), float64."""
    b = np.asarray(blocks, dtype=np.float64)
    d = sign_vector(sign_mask)
    return (b @ hadamard().T) * d / math.sqrt(BLOCK)


def fwht32_f32(v: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the last axis (length 32) in float32.

    Stages h = 1, 2, 4, 8, 16; at each stage the pair (i, i + h), i with bit h
    clear, becomes (v_i + v_{i+h}, v_i - v_{i+h}).  The result is H32 v.
    """
    u = np.array(v, dtype=np.float32, copy=True)
    h = 1
    while h < BLOCK:
        idx = np.arange(BLOCK)
        lo = idx[(idx & h) == 0]
        hi = lo + h
        a = u[..., lo].copy()
        b = u[..., hi].copy()
        u[..., lo] = a + b
        u[..., hi] = a - b
        h *= 2
    return u


def rotate_f32(blocks: np.ndarray, sign_mask: int) -> np.ndarray:
    """Canonical float32 rotation of 32-vectors: FWHT32(D w) * float32(1/sqrt 32)."""
    w = np.asarray(blocks, dtype=np.float32)
    flip = ((int(sign_mask) >> np.arange(BLOCK)) & 1).astype(bool)
    v = np.where(flip, -w, w).astype(np.float32)
    return (fwht32_f32(v) * S32).astype(np.float32)


# ----------------------------------------------------------------------------
# fp16 helpers
# ----------------------------------------------------------------------------

def fp16_sat(x: np.ndarray) -> np.ndarray:
    """float32 -> fp16 with round-to-nearest-even, saturating at 65504 (x >= 0)."""
    x = np.asarray(x, dtype=np.float32)
    return np.minimum(x, np.float32(FP16_MAX)).astype(np.float16)


def fp16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ----------------------------------------------------------------------------
# quantizer
# ----------------------------------------------------------------------------

def _pairwise_sum16(sq: np.ndarray) -> np.ndarray:
    """((((s0+s1)+(s2+s3))+((s4+s5)+(s6+s7)))+(((s8+s9)+(s10+s11))+((s12+s13)+(s14+s15))))
    over the last axis (length 16), in the array's dtype."""
    s = sq
    while s.shape[-1] > 1:
        s = s[..., 0::2] + s[..., 1::2]
    return s[..., 0]


def _as_blocks(W: np.ndarray) -> np.ndarray:
    W = np.asarray(W)
    if W.ndim != 2 or W.shape[1] % BLOCK:
        raise ValueError("W must be [N, K] with K a multiple of 32")
    n, k = W.shape
    return W.reshape(n, k // BLOCK, BLOCK)


def pack_nibbles(idx: np.ndarray) -> np.ndarray:
    """[N, K] indices 0..15 -> [N, K/2] bytes; element 2j in the low nibble of byte j."""
    idx = np.asarray(idx, dtype=np.uint8)
    return (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`: [N, K/2] bytes -> [N, K] indices."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def quantize_o32(W: np.ndarray, sign_mask: int = DEFAULT_SIGN_MASK, centroids32=None,
                 return_parts: bool = False):
    """Canonical float32 TQ4_1S quantizer.

    W: [N, K] values exactly representable in float32 (fp32 or bf16 input).
    Returns (packed uint8 [N, K/2], scales uint16 [N, K/16] = fp16 bits of
    d0, d1 per block); with ``return_parts`` also the rotated float32 blocks,
    the float32 scales dd and the index array [N, K].
    """
    c32 = codebook.tq4_codebook_f32() if centroids32 is None else np.asarray(centroids32, np.float32)
    m32 = codebook.tq4_midpoints_f32(c32)
    blocks = _as_blocks(W).astype(np.float32)
    n, nb, _ = blocks.shape

    wr = rotate_f32(blocks, sign_mask)                        # [n, nb, 32]
    halves = wr.reshape(n, nb, 2, HALF)
    sq = (halves * halves).astype(np.float32)
    ss = _pairwise_sum16(sq)                                  # [n, nb, 2]
    rms = np.sqrt((ss * np.float32(0.0625)).astype(np.float32)).astype(np.float32)
    d16 = fp16_sat(rms)                                       # [n, nb, 2] fp16
    dd = d16.astype(np.float32)

    thr = (dd[..., None] * m32).astype(np.float32)            # [n, nb, 2, 15]
    idx = (halves[..., None] > thr[..., None, :]).sum(axis=-1).astype(np.uint8)
    idx = idx.reshape(n, nb * BLOCK)

    packed = pack_nibbles(idx)
    scales = d16.reshape(n, nb * 2).view(np.uint16).copy()
    if return_parts:
        return packed, scales, wr, dd, idx
    return packed, scales


def quantize_o64(W: np.ndarray, sign_mask: int = DEFAULT_SIGN_MASK, centroids32=None):
    """The same encoding computed in float64 with a brute-force nearest centroid.

    Rotation and RMS in float64, d = fp16_sat(rms), idx = argmin_k |w'/d - c_k|
    (lower index on an exact tie; d = 0 -> index of the centroid nearest 0 from
    below).  Used to check the canonical float32 path away from near-ties.
    Returns (idx [N, K] uint8, d [N, K/16] float64).
    """
    c = np.asarray(codebook.tq4_codebook_f32() if centroids32 is None else centroids32, np.float64)
    blocks = _as_blocks(W).astype(np.float64)
    n, nb, _ = blocks.shape
    wr = rotate_f64(blocks, sign_mask).reshape(n, nb, 2, HALF)
    rms = np.sqrt(np.mean(wr * wr, axis=-1))
    d = fp16_sat(rms.astype(np.float32)).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(d[..., None] > 0, wr / d[..., None], 0.0)
    dist = np.abs(t[..., None] - c)                           # [..., 16, 16]
    idx = np.argmin(dist, axis=-1).astype(np.uint8)           # first minimum = lower index
    return idx.reshape(n, nb * BLOCK), d.reshape(n, nb * 2)


# ----------------------------------------------------------------------------
# dequantization and products
# ----------------------------------------------------------------------------

def rotated_weights_f64(packed: np.ndarray, scales: np.ndarray, centroids32=None) -> np.ndarray:
    """q = d_h * c[idx] in the rotated domain, float64 [N, K]."""
    c = np.asarray(codebook.tq4_codebook_f32() if centroids32 is None else centroids32, np.float64)
    idx = unpack_nibbles(packed)
    n, k = idx.shape
    d = fp16_bits_to_f32(scales).astype(np.float64).reshape(n, k // HALF)
    return c[idx] * np.repeat(d, HALF, axis=1)


def dequantize_o64(packed: np.ndarray, scales: np.ndarray, sign_mask: int = DEFAULT_SIGN_MASK,
                   centroids32=None) -> np.ndarray:
    """W_deq = (1/sqrt 32) D H32 (d * c[idx]) per block, float64 [N, K].

    The TQ4 page's Python reference is described as dequantizing by inverse
    rotation and rescaling; this is that inverse applied to the scaled centroids.
    """
    q = rotated_weights_f64(packed, scales, centroids32)
    n, k = q.shape
    w = inverse_rotate_f64(q.reshape(n, k // BLOCK, BLOCK), sign_mask)
    return w.reshape(n, k)


def gemm_o64(packed: np.ndarray, scales: np.ndarray, X: np.ndarray,
             sign_mask: int = DEFAULT_SIGN_MASK, centroids32=None):
    """Y[m, n] = sum_k W_deq[n, k] X[m, k] in float64, and the tolerance scale.

    X: [M, K] (or [K] for a GEMV) taken exactly as given (fp32/bf16 values),
    not rotated.  Returns (Y [M, N], A [M, N]) with A = sum_k |W_deq[n,k] X[m,k]|,
    the quantity the parity bound |dY| <= 1e-3 * A is stated against.
    """
    Wd = dequantize_o64(packed, scales, sign_mask, centroids32)
    Xa = np.atleast_2d(np.asarray(X, dtype=np.float64))
    return Xa @ Wd.T, np.abs(Xa) @ np.abs(Wd).T


def gemv_rows_o64(packed_rows: np.ndarray, scales_rows: np.ndarray, x: np.ndarray,
                  sign_mask: int = DEFAULT_SIGN_MASK, centroids32=None):
    """GEMV restricted to the given rows (for sampled checks at full size)."""
    y, a = gemm_o64(packed_rows, scales_rows, np.asarray(x)[None, :], sign_mask, centroids32)
    return y[0], a[0]
