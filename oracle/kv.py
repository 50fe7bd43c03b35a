"""turbo4 KV cache: PolarQuant V vectors (norm, rotation, 16-centroid index), q8_0 K
vectors, and decode attention over them.

Test infrastructure only (see the package docstring).

What the pages say:

* TQ4 page, the paragraph after the "格式原理" list: the weight rotation is
  the one TurboQuant's KV-cache compression uses; the fork's reference code
  builds the codebook with Lloyd's algorithm for the distribution of the
  rotated coordinates, and its PolarQuant quantize/dequantize extracts the
  norm, rotates, takes the nearest-centroid index, then inverse-rotates and
  rescales; the fast structured rotation is random signs plus a Hadamard
  transform, O(d log d).  turbo4 is the 16-centroid KV variant the TQ4_1S
  codebook came from (same paragraph).
* TQ4 page, "叠加压缩：权重 + KV 缓存" (the KV measurements on two GPUs):
  asymmetric q8_0 keys with turbo4 values beats the symmetric turbo4 cache in
  prefill and decode.

Readings taken (each also listed in the design notes):

* One head vector is the unit: head_dim d = 128 (the Llama shapes the pages
  measure), the whole vector is rotated (O(d log d)), not 32-element blocks.
* D is one 128-entry sign vector: bits 0..63 are the first splitmix64 output
  of the seed, bits 64..127 the second (bit i set flips element i).
* turbo4 encode of a vector v, float32 in this order:
    w_i  = float32(v_i)
    ss   = pairwise tree (index order, 7 levels) of fl(w_i * w_i)
    n16  = fp16_sat(sqrt(ss))   (RNE, saturating);  nn = float32(n16)
    u    = FWHT_128(D w), unnormalised, stages h = 1, 2, ..., 64
    idx_i = #{k : u_i > fl(nn * m_k)}   (m_k the N(0,1) codebook midpoints)
  u_i / ||w|| is sqrt(d) times the i-th coordinate of the rotated unit
  vector, whose law is close to N(0, 1) for d = 128, so the TQ4_1S codebook
  applies as is.  Storage: 64 bytes of nibbles (element 2j in the low nibble
  of byte j) and the fp16 norm, 4.125 bits per element.
  Decode: v_hat = (nn / d) * D H c[idx]   (R^T = D H / sqrt(d), c / sqrt(d)).
* q8_0 keys: per 32-element block of the head vector, scale fp16(amax/127),
  code = clamp(rint(k / dd), -127, 127) (the definition of oracle.q8).
* Attention for one new token per sequence: the query is quantized per
  32-element block the way the int8 GEMV quantizes its activation (dq =
  fl(amax / 127), codes by the same rule), so every key block's dot product
  is an exact integer;  s_t = (1 / sqrt d) sum_b dq_b dk_{t,b} sum_i qc_i
  kc_{t,i};  p = softmax(s) over t < length;  o = sum_t p_t v_hat_t.  With
  H_q query heads and H_kv cache heads, head h reads cache head
  h // (H_q / H_kv).
"""

import numpy as np

from . import codebook
from .q8 import Q8_MAX, _codes, quantize_act_q8
from .tq4_1s import BLOCK, _pairwise_sum16, fp16_bits_to_f32, fp16_sat, hadamard, splitmix64

HEAD_DIM = 128


def kv_sign_words(seed: int) -> list:
    """The 128 sign bits as four 32-bit words (word w holds bits 32 w .. 32 w + 31)."""
    a, b = splitmix64(seed, 2)
    return [a & 0xFFFFFFFF, a >> 32, b & 0xFFFFFFFF, b >> 32]


DEFAULT_KV_SIGN = kv_sign_words(0)


def kv_sign_vector(words) -> np.ndarray:
    """D as float64 +-1 [128]: entry i is -1 when bit i is set."""
    bits = np.array([(int(words[i // 32]) >> (i % 32)) & 1 for i in range(HEAD_DIM)])
    return np.where(bits == 1, -1.0, 1.0)


def fwht_f32(v: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of the last axis (a power of two) in float32:
    stages h = 1, 2, 4, ...; the pair (i, i + h), bit h of i clear, becomes (v_i + v_{i+h}, v_i - v_{i+h})."""
    u = np.array(v, dtype=np.float32, copy=True)
    n = u.shape[-1]
    idx = np.arange(n)
    h = 1
    while h < n:
        lo = idx[(idx & h) == 0]
        a = u[..., lo].copy()
        b = u[..., lo + h].copy()
        u[..., lo] = a + b
        u[..., lo + h] = a - b
        h *= 2
    return u


def turbo4_quantize_o32(V: np.ndarray, words=None, centroids32=None, return_parts: bool = False):
    """V [n, 128] (float32-exact values) -> (packed uint8 [n, 64], norm fp16 bits uint16 [n])."""
    w = np.asarray(V, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] != HEAD_DIM:
        raise ValueError("V must be [n, 128]")
    words = DEFAULT_KV_SIGN if words is None else words
    c32 = codebook.tq4_codebook_f32() if centroids32 is None else np.asarray(centroids32, np.float32)
    m32 = codebook.tq4_midpoints_f32(c32)
    ss = _pairwise_sum16((w * w).astype(np.float32))                    # pairwise tree over 128
    n16 = fp16_sat(np.sqrt(ss).astype(np.float32))
    nn = n16.astype(np.float32)
    flip = kv_sign_vector(words) < 0
    u = fwht_f32(np.where(flip, -w, w).astype(np.float32))
    thr = (nn[:, None] * m32[None, :]).astype(np.float32)               # [n, 15]
    idx = (u[:, :, None] > thr[:, None, :]).sum(axis=-1).astype(np.uint8)
    packed = (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)
    out = (packed, n16.view(np.uint16).copy())
    return out + (u, idx) if return_parts else out


def turbo4_indices(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    idx = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int64)
    idx[:, 0::2] = p & 0x0F
    idx[:, 1::2] = p >> 4
    return idx


def turbo4_dequantize_o64(packed: np.ndarray, norms: np.ndarray, words=None, centroids32=None) -> np.ndarray:
    """v_hat = (nn / d) D H c[idx] in float64, [n, 128]."""
    words = DEFAULT_KV_SIGN if words is None else words
    c32 = codebook.tq4_codebook_f32() if centroids32 is None else np.asarray(centroids32, np.float32)
    c = c32.astype(np.float64)[turbo4_indices(packed)]                  # [n, 128]
    nn = fp16_bits_to_f32(np.asarray(norms, dtype=np.uint16)).astype(np.float64)
    H = hadamard(HEAD_DIM)
    return (nn[:, None] / HEAD_DIM) * (c @ H.T) * kv_sign_vector(words)[None, :]


def q8_0_quantize_o32(X: np.ndarray):
    """Rows [n, d] (float32-exact, d % 32 == 0) -> int8 codes [n, d], fp16 scale bits [n, d/32]."""
    x = np.asarray(X, dtype=np.float32)
    n, d = x.shape
    if d % BLOCK:
        raise ValueError("d must be a multiple of 32")
    blocks = x.reshape(n, d // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    d16 = fp16_sat((amax / np.float32(Q8_MAX)).astype(np.float32))
    codes = _codes(blocks, d16.astype(np.float32))
    return codes.reshape(n, d), d16.view(np.uint16).copy()


def score_scale(d: int) -> float:
    """The 1 / sqrt(d) of scaled dot-product attention."""
    return 1.0 / np.sqrt(d)


def attn_decode_o64(q, lengths, k_codes, k_scales, v_packed, v_norms, words=None, centroids32=None):
    """Decode attention over the quantized cache, float64.

    q [B, Hq, 128]; lengths [B]; head-major cache: k_codes int8 [B, Hkv, T, 128]; k_scales fp16 bits
    [B, Hkv, T, 4]; v_packed uint8 [B, Hkv, T, 64]; v_norms fp16 bits [B, Hkv, T].
    Returns (o [B, Hq, 128], bound [B, Hq]) where bound = sum_t p_t (nn_t / d) sum_j |c[idx_tj]|, the
    largest magnitude any output coordinate's terms can reach (the parity bound is stated against it).
    """
    words = DEFAULT_KV_SIGN if words is None else words
    c32 = codebook.tq4_codebook_f32() if centroids32 is None else np.asarray(centroids32, np.float32)
    qa = np.asarray(q, dtype=np.float32)
    B, Hq, d = qa.shape
    _, Hkv, T, _ = k_codes.shape
    G = Hq // Hkv
    nb = d // BLOCK
    o = np.zeros((B, Hq, d))
    bound = np.zeros((B, Hq))
    for b in range(B):
        L = int(lengths[b])
        if L <= 0:
            continue
        for h in range(Hq):
            g = h // G
            qc, dq = quantize_act_q8(qa[b, h])                            # [128], [4]
            kc = k_codes[b, g, :L].astype(np.int64).reshape(L, nb, BLOCK)
            dk = fp16_bits_to_f32(k_scales[b, g, :L]).astype(np.float64)   # [L, 4]
            isum = (kc * qc.astype(np.int64).reshape(1, nb, BLOCK)).sum(axis=-1)
            s = (dk * dq.astype(np.float64)[None, :] * isum).sum(axis=1) * score_scale(d)
            p = np.exp(s - s.max())
            p /= p.sum()
            vh = turbo4_dequantize_o64(v_packed[b, g, :L], v_norms[b, g, :L], words, c32)
            o[b, h] = p @ vh
            nn = fp16_bits_to_f32(v_norms[b, g, :L]).astype(np.float64)
            cabs = np.abs(c32.astype(np.float64)[turbo4_indices(v_packed[b, g, :L])]).sum(axis=1)
            bound[b, h] = (p * nn / d * cabs).sum()
    return o, bound
