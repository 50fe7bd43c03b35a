"""RSF-lite: a search over nearby multiples of each block scale (TQ4_1S, NVFP4, MXFP6).

Test infrastructure only (see the package docstring).

What the quantizer-tool page says (section "RSF"): refined scale-factor
fitting measures the (importance-weighted) reconstruction error, searches
nearby multiples of the scale factor and keeps the one whose lattice fits
better; it was designed for NVFP4/MXFP6 and later applied to other formats.

Readings taken (each also listed in the design notes):

* No importance weights are available (no calibration data): the error is
  the plain squared error of the 16 values a scale serves, measured in the
  rotated domain (the rotation is orthogonal, so this is the weight-domain
  error up to rounding).
* "Nearby multiples": nine multipliers 1 + j/16, j = -4..4 (0.75 .. 1.25),
  applied to the TQ4_1S base scale d = fp16(RMS).  Candidate
  d_j = fp16_sat(float32(dd * (1 + j/16))) (the float32 product is exact).
* For every candidate, the indices are re-chosen with the quantizer's own
  rule (count of thresholds fl(d_j * m_k) strictly below w'), and the error
  is, in float32: e_i = w'_i - fl(d_j * c[idx_i]); s_i = e_i * e_i; E = the
  pairwise tree of the 16 s_i in index order.
* The smallest E wins; on equal E the multiplier closest to 1 wins, and of
  two equally close the smaller one (candidates are tried in the order
  j = 0, -1, +1, -2, +2, -3, +3, -4, +4 and only a strictly smaller error
  replaces the current choice).  j = 0 reproduces the plain quantizer, so the
  result is never worse than it.  A zero base scale stays zero.

The same search for the block-float formats (the page built RSF for them):

* NVFP4: for each 16-element block, candidates sb_j = E4M3_RNE_satfinite(
  dec(sb_0) * (1 + j/16)), j = -4..4, in the same order, where sb_0 is the
  plain block scale (the float32 product is exact: at most 4 x 5 significant
  bits).  Each candidate re-encodes the block exactly as the plain encoder
  does (eff_j = fl(dec(sb_j) * s_t), code = E2M1(fl(w / eff_j)), all codes +0
  when eff_j = 0) and is scored by e_i = w_i - fl(e2m1(code_i) * eff_j),
  E = pairwise tree of the 16 fl(e_i * e_i).  The tensor scale s_t is not
  searched.
* MXFP6: the E8M0 scale is a power of two, so its nearby multiples are the
  neighbouring exponents: e_0 + j for j = 0, -1, +1 (tried in that order,
  clamped to [-127, 127]), e_0 the plain exponent.  Each re-encodes the block
  (code = E3M2(w * 2^-e)), e_i = w_i - e3m2(code_i) * 2^e (exact in float32),
  E = the pairwise tree of the 32 fl(e_i * e_i) (two 16-element trees, then
  their sum).  An all-zero block keeps scale byte 0 and +0 codes.
"""

import numpy as np

from . import blockfp
from . import codebook
from .minifloat import E2M1, E3M2, E4M3FN
from .tq4_1s import BLOCK, HALF, DEFAULT_SIGN_MASK, _pairwise_sum16, fp16_sat, pack_nibbles, quantize_o32

ORDER = (0, -1, 1, -2, 2, -3, 3, -4, 4)


def multiplier(j: int) -> np.float32:
    return np.float32(1.0 + j / 16.0)


def half_error_f32(wh: np.ndarray, dd: np.ndarray, idx: np.ndarray, c32: np.ndarray) -> np.ndarray:
    """Canonical float32 squared error of halves wh [..., 16] decoded as fl(dd * c[idx])."""
    q = (dd[..., None] * c32[idx]).astype(np.float32)
    e = (wh - q).astype(np.float32)
    return _pairwise_sum16((e * e).astype(np.float32))


def search_halves(halves: np.ndarray, dd0: np.ndarray, c32: np.ndarray, m32: np.ndarray):
    """The scale search on rotated halves [..., 16] with plain scales dd0 [...] (float32).

    Returns (fp16 scales [...], indices [..., 16] uint8, float32 errors [...]).
    """
    best_err = best_d = best_idx = None
    for j in ORDER:
        dj = fp16_sat((dd0 * multiplier(j)).astype(np.float32))            # fp16
        ddj = dj.astype(np.float32)
        thr = (ddj[..., None] * m32).astype(np.float32)                    # [..., 15]
        idx = (halves[..., None] > thr[..., None, :]).sum(axis=-1).astype(np.uint8)
        err = half_error_f32(halves, ddj, idx, c32)
        if best_err is None:
            best_err, best_d, best_idx = err, dj, idx
        else:
            take = err < best_err
            best_err = np.where(take, err, best_err)
            best_d = np.where(take, dj, best_d)
            best_idx = np.where(take[..., None], idx, best_idx)
    return best_d, best_idx, best_err


def quantize_rsf_o32(W: np.ndarray, sign_mask: int = DEFAULT_SIGN_MASK, centroids32=None, return_parts: bool = False):
    """TQ4_1S quantization with the RSF-lite scale search; same outputs and layout as
    :func:`oracle.tq4_1s.quantize_o32` (packed [N, K/2], scales [N, K/16] fp16 bits)."""
    c32 = codebook.tq4_codebook_f32() if centroids32 is None else np.asarray(centroids32, np.float32)
    m32 = codebook.tq4_midpoints_f32(c32)
    _, _, wr, dd0, _ = quantize_o32(W, sign_mask, c32, return_parts=True)
    n, nb, _ = wr.shape
    best_d, best_idx, best_err = search_halves(wr.reshape(n, nb, 2, HALF), dd0, c32, m32)
    packed = pack_nibbles(best_idx.reshape(n, nb * BLOCK))
    scales = best_d.reshape(n, nb * 2).view(np.uint16).copy()
    if return_parts:
        return packed, scales, wr, best_err
    return packed, scales


# ----------------------------------------------------------------------------
# block-float formats
# ----------------------------------------------------------------------------

MX_ORDER = (0, -1, 1)


def tree32_f32(s: np.ndarray) -> np.ndarray:
    """Pairwise float32 sum of the last axis (length 32): tree(s[:16]) + tree(s[16:])."""
    s = np.asarray(s, dtype=np.float32)
    return (_pairwise_sum16(s[..., :16]) + _pairwise_sum16(s[..., 16:])).astype(np.float32)


def _keep_better(best, cand):
    """best/cand = (err, scale byte, codes); a strictly smaller error replaces the current choice."""
    if best is None:
        return cand
    take = cand[0] < best[0]
    return (np.where(take, cand[0], best[0]), np.where(take, cand[1], best[1]),
            np.where(take[..., None], cand[2], best[2]))


def nvfp4_quantize_rsf_o32(W: np.ndarray, return_errors: bool = False):
    """NVFP4 with the block-scale search; outputs as :func:`oracle.blockfp.nvfp4_quantize_o32`."""
    W = np.asarray(W, dtype=np.float32)
    n, k = W.shape
    if k % blockfp.NVFP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    s_t = blockfp.nvfp4_tensor_scale(W)
    nb = k // blockfp.NVFP4_BLOCK
    if s_t == 0:
        z = (np.zeros((n, k // 2), np.uint8), np.zeros((n, nb), np.uint8), s_t)
        return z + (np.zeros((n, nb), np.float32),) if return_errors else z
    blocks = W.reshape(n, nb, blockfp.NVFP4_BLOCK)
    amax_b = np.max(np.abs(blocks), axis=-1)
    r = (amax_b / np.float32(np.float32(blockfp.E2M1_MAX) * s_t)).astype(np.float32)
    base = E4M3FN.decode(E4M3FN.encode(r.astype(np.float64))).astype(np.float32)
    best = None
    for j in ORDER:
        rj = (base * multiplier(j)).astype(np.float32)
        sbj = E4M3FN.encode(rj.astype(np.float64)).astype(np.int64)
        eff = (E4M3FN.decode(sbj).astype(np.float32) * s_t).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (blocks / eff[..., None]).astype(np.float32)
        codes = np.where(eff[..., None] == 0, 0, E2M1.encode(q.astype(np.float64))).astype(np.int64)
        qhat = (E2M1.decode(codes).astype(np.float32) * eff[..., None]).astype(np.float32)
        e = (blocks - qhat).astype(np.float32)
        err = _pairwise_sum16((e * e).astype(np.float32))
        best = _keep_better(best, (err, sbj, codes))
    err, sb, codes = best
    codes = codes.astype(np.uint8).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    out = (packed, sb.astype(np.uint8), s_t)
    return out + (err,) if return_errors else out


def mxfp6_quantize_rsf_o32(W: np.ndarray, return_errors: bool = False):
    """MXFP6 with the scale-exponent search; outputs as :func:`oracle.blockfp.mxfp6_quantize_o32`."""
    W = np.asarray(W, dtype=np.float32)
    n, k = W.shape
    if k % blockfp.MXFP6_BLOCK:
        raise ValueError("K must be a multiple of 32")
    nb = k // blockfp.MXFP6_BLOCK
    b32 = W.reshape(n, nb, blockfp.MXFP6_BLOCK)
    b64 = b32.astype(np.float64)
    amax_b = np.max(np.abs(b64), axis=-1)
    e0 = blockfp.mxfp6_scale_exponent(amax_b)
    best = None
    for j in MX_ORDER:
        ej = np.clip(e0 + j, -127, 127)
        codes = E3M2.encode(np.ldexp(b64, (-ej)[..., None])).astype(np.int64)
        qhat = np.ldexp(E3M2.decode(codes), ej[..., None]).astype(np.float32)
        e = (b32 - qhat).astype(np.float32)
        err = tree32_f32((e * e).astype(np.float32))
        best = _keep_better(best, (err, ej + 127, codes))
    err, byte, codes = best
    zero = amax_b == 0
    codes = np.where(zero[..., None], 0, codes).astype(np.uint8)
    byte = np.where(zero, 0, byte).astype(np.uint8)
    err = np.where(zero, np.float32(0), err).astype(np.float32)
    out = (blockfp.pack6(codes.reshape(n, k)), byte)
    return out + (err,) if return_errors else out
