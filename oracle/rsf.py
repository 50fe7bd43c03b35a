"""RSF-lite for TQ4_1S: a search over nearby multiples of each half-block scale.

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
"""

import numpy as np

from . import codebook
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
