"""Pins for the oracle's TQ4_1S -> int8 transcode and the int8 GEMV (CPU only).

Independent anchors used here:
* the float64 dequantization (matrix Hadamard, float64 arithmetic) against
  the canonical float32 order the transcode starts from;
* rounding to the nearest integer checked in float64, with exact ties built
  by hand (ties go to even);
* closed forms: a block's largest element maps to +-127 exactly, a
  single-spike TQ4_1S block transcodes to +-127 at the spike and 0 elsewhere,
  integer activations with amax 127 keep their values;
* the GEMV as explicit integer loops on tiny inputs, and against the float64
  TQ4_1S GEMV (the transcode keeps the weights within half a q8 step).
"""

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import q8
from oracle import tq4_1s as tq

C32 = cb.tq4_codebook_f32()
MASK = tq.DEFAULT_SIGN_MASK


def _tq4(n, k, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, k)) * scale).astype(np.float32)
    return tq.quantize_o32(W, MASK)


def test_canonical_dequantization_matches_float64():
    packed, scales = _tq4(24, 512, 1)
    w32 = q8.dequantize_o32_blocks(packed, scales, MASK).reshape(24, 512).astype(np.float64)
    w64 = tq.dequantize_o64(packed, scales, MASK)
    qabs = np.abs(tq.rotated_weights_f64(packed, scales)).reshape(24, 16, 32).sum(axis=-1)
    err = np.abs(w32 - w64).reshape(24, 16, 32).max(axis=-1)
    assert np.all(err <= 4e-7 * qabs + 1e-30)


def test_codes_are_the_nearest_integers_ties_to_even():
    packed, scales = _tq4(40, 1024, 2)
    w = q8.dequantize_o32_blocks(packed, scales, MASK).astype(np.float64)       # [n, nb, 32]
    codes, sbits = q8.transcode_q8_o32(packed, scales, MASK)
    dd = tq.fp16_bits_to_f32(sbits).astype(np.float64)[..., None]
    t = w / dd                                                                 # float64 ratio
    c = codes.reshape(w.shape).astype(np.float64)
    assert np.all(np.abs(c) <= 127)
    # away from the float32 rounding of the ratio, the code is the nearest integer
    frac = np.abs(t - np.floor(t) - 0.5)
    clear = frac > 1e-5
    assert np.array_equal(c[clear], np.clip(np.round(t[clear]), -127, 127))
    # every code reconstructs its weight within half a step (plus float32 rounding)
    assert np.all(np.abs(c * dd - w) <= 0.5 * dd * (1 + 1e-6))


def test_block_maximum_maps_to_127():
    packed, scales = _tq4(32, 2048, 3)
    w = q8.dequantize_o32_blocks(packed, scales, MASK)
    codes, _ = q8.transcode_q8_o32(packed, scales, MASK)
    c = codes.reshape(w.shape).astype(np.int64)
    arg = np.abs(w).argmax(axis=-1)
    top = np.take_along_axis(c, arg[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.sign(top) == np.sign(np.take_along_axis(w, arg[..., None], axis=-1)[..., 0]))


def test_single_spike_block_closed_form():
    """A block holding a single spike a e_j quantizes to indices 11/4 with d0 = d1 = d, whose
    float32 dequantization is 32 * fl(d * 0.94234...) * s32 at j and exactly 0 elsewhere:
    the transcode gives codes sign(a) * 127 e_j and the scale fp16(|w_j| / 127)."""
    rng = np.random.default_rng(4)
    n, k = 6, 128
    W = np.zeros((n, k), dtype=np.float32)
    js = rng.integers(0, 32, (n, k // 32))
    amps = (rng.uniform(0.01, 3.0, (n, k // 32)) * rng.choice([-1, 1], (n, k // 32))).astype(np.float32)
    for r in range(n):
        for b in range(k // 32):
            W[r, 32 * b + js[r, b]] = amps[r, b]
    packed, scales = tq.quantize_o32(W, MASK)
    codes, sbits = q8.transcode_q8_o32(packed, scales, MASK)
    d = tq.fp16_bits_to_f32(scales).reshape(n, k // 32, 2)
    assert np.array_equal(d[..., 0], d[..., 1])
    cmag = np.float32(C32[11])                              # the centroid every index selects, up to sign
    wj = ((np.float32(32) * (d[..., 0] * cmag).astype(np.float32)).astype(np.float32) * tq.S32).astype(np.float32)
    expect_scale = np.minimum(wj / np.float32(127), np.float32(65504)).astype(np.float16).view(np.uint16)
    assert np.array_equal(sbits, expect_scale)
    want = np.zeros((n, k), dtype=np.int8)
    for r in range(n):
        for b in range(k // 32):
            want[r, 32 * b + js[r, b]] = 127 if amps[r, b] > 0 else -127
    assert np.array_equal(codes, want)


def test_activation_quantization_pins():
    # integers with amax 127 keep their values (dx = 1)
    rng = np.random.default_rng(5)
    x = rng.integers(-126, 127, 64).astype(np.float32)
    x[0], x[40] = 127, -127
    qx, dx = q8.quantize_act_q8(x)
    assert np.array_equal(dx, np.ones(2, np.float32)) and np.array_equal(qx.astype(np.float32), x)
    # exact half-way ratios go to the even neighbour
    x = np.zeros(32, np.float32)
    x[:9] = [127, 2.5, -2.5, 3.5, -3.5, 0.5, -0.5, 1.5, -1.5]
    qx, _ = q8.quantize_act_q8(x)
    assert list(qx[:9]) == [127, 2, -2, 4, -4, 0, 0, 2, -2]
    # one-hot and zero blocks
    x = np.zeros(64, np.float32)
    x[37] = -0.3
    qx, dx = q8.quantize_act_q8(x)
    assert qx[37] == -127 and np.count_nonzero(qx) == 1 and dx[0] == 0 and dx[1] == np.float32(np.float32(0.3) / 127)


def test_gemv_against_integer_loops():
    packed, scales = _tq4(3, 64, 6)
    codes, sbits = q8.transcode_q8_o32(packed, scales, MASK)
    x = np.random.default_rng(7).standard_normal(64).astype(np.float32)
    y, a = q8.q8_gemv_o64(codes, sbits, x)
    qx, dx = q8.quantize_act_q8(x)
    dd = tq.fp16_bits_to_f32(sbits)
    for r in range(3):
        total = 0.0
        for b in range(2):
            isum = 0
            for i in range(32):
                isum += int(codes[r, 32 * b + i]) * int(qx[32 * b + i])
            total += float(dd[r, b]) * float(dx[b]) * isum
        assert abs(y[r] - total) <= 1e-12 * max(a[r], 1e-30)


def test_q8_keeps_the_tq4_weights_and_products():
    packed, scales = _tq4(64, 4096, 8)
    codes, sbits = q8.transcode_q8_o32(packed, scales, MASK)
    wq = q8.q8_dequantize_o64(codes, sbits)
    w64 = tq.dequantize_o64(packed, scales, MASK)
    dd = np.repeat(tq.fp16_bits_to_f32(sbits).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(wq - w64) <= 0.5 * dd * (1 + 1e-5) + 1e-6 * np.abs(w64))
    x = np.random.default_rng(9).standard_normal(4096).astype(np.float32)
    y8, _ = q8.q8_gemv_o64(codes, sbits, x)
    y4, a4 = tq.gemv_rows_o64(packed, scales, x, MASK)
    assert np.all(np.abs(y8 - y4) <= 2e-2 * a4)          # quality, not parity: two roundings of 8 bits


# ---------------------------------------------------------------------------
# planted mistakes: each must fail one of the pins above
# ---------------------------------------------------------------------------

def _fails(*tests):
    for t in tests:
        try:
            t()
        except AssertionError:
            return True
    return False


def test_mistake_wrong_range_is_caught(monkeypatch):
    monkeypatch.setattr(q8, "Q8_MAX", 128)
    assert _fails(test_codes_are_the_nearest_integers_ties_to_even, test_block_maximum_maps_to_127)


def test_mistake_half_away_from_zero_is_caught(monkeypatch):
    real = q8._codes

    def wrong(v, dd):
        with np.errstate(divide="ignore", invalid="ignore"):
            t = np.where(dd[..., None] > 0, v / np.where(dd > 0, dd, np.float32(1))[..., None], np.float32(0))
        t = t.astype(np.float32)
        return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -127, 127).astype(np.int8)

    monkeypatch.setattr(q8, "_codes", wrong)
    assert _fails(test_activation_quantization_pins)
    monkeypatch.setattr(q8, "_codes", real)


def test_mistake_missing_sign_flip_is_caught(monkeypatch):
    real = q8.dequantize_o32_blocks

    def wrong(packed, scales, sign_mask, centroids32=None):
        return real(packed, scales, 0, centroids32)

    monkeypatch.setattr(q8, "dequantize_o32_blocks", wrong)
    assert _fails(test_canonical_dequantization_matches_float64)


def test_mistake_missing_normalisation_is_caught(monkeypatch):
    monkeypatch.setattr(q8, "S32", np.float32(1.0))
    assert _fails(test_canonical_dequantization_matches_float64, test_single_spike_block_closed_form)
