"""Pins for the oracle's TQ4_1S quantizer, dequantizer and products (CPU only).

Independent anchors used here:
* the single-spike closed form (every float32 step is exact or known);
* brute-force nearest centroid in float64 on tiny inputs;
* the float64 variant of the encoding;
* brute-force nearest-fp16 with ties to even (for the scale rounding);
* the TQ4 page's size figures (5.0 bits per weight against Q8_0's 8.5);
* the quantization error of the Lloyd-Max codebook (D16) on Gaussian data;
* matrix identities for the products (one-hot activations, M = 1, zeros).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codebook as cb
from oracle import tq4_1s as tq
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
C32 = cb.tq4_codebook_f32()
M32 = cb.tq4_midpoints_f32(C32)


def _nearest_fp16_bits(x):
    """Brute force: nearest non-negative finite fp16 to x (>= 0), ties to even bits; >= 65520 saturates."""
    allbits = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = allbits.view(np.float16).astype(np.float64)
    out = []
    for v in np.asarray(x, dtype=np.float64).ravel():
        if v >= 65504.0:
            out.append(0x7BFF)
            continue
        dist = np.abs(vals - v)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:
            best = best[(allbits[best] & 1) == 0]
        out.append(int(allbits[best[0]]))
    return np.array(out, dtype=np.uint16)


def test_fp16_rounding_against_brute_force():
    rng = np.random.default_rng(0)
    allbits = np.arange(0, 0x7BFF, dtype=np.uint16)
    vals = allbits.view(np.float16).astype(np.float64)
    pick = rng.choice(len(vals) - 1, 300, replace=False)
    mids = ((vals[pick] + vals[pick + 1]) / 2).astype(np.float32)   # exact ties (fp32 holds them)
    rand = (rng.random(300) * 10.0 ** rng.uniform(-8, 5, 300)).astype(np.float32)
    edge = np.array([0.0, 6e-8, 2.98e-8, 65504, 65519, 65520, 1e6], dtype=np.float32)
    x = np.concatenate([mids, rand, edge])
    np.testing.assert_array_equal(tq.fp16_sat(x).view(np.uint16), _nearest_fp16_bits(x))


def test_single_spike_closed_form_bit_exact():
    """w = a e_j: all |w'| = fp32(|a| s32), d0 = d1 = fp16(that), indices 11 or 4."""
    mask = tq.DEFAULT_SIGN_MASK
    h = tq.hadamard()
    d = tq.sign_vector(mask)
    rows = []
    expect_idx = []
    expect_scale = []
    for j, a in [(0, 1.0), (7, -3.25), (16, 0.02), (31, -1e-3), (12, 100.0)]:
        w = np.zeros(32, np.float32)
        w[j] = a
        rows.append(w)
        t = np.float32(np.float32(abs(a)) * tq.S32)
        sgn = np.sign(a) * d[j] * h[:, j]
        expect_idx.append(np.where(sgn > 0, 11, 4))
        expect_scale.append([np.float16(t).view(np.uint16)] * 2)
    W = np.stack(rows)
    packed, scales = tq.quantize_o32(W, mask)
    idx = np.array(expect_idx, dtype=np.uint8)
    exp_packed = (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)
    np.testing.assert_array_equal(packed, exp_packed)
    np.testing.assert_array_equal(scales, np.array(expect_scale, dtype=np.uint16))
    # dequantized spike ~ 0.94234 * sqrt(32) * d * a e_j
    Wd = tq.dequantize_o64(packed, scales, mask)
    for r, (j, a) in enumerate([(0, 1.0), (7, -3.25), (16, 0.02), (31, -1e-3), (12, 100.0)]):
        dd = float(np.float16(np.float32(abs(a)) * tq.S32))
        peak = float(C32[11]) * math.sqrt(32) * dd * np.sign(a)
        assert Wd[r, j] == pytest.approx(peak, rel=1e-12)
        off = np.delete(Wd[r], j)
        np.testing.assert_allclose(off, 0.0, atol=1e-12 * abs(peak))


def test_nibble_order_and_scale_slots():
    """A row whose rotated halves have RMS 1 and 4 and increasing / decreasing values."""
    mask = tq.DEFAULT_SIGN_MASK
    ramp = np.linspace(-2.5, 2.5, 16)
    t0 = ramp / np.sqrt(np.mean(ramp ** 2))
    t1 = -ramp / np.sqrt(np.mean(ramp ** 2)) * 4.0
    wr = np.concatenate([t0, t1])
    w = tq.inverse_rotate_f64(wr[None, :], mask).astype(np.float32)
    packed, scales = tq.quantize_o32(w, mask)
    d = tq.fp16_bits_to_f32(scales)[0].astype(np.float64)
    assert d[0] == pytest.approx(1.0, rel=2e-3)
    assert d[1] == pytest.approx(4.0, rel=2e-3)
    # expected indices by brute-force nearest centroid (float64) from the designed values
    t = np.concatenate([t0 / d[0], t1 / d[1]])
    exp = np.argmin(np.abs(t[:, None] - C32.astype(np.float64)[None, :]), axis=1)
    assert exp[0] < exp[15] and exp[16] > exp[31]          # the halves are not symmetric
    np.testing.assert_array_equal(tq.unpack_nibbles(packed)[0], exp)
    assert packed[0, 0] == exp[0] | (exp[1] << 4)
    assert packed[0, 15] == exp[30] | (exp[31] << 4)


def test_brute_force_nearest_on_tiny_blocks():
    rng = np.random.default_rng(4)
    near = 0
    total = 0
    for nblk in (1, 2, 3, 4):
        W = rng.normal(size=(8, 32 * nblk)).astype(np.float32)
        _, _, wr, dd, idx = tq.quantize_o32(W, return_parts=True)
        n = W.shape[0]
        t = wr.reshape(n, nblk, 2, 16).astype(np.float64) / dd[..., None].astype(np.float64)
        brute = np.argmin(np.abs(t[..., None] - C32.astype(np.float64)), axis=-1).reshape(n, -1)
        gap = np.min(np.abs(t[..., None] - M32.astype(np.float64)), axis=-1).reshape(n, -1)
        tie = gap <= 4 * np.finfo(np.float32).eps * np.abs(t.reshape(n, -1)).clip(1e-30)
        near += int(tie.sum())
        total += tie.size
        np.testing.assert_array_equal(idx[~tie], brute[~tie])
    assert near <= total * 1e-3


def test_float64_encoding_agrees_away_from_ties():
    W, _ = workloads.tiny_tq("cpu")
    W = W.numpy()
    _, scales, wr, dd, idx = tq.quantize_o32(W, return_parts=True)
    idx64, d64 = tq.quantize_o64(W)
    same_d = np.repeat(d64 == tq.fp16_bits_to_f32(scales).astype(np.float64), 16, axis=1)
    n = W.shape[0]
    t = wr.reshape(n, -1).astype(np.float64) / np.repeat(dd.reshape(n, -1), 16, axis=1)
    gap = np.min(np.abs(t[..., None] - M32.astype(np.float64)), axis=-1)
    safe = same_d & (gap > 1e-5)
    assert safe.mean() > 0.99
    np.testing.assert_array_equal(idx[safe], idx64[safe])


def test_scale_is_fp16_of_half_rms():
    rng = np.random.default_rng(5)
    W = rng.standard_t(4, size=(16, 256)).astype(np.float32)
    _, scales = tq.quantize_o32(W)
    wr = tq.rotate_f64(W.reshape(16, 8, 32).astype(np.float64), tq.DEFAULT_SIGN_MASK).reshape(16, 8, 2, 16)
    rms = np.sqrt(np.mean(wr ** 2, axis=-1)).reshape(16, 16)
    got = tq.fp16_bits_to_f32(scales).astype(np.float64)
    np.testing.assert_allclose(got, rms, rtol=2 ** -10)


def test_zero_saturated_and_subnormal_scales():
    W = np.zeros((3, 64), np.float32)
    W[1, :32] = 1e6          # rms >> 65504 -> saturates
    W[2, 40] = 1e-6          # a spike: |w'| = fp32(1e-6 * s32), an fp16 subnormal
    packed, scales = tq.quantize_o32(W)
    assert np.all(scales[0] == 0)
    assert np.all(packed[0] == 0)
    assert np.all(scales[1, :2] == 0x7BFF)
    sub = scales[2, 2:]
    assert np.all((sub > 0) & (sub < 0x0400))        # fp16 subnormal bit patterns
    t = float(np.float32(np.float32(1e-6) * tq.S32))
    np.testing.assert_array_equal(sub, _nearest_fp16_bits([t, t]))
    Wd = tq.dequantize_o64(packed, scales)
    np.testing.assert_array_equal(Wd[0], 0.0)


def test_five_bits_per_weight_matches_page_size_figure():
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["size_reduction_vs_q8_0"]
    W = np.random.default_rng(6).normal(size=(4, 128)).astype(np.float32)
    packed, scales = tq.quantize_o32(W)
    bpw = 8.0 * (packed.nbytes + scales.nbytes) / W.size
    assert bpw == 5.0
    q8_0_bpw = 8.5                       # 32 int8 + one fp16 scale per 32 weights
    saving = 1 - bpw / q8_0_bpw
    assert fig["min"] <= saving <= fig["max"]


def test_reconstruction_error_near_codebook_distortion():
    d16 = cb.distortion(cb.lloyd_max_normal(16))
    W = np.random.default_rng(7).normal(size=(128, 1024)).astype(np.float32)
    packed, scales = tq.quantize_o32(W)
    Wd = tq.dequantize_o64(packed, scales)
    rel = np.mean((Wd - W) ** 2) / np.mean(W.astype(np.float64) ** 2)
    # per-half RMS scaling (not the true sigma) and fp16 d keep it near, slightly below, D16
    assert 0.75 * d16 < rel < 1.1 * d16


def test_gemv_one_hot_zero_and_m1():
    W, x = workloads.tiny_tq("cpu")
    packed, scales = tq.quantize_o32(W.numpy())
    Wd = tq.dequantize_o64(packed, scales)
    for j in (0, 17, 511):
        e = np.zeros(512)
        e[j] = 1.0
        y, a = tq.gemm_o64(packed, scales, e)
        np.testing.assert_array_equal(y[0], Wd[:, j])
    y1, _ = tq.gemm_o64(packed, scales, x.numpy())
    X = np.stack([x.numpy(), 2 * x.numpy()])
    y2, _ = tq.gemm_o64(packed, scales, X)
    np.testing.assert_allclose(y2[0], y1[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(y2[1], 2 * y1[0], rtol=1e-12, atol=1e-15)
    zp, zs = tq.quantize_o32(np.zeros((4, 64), np.float32))
    yz, _ = tq.gemm_o64(zp, zs, np.ones(64))
    np.testing.assert_array_equal(yz, 0.0)


def test_gemv_in_rotated_domain_equals_original():
    """y = sum_b d * c[idx] . (R x)_b — the identity the fused kernel relies on."""
    W, x = workloads.tiny_tq("cpu")
    packed, scales = tq.quantize_o32(W.numpy())
    y, _ = tq.gemm_o64(packed, scales, x.numpy())
    q = tq.rotated_weights_f64(packed, scales)
    xr = tq.rotate_f64(x.numpy().astype(np.float64).reshape(-1, 32), tq.DEFAULT_SIGN_MASK).reshape(-1)
    np.testing.assert_allclose(q @ xr, y[0], rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_bf16_input_is_taken_exactly():
    w = workloads.llama8b_weight("k", 0, "cpu", rows=4)
    assert w.dtype == torch.bfloat16
    f32 = w.float().numpy()
    p1, s1 = tq.quantize_o32(f32)
    p2, s2 = tq.quantize_o32(f32.astype(np.float64).astype(np.float32))
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(s1, s2)
