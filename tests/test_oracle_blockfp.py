"""Pins for the oracle's small-float encoders and the NVFP4 / MXFP6 block codecs (CPU only).

Independent anchors:
* a second rounding route (exponent/significand split + numpy.rint, which
  rounds half to even) run exhaustively over every finite bf16 value;
* torch's float8_e4m3fn cast (a separate library implementation);
* code points fixed by the format definitions (max finite, smallest
  subnormal, 1.0);
* hand-computed packing examples and closed-form block scales.
"""

import numpy as np
import pytest
import torch

from oracle import blockfp as bf
from oracle import minifloat as mf


def _all_finite_bf16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)].astype(np.float64)


def _rint_route(x, ebits, mbits, bias, maxval):
    """RNE by scaling to an integer significand and numpy.rint (half to even)."""
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, 1 - bias)                      # subnormals share the lowest exponent
    # guard the log2 floor against representation error
    e = np.where(a >= 2.0 ** (e + 1), e + 1, e)
    e = np.where(a < 2.0 ** e, np.maximum(e - 1, 1 - bias), e)
    step = 2.0 ** (e - mbits)
    r = np.rint(a / step) * step
    r = np.minimum(r, maxval)
    return np.where(np.signbit(x), -r, r)


@pytest.mark.parametrize("fmt,args", [
    (mf.E2M1, (2, 1, 1, 6.0)),
    (mf.E3M2, (3, 2, 3, 28.0)),
    (mf.E4M3FN, (4, 3, 7, 448.0)),
])
def test_encoder_exhaustive_over_bf16(fmt, args):
    x = _all_finite_bf16()
    got = fmt.decode(fmt.encode(x))
    ref = _rint_route(x, *args)
    np.testing.assert_array_equal(got, ref)
    # the sign bit follows the input, including -0 and negatives that round to 0
    np.testing.assert_array_equal(np.signbit(got), np.signbit(x))


def test_e4m3_against_torch_float8():
    x = _all_finite_bf16()
    x = x[np.abs(x) <= 448.0]
    ours = mf.E4M3FN.encode(x)
    theirs = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_code_points():
    assert mf.E2M1.encode([6.0, 0.5, 1.0, -6.0, 7.0, 0.25, 0.75])[:].tolist() == [7, 1, 2, 15, 7, 0, 2]
    assert mf.E4M3FN.encode([448.0, 1.0, 2.0 ** -9, 500.0]).tolist() == [0x7E, 0x38, 0x01, 0x7E]
    assert mf.E3M2.encode([28.0, 0.0625, 1.0, 0.25, 100.0]).tolist() == [0x1F, 0x01, 0x0C, 0x04, 0x1F]
    assert mf.E2M1.decode(np.arange(16)).tolist() == [0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6]
    np.testing.assert_array_equal(mf.e8m0_decode([127, 0, 254]), [1.0, 2.0 ** -127, 2.0 ** 127])
    assert np.isnan(mf.e8m0_decode([255])[0])
    assert np.isnan(mf.E4M3FN.decode([0x7F])[0])


def test_pack6_hand_example():
    codes = np.array([[1, 2, 3, 4, 63, 0, 0, 63]], dtype=np.uint8)
    packed = bf.pack6(codes)
    # word0 = 1 | 2<<6 | 3<<12 | 4<<18 = 0x103081; word1 = 63 | 63<<18 = 0xFC003F
    assert packed.tolist() == [[0x81, 0x30, 0x10, 0x3F, 0x00, 0xFC]]
    np.testing.assert_array_equal(bf.unpack6(packed), codes)


def test_nvfp4_closed_form_scales():
    W = np.zeros((2, 32), np.float32)
    W[0, :16] = np.linspace(-1, 1, 16)
    W[0, 5] = 3.0                       # tensor amax
    W[1, 16:] = 0.75                    # a flat block
    codes, sb, st = bf.nvfp4_quantize_o32(W)
    assert st == np.float32(np.float32(3.0) / np.float32(2688.0))
    assert sb[0, 0] == 0x7E             # the amax block gets the largest scale, 448
    assert sb[0, 1] == 0 and sb[1, 0] == 0
    lo = codes[0, 2] & 0x0F             # element 4 -> byte 2 low nibble
    hi = codes[0, 2] >> 4               # element 5 -> byte 2 high nibble
    assert hi == 0x7                    # 3.0 / (448 * s_t) = 6.0 exactly -> E2M1 max
    assert lo == mf.E2M1.encode([float(np.float32(np.float32(W[0, 4]) / np.float32(mf.E4M3FN.decode([0x7E])[0] * st)))])[0]
    Wd = bf.nvfp4_dequantize_o64(codes, sb, st)
    assert Wd[0, 5] == pytest.approx(3.0, rel=1e-7)
    # the flat block: all equal values -> all equal codes, value recovered to the E4M3 step
    flat = Wd[1, 16:]
    assert np.all(flat == flat[0]) and flat[0] == pytest.approx(0.75, rel=0.07)


def test_nvfp4_all_zero_tensor():
    codes, sb, st = bf.nvfp4_quantize_o32(np.zeros((3, 32), np.float32))
    assert st == 0 and not codes.any() and not sb.any()


def test_mxfp6_closed_form_scale():
    W = np.zeros((1, 64), np.float32)
    W[0, :32] = np.linspace(-1.0, 1.0, 32)      # amax 1 -> e = -4 -> byte 123, values x16
    W[0, 40] = -0.3                              # amax 0.3 -> floor(log2 .3) = -2 -> e = -6
    codes, sc = bf.mxfp6_quantize_o32(W)
    assert sc.tolist() == [[123, 121]]
    c = bf.unpack6(codes)[0]
    assert c[31] == mf.E3M2.encode([16.0])[0] and c[0] == mf.E3M2.encode([-16.0])[0]
    Wd = bf.mxfp6_dequantize_o64(codes, sc)
    assert Wd[0, 40] == pytest.approx(-0.3, rel=1 / 16)
    assert Wd[0, 41] == 0.0


def test_blockfp_reconstruction_error_scale():
    rng = np.random.default_rng(0)
    W = (rng.normal(size=(64, 512)) / np.sqrt(512)).astype(np.float32)
    c, s, st = bf.nvfp4_quantize_o32(W)
    e4 = np.mean((bf.nvfp4_dequantize_o64(c, s, st) - W) ** 2) / np.mean(W.astype(np.float64) ** 2)
    c6, s6 = bf.mxfp6_quantize_o32(W)
    e6 = np.mean((bf.mxfp6_dequantize_o64(c6, s6) - W) ** 2) / np.mean(W.astype(np.float64) ** 2)
    assert 0.005 < e4 < 0.02          # 4-bit float with E4M3 block scales
    assert e6 < e4 / 2                # 6 bits: two more mantissa/exponent bits
    assert bf.bytes_per_weight("nvfp4") == 0.5625 and bf.bytes_per_weight("mxfp6") == 0.78125


# ----------------------------------------------------------------------------
# gemm_deq_o64: the float64 product that judges every NVFP4 / MXFP6 GEMV/GEMM
# (quantizer-tool page, "目前能实现的部分功能": the weights are stored in these
# formats and multiplied as their dequantized values).  Pinned by special
# cases that do not restate its formula: one-hot activations select columns,
# rows scale linearly, zero weights give zero, and a tiny explicit loop.
# ----------------------------------------------------------------------------

def _bf_weights(fmt, n, k, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)
    W[0, 3] = 4.0 / np.sqrt(k)                                 # one outlier so the block scales differ
    if fmt == "nvfp4":
        c, s, st = bf.nvfp4_quantize_o32(W)
        return bf.nvfp4_dequantize_o64(c, s, st)
    c, s = bf.mxfp6_quantize_o32(W)
    return bf.mxfp6_dequantize_o64(c, s)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_gemm_deq_one_hot_selects_columns(fmt):
    n, k = 24, 96                                               # non-square: a transposed product cannot pass
    Wd = _bf_weights(fmt, n, k, 1)
    cols = [0, 5, 31, 64, 95]
    X = np.zeros((len(cols), k))
    for m, j in enumerate(cols):
        X[m, j] = 1.0
    Y, A = bf.gemm_deq_o64(Wd, X)
    assert Y.shape == (len(cols), n) and A.shape == (len(cols), n)
    for m, j in enumerate(cols):
        np.testing.assert_array_equal(Y[m], Wd[:, j])           # exact: one product per output
        np.testing.assert_array_equal(A[m], np.abs(Wd[:, j]))   # the tolerance scale keeps the magnitude


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_gemm_deq_rows_scale_and_m1(fmt):
    n, k = 40, 64
    Wd = _bf_weights(fmt, n, k, 2)
    x = np.random.default_rng(3).standard_normal(k)
    y1, a1 = bf.gemm_deq_o64(Wd, x)                              # a vector is one activation row
    assert y1.shape == (1, n)
    Y2, A2 = bf.gemm_deq_o64(Wd, np.stack([x, 2.0 * x, -x]))
    tol = 1e-13 * a1[0]                                         # BLAS may sum one row and three rows in different orders
    np.testing.assert_allclose(Y2[0], y1[0], rtol=0, atol=tol.max())
    np.testing.assert_allclose(Y2[1], 2.0 * y1[0], rtol=0, atol=2 * tol.max())
    np.testing.assert_allclose(Y2[2], -y1[0], rtol=0, atol=tol.max())
    np.testing.assert_allclose(A2[2], a1[0], rtol=1e-13)        # |-x| = |x|
    np.testing.assert_allclose(A2[1], 2.0 * a1[0], rtol=1e-13)


def test_gemm_deq_zero_weights_and_scale_bounds():
    c, s, st = bf.nvfp4_quantize_o32(np.zeros((6, 32), np.float32))
    Wz = bf.nvfp4_dequantize_o64(c, s, st)
    Y, A = bf.gemm_deq_o64(Wz, np.random.default_rng(4).standard_normal((3, 32)))
    assert not Y.any() and not A.any()
    Wd = _bf_weights("mxfp6", 16, 64, 5)
    X = np.random.default_rng(6).standard_normal((4, 64))
    Y, A = bf.gemm_deq_o64(Wd, X)
    assert np.all(A >= np.abs(Y))                               # triangle inequality
    assert np.any(A > np.abs(Y) * (1 + 1e-6))                   # mixed signs cancel in Y, not in A
    Yp, Ap = bf.gemm_deq_o64(np.abs(Wd), np.abs(X))
    np.testing.assert_allclose(Ap, Yp, rtol=1e-15)              # nonnegative operands: A equals Y


def test_gemm_deq_tiny_explicit_loop():
    Wd = _bf_weights("nvfp4", 3, 32, 7)
    X = np.random.default_rng(8).standard_normal((2, 32))
    Y, A = bf.gemm_deq_o64(Wd, X)
    import math
    for m in range(2):
        for nn in range(3):
            terms = [float(X[m, kk]) * float(Wd[nn, kk]) for kk in range(32)]
            assert Y[m, nn] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-15)
            assert A[m, nn] == pytest.approx(math.fsum(abs(t) for t in terms), rel=1e-13)
