"""GPU parity of the NVFP4 / MXFP6 path against the CPU oracle (through the C ABI):
codes, block scales and the tensor scale bit-exact; decode GEMV/GEMM within
|dy| <= 1e-3 * sum |W_deq x|."""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa
from oracle import blockfp as obf
import workloads
from gpu_helpers import say, f32np, assert_within

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(fmt, W):
    say(f"[{fmt} quantize] shape={tuple(W.shape)} dtype={W.dtype}")
    codes, bs, ts = tqa.blockfp_quantize(fmt, W)
    torch.cuda.synchronize()
    Wh = W.float().cpu().numpy()
    if fmt == "nvfp4":
        oc, osb, ost = obf.nvfp4_quantize_o32(Wh)
        assert np.float32(ts.cpu().numpy()[0]).view(np.uint32) == np.float32(ost).view(np.uint32)
        Wd = obf.nvfp4_dequantize_o64(oc, osb, ost)
    else:
        oc, osb = obf.mxfp6_quantize_o32(Wh)
        Wd = obf.mxfp6_dequantize_o64(oc, osb)
    np.testing.assert_array_equal(bs.cpu().numpy(), osb, err_msg=f"{fmt} block scales")
    np.testing.assert_array_equal(codes.cpu().numpy(), oc, err_msg=f"{fmt} codes")
    return codes, bs, ts, Wd


def _outlier_weight(n, k, seed, dtype):
    g = workloads.generator(seed, DEV)
    w = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.float32)
    return workloads.add_outliers(w, 0.001, 20.0, g).to(dtype)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
@pytest.mark.parametrize("n,k,dt", [(1, 32, torch.float32), (13, 512, torch.bfloat16), (64, 5120, torch.bfloat16),
                                    (7, 17408, torch.bfloat16), (33, 96, torch.float32)])
def test_blockfp_quantize_bit_exact(fmt, n, k, dt):
    _check(fmt, _outlier_weight(n, k, n * 31 + k, dt))


def test_nvfp4_quotients_near_rounding_boundaries():
    """Enough blocks that tens of scaled quotients |w| / eff * 2^(1 - e) fall within 1e-5 of a half-integer,
    where the E2M1 code depends on the last bits of the quotient; all codes bit-exact."""
    W = _outlier_weight(2048, 1024, 4242, torch.float32)
    Wh = W.cpu().numpy()
    oc, osb, ost = obf.nvfp4_quantize_o32(Wh)
    eff = (obf.E4M3FN.decode(osb).astype(np.float32) * np.float32(ost)).astype(np.float32)
    q = (np.abs(Wh).reshape(2048, 64, 16) / eff[..., None]).astype(np.float32)
    with np.errstate(divide="ignore"):
        e = np.maximum(np.floor(np.log2(np.where(q > 0, q, 1))), 0)
    sc = (q * np.exp2(1 - e)).astype(np.float32)
    near = int(((np.abs(np.abs(sc - np.rint(sc)) - 0.5) < 1e-5) & (q < 8)).sum())
    say(f"[nvfp4] {near} scaled quotients within 1e-5 of a half-integer")
    assert near >= 20
    _check("nvfp4", W)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_blockfp_edge_values(fmt):
    W = torch.zeros(6, 64)
    W[1, :] = -0.0
    W[2, 3] = 1e-40                       # subnormal amax
    W[3, :32] = torch.linspace(-1, 1, 32)
    W[3, 40] = 3e4                        # huge tensor amax
    W[4, :] = 2.0 ** -126
    W[5, ::2] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4)   # E2M1 midpoints
    _check(fmt, W.to(DEV))
    _check(fmt, torch.zeros(3, 32, device=DEV))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
@pytest.mark.parametrize("m", [1, 2, 3, 8, 16])
def test_blockfp_gemm(fmt, m):
    n, k = 96, 5120
    W = _outlier_weight(n, k, 500 + m, torch.bfloat16)
    codes, bs, ts, Wd = _check(fmt, W)
    g = workloads.generator(900 + m, DEV)
    X = workloads.activation(m, k, g, DEV, torch.bfloat16)
    say(f"[{fmt} gemm] M={m}")
    Y = tqa.blockfp_gemm(fmt, codes, bs, ts, X)
    yr, a = obf.gemm_deq_o64(Wd, X.float().cpu().numpy())
    worst = assert_within(f32np(Y), yr, a, what=f"{fmt} M={m}")
    assert worst < 1e-4
    if m == 1:
        y1 = tqa.blockfp_gemm(fmt, codes, bs, ts, X[0].contiguous())
        assert torch.equal(y1, Y[0])


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
@pytest.mark.parametrize("m", [3, 4, 5, 8, 17, 32, 33, 64, 65, 100])
def test_blockfp_gemm_mfma(fmt, m):
    """bf16 activations with M >= 3 take the MFMA kernel: exact bf16 weight operands, float32 sums (relative
    error far below the bound).  Shapes: several passes over K (5120, 17408), one pass in which half the
    wavefronts take a single group (3072), a partial group of four blocks (K = 96, 32), ragged row tiles."""
    for n, k in ((300, 5120), (37, 96), (130, 32), (64, 17408), (200, 3072)):
        W = _outlier_weight(n, k, 700 + m + k, torch.bfloat16)
        codes, bs, ts, Wd = _check(fmt, W)
        X = workloads.activation(m, k, workloads.generator(910 + m + k, DEV), DEV, torch.bfloat16)
        say(f"[{fmt} gemm mfma] M={m} {n}x{k}")
        Y = tqa.blockfp_gemm(fmt, codes, bs, ts, X)
        torch.cuda.synchronize()
        yr, a = obf.gemm_deq_o64(Wd, X.float().cpu().numpy())
        worst = assert_within(f32np(Y), yr, a, what=f"{fmt} mfma M={m} {n}x{k}")
        assert worst < 1e-4


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_blockfp_gemm_fp32_many_rows(fmt):
    """float32 activations at any M stay on the VALU kernel (rows in chunks)."""
    n, k, m = 70, 1024, 21
    W = _outlier_weight(n, k, 811, torch.bfloat16)
    codes, bs, ts, Wd = _check(fmt, W)
    X = workloads.activation(m, k, workloads.generator(812, DEV), DEV, torch.float32)
    say(f"[{fmt} gemm fp32] M={m}")
    Y = tqa.blockfp_gemm(fmt, codes, bs, ts, X)
    torch.cuda.synchronize()
    yr, a = obf.gemm_deq_o64(Wd, X.cpu().numpy())
    assert assert_within(f32np(Y), yr, a, what=f"{fmt} fp32 M={m}") < 1e-4


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
@pytest.mark.parametrize("m", [2, 16, 64])
def test_blockfp_gemm_padded_row_strides(fmt, m):
    """Block-float products through activation and output row strides above K and N (VALU rows at M = 2,
    the MFMA kernel with K split over workgroups at K = 8192 above); the output's padding stays untouched."""
    n, k = 80, 8192
    W = _outlier_weight(n, k, 1200 + m, torch.bfloat16)
    codes, bs, ts, Wd = _check(fmt, W)
    X = workloads.activation(m, k, workloads.generator(1300 + m, DEV), DEV, torch.bfloat16)
    x_full = torch.zeros((m, k + 64), dtype=torch.bfloat16, device=DEV)
    x = x_full[:, :k]
    x.copy_(X)
    y_full = torch.full((m, n + 24), -7.0, dtype=torch.float32, device=DEV)
    y = y_full[:, :n]
    say(f"[{fmt} gemm] padded strides M={m} ldx={x.stride(0)} ldy={y.stride(0)}")
    tqa.blockfp_gemm(fmt, codes, bs, ts, x, out=y)
    torch.cuda.synchronize()
    assert torch.all(y_full[:, n:] == -7.0)
    yr, a = obf.gemm_deq_o64(Wd, X.float().cpu().numpy())
    assert assert_within(f32np(y), yr, a, what=f"{fmt} padded M={m}") < 1e-4
