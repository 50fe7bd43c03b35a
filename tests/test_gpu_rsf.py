"""GPU parity of the RSF-lite quantizers (tq_quantize_rsf, tq_blockfp_quantize_rsf) against the CPU oracle.

Packed nibbles and fp16 scales bit-exact against oracle.rsf (ragged shapes,
fp32 and bf16 input, sign masks, edge rows), the result decodes with every
other call, and the search lowers the reconstruction error; the same for the
NVFP4 and MXFP6 block-scale search (codes, block scales and tensor scale
bit-exact, output read by the block-float GEMV).
"""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa
from oracle import rsf as orsf
from oracle import tq4_1s as otq
import workloads
from gpu_helpers import say, u16, f32np, assert_within, edge_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(W, label, mask=otq.DEFAULT_SIGN_MASK):
    say(f"[quantize_rsf] {label} shape={tuple(W.shape)} dtype={W.dtype} mask={mask:#x}")
    packed, scales = tqa.quantize(W, sign_mask=mask, rsf=True)
    torch.cuda.synchronize()
    op, osc = orsf.quantize_rsf_o32(W.float().cpu().numpy(), mask)
    np.testing.assert_array_equal(u16(scales), osc, err_msg=f"scales {label}")
    np.testing.assert_array_equal(packed.cpu().numpy(), op, err_msg=f"packed {label}")
    return packed, scales


@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (257, 512), (64, 4096), (9, 14336), (5, 5120)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rsf_bit_exact_shapes(n, k, dtype):
    g = workloads.generator(3000 + n + k, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, dtype)
    _check(W, f"{n}x{k}")


def test_rsf_masks_heavy_tails_and_edge_rows():
    g = workloads.generator(3100, DEV)
    W = workloads.student_t4_weight(64, 1024, g, DEV, torch.bfloat16)
    for mask in (0, 0xFFFFFFFF, otq.sign_mask_from_seed(5)):
        _check(W, "t4", mask)
    _check(torch.from_numpy(edge_rows(512)).to(DEV), "edge rows")


def test_rsf_output_decodes_and_lowers_error():
    g = workloads.generator(3200, DEV)
    W = workloads.normal_weight(512, 4096, 4096 ** -0.5, g, DEV, torch.bfloat16)
    p0, s0 = tqa.quantize(W)
    p1, s1 = tqa.quantize(W, rsf=True)
    Wf = W.float()
    e0 = (tqa.dequantize(p0, s0) - Wf).pow(2).sum().item()
    e1 = (tqa.dequantize(p1, s1) - Wf).pow(2).sum().item()
    say(f"[quantize_rsf] squared error plain {e0:.4e} rsf {e1:.4e} ({100 * (1 - e1 / e0):.1f}% less)")
    assert e1 < 0.8 * e0
    x = workloads.activation(1, 4096, workloads.generator(3201, DEV), DEV, torch.bfloat16)[0].contiguous()
    y = tqa.gemv(p1, s1, x)
    torch.cuda.synchronize()
    rows = np.arange(0, 512, 7)
    yr, a = otq.gemv_rows_o64(p1.cpu().numpy()[rows], u16(s1)[rows], f32np(x))
    assert_within(f32np(y)[rows], yr, a, 1e-3, "gemv on rsf weights")


# ---------------------------------------------------------------------------
# NVFP4 / MXFP6 block-scale search (tq_blockfp_quantize_rsf)
# ---------------------------------------------------------------------------

from oracle import blockfp as obf  # noqa: E402


def _check_blockfp(fmt, W, label):
    say(f"[{fmt} quantize_rsf] {label} shape={tuple(W.shape)} dtype={W.dtype}")
    codes, bs, ts = tqa.blockfp_quantize(fmt, W, rsf=True)
    torch.cuda.synchronize()
    Wh = W.float().cpu().numpy()
    if fmt == "nvfp4":
        oc, osb, ost = orsf.nvfp4_quantize_rsf_o32(Wh)
        assert np.float32(ts.cpu().numpy()[0]).view(np.uint32) == np.float32(ost).view(np.uint32)
    else:
        oc, osb = orsf.mxfp6_quantize_rsf_o32(Wh)
    np.testing.assert_array_equal(bs.cpu().numpy(), osb, err_msg=f"{fmt} block scales {label}")
    np.testing.assert_array_equal(codes.cpu().numpy(), oc, err_msg=f"{fmt} codes {label}")
    return codes, bs, ts


def _outlier_weight(n, k, seed, dtype):
    g = workloads.generator(seed, DEV)
    w = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.float32)
    return workloads.add_outliers(w, 0.001, 20.0, g).to(dtype)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
@pytest.mark.parametrize("n,k,dt", [(1, 32, torch.float32), (13, 512, torch.bfloat16), (64, 5120, torch.bfloat16),
                                    (7, 17408, torch.bfloat16), (33, 96, torch.float32)])
def test_blockfp_rsf_bit_exact(fmt, n, k, dt):
    _check_blockfp(fmt, _outlier_weight(n, k, 4000 + n * 31 + k, dt), f"{n}x{k}")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_blockfp_rsf_edge_values_and_heavy_tails(fmt):
    W = torch.zeros(7, 64)
    W[1, :] = -0.0
    W[2, 3] = 1e-40                       # subnormal amax
    W[3, :32] = torch.linspace(-1, 1, 32)
    W[3, 40] = 3e4                        # huge tensor amax
    W[4, :] = 2.0 ** -126
    W[5, ::2] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4)
    W[6, 5] = 31.5                        # clipped at the plain MXFP6 exponent
    _check_blockfp(fmt, W.to(DEV), "edge rows")
    _check_blockfp(fmt, torch.zeros(3, 32, device=DEV), "zeros")
    g = workloads.generator(4100, DEV)
    _check_blockfp(fmt, workloads.student_t4_weight(48, 1024, g, DEV, torch.bfloat16), "t4")


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_blockfp_rsf_lowers_error_and_feeds_the_gemv(fmt):
    n, k = 256, 5120
    W = _outlier_weight(n, k, 4200, torch.bfloat16)
    Wh = W.float().cpu().numpy().astype(np.float64)
    c0, b0, t0 = tqa.blockfp_quantize(fmt, W)
    c1, b1, t1 = _check_blockfp(fmt, W, "error")
    if fmt == "nvfp4":
        d0 = obf.nvfp4_dequantize_o64(c0.cpu().numpy(), b0.cpu().numpy(), t0.cpu().numpy()[0])
        d1 = obf.nvfp4_dequantize_o64(c1.cpu().numpy(), b1.cpu().numpy(), t1.cpu().numpy()[0])
    else:
        d0 = obf.mxfp6_dequantize_o64(c0.cpu().numpy(), b0.cpu().numpy())
        d1 = obf.mxfp6_dequantize_o64(c1.cpu().numpy(), b1.cpu().numpy())
    e0, e1 = ((d0 - Wh) ** 2).sum(), ((d1 - Wh) ** 2).sum()
    say(f"[{fmt} quantize_rsf] squared error plain {e0:.4e} rsf {e1:.4e} ({100 * (1 - e1 / e0):.1f}% less)")
    assert e1 < e0
    X = workloads.activation(8, k, workloads.generator(4201, DEV), DEV, torch.bfloat16)
    Y = tqa.blockfp_gemm(fmt, c1, b1, t1, X)
    torch.cuda.synchronize()
    yr, a = obf.gemm_deq_o64(d1, X.float().cpu().numpy())
    assert assert_within(f32np(Y), yr, a, what=f"{fmt} gemm on rsf weights") < 1e-4
