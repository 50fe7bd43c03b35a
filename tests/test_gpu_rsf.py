"""GPU parity of the RSF-lite TQ4_1S quantizer (tq_quantize_rsf) against the CPU oracle.

Packed nibbles and fp16 scales bit-exact against oracle.rsf (ragged shapes,
fp32 and bf16 input, sign masks, edge rows), the result decodes with every
other call, and the search lowers the reconstruction error.
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
