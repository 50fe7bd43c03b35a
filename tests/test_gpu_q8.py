"""GPU parity of the load-time int8 transcode and the int8 GEMV against the CPU oracle (through the C ABI).

* transcode: int8 codes and fp16 block scales bit-exact against the oracle's
  canonical float32 order (ragged shapes, sign masks, edge rows: zeros,
  saturated and subnormal TQ4_1S scales, single spikes);
* q8 GEMV: |dy| <= 1e-3 * sum_b |d dx| sum_i |code_w code_x| against the
  oracle's integer block sums (activation quantized the same way), bf16 and
  float32 activations, one-hot and zero activations, K up to 32768, and the
  full-size decode shapes on sampled rows.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa
from oracle import q8 as oq8
from oracle import tq4_1s as otq
import workloads
from gpu_helpers import say, u16, f32np, assert_within, edge_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _tq4(n, k, seed, dtype=torch.bfloat16, mask=otq.DEFAULT_SIGN_MASK):
    g = workloads.generator(seed, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, dtype)
    return tqa.quantize(W, sign_mask=mask)


def _transcode_check(packed, scales, mask, label):
    say(f"[transcode] {label} N={packed.shape[0]} K={packed.shape[1] * 2} mask={mask:#x}")
    codes, qs = tqa.transcode_q8(packed, scales, sign_mask=mask)
    torch.cuda.synchronize()
    oc, os_ = oq8.transcode_q8_o32(packed.cpu().numpy(), u16(scales), mask)
    np.testing.assert_array_equal(u16(qs), os_, err_msg=f"scales {label}")
    np.testing.assert_array_equal(codes.cpu().numpy(), oc, err_msg=f"codes {label}")
    return codes, qs


@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (257, 512), (64, 4096), (17, 14336), (5, 5120), (2, 28672)])
def test_transcode_bit_exact_shapes(n, k):
    packed, scales = _tq4(n, k, 100 + n * 31 + k)
    _transcode_check(packed, scales, otq.DEFAULT_SIGN_MASK, f"{n}x{k}")


def test_transcode_sign_masks_and_edge_rows():
    for mask in (0, 0xFFFFFFFF, otq.sign_mask_from_seed(9)):
        packed, scales = _tq4(40, 1024, 7, torch.float32, mask)
        _transcode_check(packed, scales, mask, "random")
    W = torch.from_numpy(edge_rows(256)).to(DEV)
    packed, scales = tqa.quantize(W)
    _transcode_check(packed, scales, otq.DEFAULT_SIGN_MASK, "edge rows")
    # hand-made TQ4_1S data: every byte value, every scale class
    rng = np.random.default_rng(3)
    p = torch.from_numpy(rng.integers(0, 256, (64, 256), dtype=np.uint8)).to(DEV)
    sbits = rng.choice(np.array([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x2E66, 0x1234], np.uint16), (64, 32))
    s = torch.from_numpy(sbits.view(np.int16)).to(DEV)
    _transcode_check(p, s, otq.DEFAULT_SIGN_MASK, "all bytes, scale classes")


def test_transcode_quotients_near_half_integers():
    """Many blocks, so that a few hundred quotients w / dd fall within 1e-4 of a half-integer (a few exactly
    on one: ties to even), where the code depends on the last bits of the quotient; all codes bit-exact."""
    rng = np.random.default_rng(11)
    n, k = 2048, 1024
    pk = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    sbits = np.float16(rng.uniform(0.005, 2.0, (n, k // 16))).view(np.uint16)
    w = oq8.dequantize_o32_blocks(pk, sbits, otq.DEFAULT_SIGN_MASK)
    dd = otq.fp16_sat((np.abs(w).max(axis=-1) / np.float32(127)).astype(np.float32)).astype(np.float32)
    q = (w / dd[..., None]).astype(np.float32)
    frac = np.abs(q - np.rint(q))
    near, ties = int((np.abs(frac - np.float32(0.5)) < 1e-4).sum()), int((frac == 0.5).sum())
    say(f"[transcode] {near} quotients within 1e-4 of a half-integer, {ties} exactly on one")
    assert near >= 50 and ties >= 1
    _transcode_check(torch.from_numpy(pk).to(DEV), torch.from_numpy(sbits.view(np.int16)).to(DEV),
                     otq.DEFAULT_SIGN_MASK, "near half-integers")


def _gemv_check(codes, qs, x, label):
    say(f"[q8_gemv] {label} N={codes.shape[0]} K={codes.shape[1]} x={x.dtype}")
    y = tqa.q8_gemv(codes, qs, x)
    torch.cuda.synchronize()
    yr, a = oq8.q8_gemv_o64(codes.cpu().numpy(), u16(qs), f32np(x))
    return assert_within(f32np(y), yr, a, 1e-3, label)


@pytest.mark.parametrize("n,k", [(1, 32), (7, 64), (300, 1024), (128, 4096), (33, 14336), (9, 32768), (1000, 96)])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float32])
def test_q8_gemv_shapes(n, k, xdtype):
    packed, scales = _tq4(n, k, 500 + n + k)
    codes, qs = tqa.transcode_q8(packed, scales)
    x = workloads.activation(1, k, workloads.generator(600 + k, DEV), DEV, xdtype)[0].contiguous()
    _gemv_check(codes, qs, x, f"{n}x{k}")


def test_q8_gemv_one_hot_and_zero():
    packed, scales = _tq4(96, 2048, 42)
    codes, qs = tqa.transcode_q8(packed, scales)
    for j in (0, 31, 1000, 2047):
        x = torch.zeros(2048, device=DEV, dtype=torch.float32)
        x[j] = -1.75
        y = tqa.q8_gemv(codes, qs, x)
        torch.cuda.synchronize()
        # one-hot: x quantizes to -127 at j with dx = 1.75 / 127, so y = d * code[:, j] * (-1.75) up to rounding
        yr, a = oq8.q8_gemv_o64(codes.cpu().numpy(), u16(qs), f32np(x))
        assert_within(f32np(y), yr, a, 1e-3, f"one-hot {j}")
    y = tqa.q8_gemv(codes, qs, torch.zeros(2048, device=DEV, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0


def test_q8_repeat_runs_are_bit_identical():
    packed, scales = _tq4(4096, 4096, 77)
    codes, qs = tqa.transcode_q8(packed, scales)
    x = workloads.activation(1, 4096, workloads.generator(78, DEV), DEV, torch.bfloat16)[0].contiguous()
    y0 = tqa.q8_gemv(codes, qs, x).clone()
    for _ in range(3):
        y1 = tqa.q8_gemv(codes, qs, x)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


@pytest.mark.parametrize("name,n,k", [("q|k|v 8B", 6144, 4096), ("gate|up 8B", 28672, 4096), ("down 8B", 4096, 14336),
                                      ("down 70B", 8192, 28672)])
def test_q8_full_size_sampled_rows(name, n, k):
    """Full decode shapes in the benchmarked configuration: transcode bit-exact and GEMV on sampled rows."""
    packed, scales = _tq4(n, k, 900 + n % 97 + k % 89)
    codes, qs = tqa.transcode_q8(packed, scales)
    x = workloads.activation(1, k, workloads.generator(901, DEV), DEV, torch.bfloat16)[0].contiguous()
    y = tqa.q8_gemv(codes, qs, x)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(4), n - 4 + np.arange(4),
                                     np.random.default_rng(n + k).integers(0, n, 56)]))
    say(f"[q8 full] {name} {n}x{k}: {len(rows)} sampled rows")
    pk = packed.cpu().numpy()[rows]
    sc = u16(scales)[rows]
    oc, os_ = oq8.transcode_q8_o32(pk, sc, otq.DEFAULT_SIGN_MASK)
    np.testing.assert_array_equal(codes.cpu().numpy()[rows], oc)
    np.testing.assert_array_equal(u16(qs)[rows], os_)
    yr, a = oq8.q8_gemv_o64(oc, os_, f32np(x))
    assert_within(f32np(y)[rows], yr, a, 1e-3, name)
