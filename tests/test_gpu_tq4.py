"""GPU parity of the TQ4_1S path against the CPU oracle (through the C ABI).

* quantize: packed nibbles and fp16 scales bit-exact (fp32 and bf16 input,
  padded row strides, ragged shapes, edge rows, constructed exact ties);
* rotate: float32 output bit-exact (same butterfly order), bf16 = RNE of it;
* dequantize: within float32 rounding of the float64 definition;
* gemv / gemm: |dy| <= 1e-3 * sum_k |W_deq[n,k] x[k]| on the GPU's own
  packed weights (the stated parity bound), for rotated and raw activations.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa
from oracle import tq4_1s as otq
import workloads
from gpu_helpers import say, u16, f32np, assert_within, edge_rows, tie_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _quant_check(W: torch.Tensor, label: str):
    say(f"[quantize] {label} shape={tuple(W.shape)} dtype={W.dtype}")
    packed, scales = tqa.quantize(W)
    torch.cuda.synchronize()
    Wh = W.float().cpu().numpy()
    op, osc = otq.quantize_o32(Wh)
    gp = packed.cpu().numpy()
    gs = u16(scales)
    np.testing.assert_array_equal(gs, osc, err_msg=f"scales {label}")
    np.testing.assert_array_equal(gp, op, err_msg=f"packed {label}")
    return packed, scales


def test_quantize_tiny_fp32():
    W, _ = workloads.tiny_tq(DEV)
    _quant_check(W, "tiny fp32 256x512")


@pytest.mark.parametrize("n,k", [(1, 32), (3, 64), (257, 512), (64, 4096), (17, 14336), (5, 5120)])
@pytest.mark.parametrize("variant", ["gauss", "t4"])
def test_quantize_bf16_shapes(n, k, variant):
    g = workloads.generator(n * 7919 + k, DEV)
    if variant == "t4":
        W = workloads.student_t4_weight(n, k, g, DEV, torch.bfloat16)
    else:
        W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    _quant_check(W, f"{variant} {n}x{k}")


def test_quantize_padded_stride_and_sign_masks():
    g = workloads.generator(11, DEV)
    big = torch.randn(33, 160, generator=g, device=DEV)
    W = big[:, :128]
    assert W.stride(0) == 160
    for mask in (0, 0xFFFFFFFF, otq.sign_mask_from_seed(7)):
        say(f"[quantize] padded stride mask={mask:#x}")
        packed, scales = tqa.quantize(W, sign_mask=mask)
        op, osc = otq.quantize_o32(W.cpu().numpy(), mask)
        np.testing.assert_array_equal(u16(scales), osc)
        np.testing.assert_array_equal(packed.cpu().numpy(), op)


def test_quantize_edge_rows():
    W = torch.from_numpy(edge_rows(96)).to(DEV)
    _quant_check(W, "edge rows")


def test_quantize_exact_threshold_ties():
    rows = tie_rows(K=64, want=10)
    _quant_check(torch.from_numpy(rows).to(DEV), "exact ties")


def test_rotate_bit_exact():
    for dt in (torch.float32, torch.bfloat16):
        g = workloads.generator(5, DEV)
        x = workloads.activation(7, 4096, g, DEV, dt)
        say(f"[rotate] 7x4096 {dt}")
        xr = tqa.rotate(x)
        ref = otq.rotate_f32(x.float().cpu().numpy().reshape(7, -1, 32), otq.DEFAULT_SIGN_MASK).reshape(7, -1)
        np.testing.assert_array_equal(xr.cpu().numpy(), ref)
        xb = tqa.rotate(x, dtype=torch.bfloat16)
        np.testing.assert_array_equal(xb.cpu().float().numpy(), torch.from_numpy(ref).bfloat16().float().numpy())


def test_dequantize_matches_definition():
    W, _ = workloads.tiny_tq(DEV)
    packed, scales = tqa.quantize(W)
    say("[dequantize] tiny fp32 + bf16 out")
    Wd = tqa.dequantize(packed, scales)
    ref = otq.dequantize_o64(packed.cpu().numpy(), u16(scales))
    q = otq.rotated_weights_f64(packed.cpu().numpy(), u16(scales))
    n = q.shape[0]
    bound = 4e-7 * np.repeat(np.abs(q).reshape(n, -1, 32).sum(-1), 32, axis=1) + 1e-30
    assert np.all(np.abs(f32np(Wd) - ref) <= bound)
    Wb = tqa.dequantize(packed, scales, dtype=torch.bfloat16)
    np.testing.assert_array_equal(Wb.cpu().float().numpy(), Wd.cpu().bfloat16().float().numpy())


def _gemv_case(n, k, xdtype, rotated, seed):
    g = workloads.generator(seed, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    x = workloads.activation(1, k, g, DEV, xdtype)[0].contiguous()
    packed, scales = tqa.quantize(W)
    say(f"[gemv] {n}x{k} x={xdtype} rotated={rotated}")
    if rotated:
        y = tqa.gemv(packed, scales, tqa.rotate(x), rotated=True)
    else:
        y = tqa.gemv(packed, scales, x)
    yr, a = otq.gemv_rows_o64(packed.cpu().numpy(), u16(scales), x.float().cpu().numpy())
    return assert_within(f32np(y), yr, a, what=f"gemv {n}x{k}")


@pytest.mark.parametrize("n,k", [(1, 32), (7, 512), (256, 4096), (33, 14336), (65, 5120), (9, 40960), (3, 131072)])
@pytest.mark.parametrize("mode", ["rot_f32", "raw_f32", "raw_bf16"])
def test_gemv_shapes(n, k, mode):
    xdt = torch.bfloat16 if mode == "raw_bf16" else torch.float32
    worst = _gemv_case(n, k, xdt, mode == "rot_f32", seed=n + k)
    assert worst < 1e-4


def test_gemv_tiny_config_and_special_vectors():
    W, x = workloads.tiny_tq(DEV)
    packed, scales = tqa.quantize(W)
    say("[gemv] tiny config")
    y = tqa.gemv(packed, scales, x)
    yr, a = otq.gemv_rows_o64(packed.cpu().numpy(), u16(scales), x.cpu().numpy())
    assert_within(f32np(y), yr, a, what="tiny")
    Wd = otq.dequantize_o64(packed.cpu().numpy(), u16(scales))
    for j in (0, 31, 300, 511):                     # one-hot x -> a column of W_deq
        e = torch.zeros(512, device=DEV)
        e[j] = 1.0
        yj = f32np(tqa.gemv(packed, scales, e))
        np.testing.assert_allclose(yj, Wd[:, j], rtol=1e-5, atol=1e-7)
    zp, zs = tqa.quantize(torch.zeros(5, 64, device=DEV))
    assert not tqa.gemv(zp, zs, torch.ones(64, device=DEV)).any()


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 15, 16, 17, 32, 33, 48, 64, 65, 100])
def test_gemm_batch_sizes(m):
    n, k = 80, 1024
    g = workloads.generator(1000 + m, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    X = workloads.activation(m, k, g, DEV, torch.bfloat16)
    packed, scales = tqa.quantize(W)
    say(f"[gemm] M={m} {n}x{k}")
    Y = tqa.gemm(packed, scales, tqa.rotate(X, dtype=torch.bfloat16))
    yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.float().cpu().numpy())
    assert_within(f32np(Y), yr, a, what=f"gemm M={m}")


@pytest.mark.parametrize("m", [1, 3, 4, 7])
def test_gemm_fp32_small_batch(m):
    n, k = 50, 4096
    g = workloads.generator(2000 + m, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    X = workloads.activation(m, k, g, DEV, torch.float32)
    packed, scales = tqa.quantize(W)
    say(f"[gemm] fp32 M={m}")
    Y = tqa.gemm(packed, scales, tqa.rotate(X))
    yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.cpu().numpy())
    worst = assert_within(f32np(Y), yr, a, what=f"gemm fp32 M={m}")
    assert worst < 1e-4


@pytest.mark.parametrize("m", [16, 20, 64, 70])
def test_gemm_fp32_split_mfma_any_k(m):
    """float32 activations at M >= 16 take the three-pass hi/lo bf16 MFMA: the bound holds even at K = 32."""
    for k in (32, 96, 4128):
        n = 37
        g = workloads.generator(k + m, DEV)
        W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
        X = workloads.activation(m, k, g, DEV, torch.bfloat16)
        packed, scales = tqa.quantize(W)
        say(f"[gemm] fp32 split M={m} K={k}")
        Y = tqa.gemm(packed, scales, tqa.rotate(X))
        yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.float().cpu().numpy())
        worst = assert_within(f32np(Y), yr, a, what=f"gemm fp32 M={m} K={k}")
        assert worst < 1e-4


@pytest.mark.parametrize("m", [16, 40, 64])
def test_gemm_tall_row_tiles(m):
    """Shapes tall enough for the 2- and 4-row-tile workgroups, with K leaving a partial group of four blocks
    (bf16 operands: K in the thousands, where their rounding stays inside the bound)."""
    for n, k in ((32784, 1056), (17000, 1120)):
        g = workloads.generator(n + k + m, DEV)
        W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
        X = workloads.activation(m, k, g, DEV, torch.bfloat16)
        packed, scales = tqa.quantize(W)
        say(f"[gemm] tall M={m} {n}x{k}")
        Y = tqa.gemm(packed, scales, tqa.rotate(X, dtype=torch.bfloat16))
        yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.float().cpu().numpy())
        assert_within(f32np(Y), yr, a, what=f"gemm tall M={m} {n}x{k}")


@pytest.mark.parametrize("n,k", [(300, 1120), (1000, 3200), (517, 4096), (4100, 4096), (33, 2048), (90, 5120)])
def test_gemm_m16_persistent(n, k):
    """M = 16 with bf16 activations and K <= 4096 runs the persistent kernel whose 16 wavefronts split K:
    one or two groups of four blocks per wavefront, some wavefronts idle, ragged row tiles (K = 5120 takes
    the other kernel)."""
    m = 16
    g = workloads.generator(n * 7 + k, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    X = workloads.activation(m, k, g, DEV, torch.bfloat16)
    packed, scales = tqa.quantize(W)
    say(f"[gemm] persistent M=16 {n}x{k}")
    Y = tqa.gemm(packed, scales, tqa.rotate(X, dtype=torch.bfloat16))
    yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.float().cpu().numpy())
    assert_within(f32np(Y), yr, a, what=f"gemm M=16 {n}x{k}")


def test_gemm_bf16_large_k():
    """bf16 activations (one MFMA pass) at the decode shapes' K."""
    for k in (4096, 14336):
        n, m = 48, 32
        g = workloads.generator(k, DEV)
        W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
        X = workloads.activation(m, k, g, DEV, torch.bfloat16)
        packed, scales = tqa.quantize(W)
        say(f"[gemm] bf16 M={m} K={k}")
        Y = tqa.gemm(packed, scales, tqa.rotate(X, dtype=torch.bfloat16))
        yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.float().cpu().numpy())
        assert_within(f32np(Y), yr, a, what=f"gemm bf16 K={k}")


@pytest.mark.parametrize("n,k,m", [(300, 8192, 8), (4096, 14336, 16), (48, 14336, 32)])
def test_gemm_split_k_repeat_runs_are_bit_identical(n, k, m):
    """Few row tiles and K in several passes: K is split over two workgroups whose sums meet in Y; the
    result must not depend on which half lands first."""
    g = workloads.generator(n + k + m, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    X = workloads.activation(m, k, g, DEV, torch.bfloat16)
    packed, scales = tqa.quantize(W)
    xr = tqa.rotate(X, dtype=torch.bfloat16)
    say(f"[gemm] split K repeat M={m} {n}x{k}")
    Y1 = tqa.gemm(packed, scales, xr)
    for _ in range(3):
        Y2 = tqa.gemm(packed, scales, xr)
        assert torch.equal(Y1, Y2)
    rows = np.arange(0, n, max(1, n // 64))
    yr, a = otq.gemm_o64(packed.cpu().numpy()[rows], u16(scales)[rows], X.float().cpu().numpy())
    assert_within(f32np(Y1)[:, rows], yr, a, what=f"gemm split K M={m} {n}x{k}")


def test_repeat_runs_are_bit_identical():
    g = workloads.generator(77, DEV)
    W = workloads.normal_weight(300, 4096, 4096 ** -0.5, g, DEV, torch.bfloat16)
    x = workloads.activation(1, 4096, g, DEV, torch.bfloat16)[0].contiguous()
    p1, s1 = tqa.quantize(W)
    p2, s2 = tqa.quantize(W)
    assert torch.equal(p1, p2) and torch.equal(s1, s2)
    y1 = tqa.gemv(p1, s1, x)
    y2 = tqa.gemv(p1, s1, x)
    assert torch.equal(y1, y2)
