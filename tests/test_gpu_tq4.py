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


@pytest.mark.parametrize("k", [11296, 22400, 32000])
def test_gemv_bf16_rotation_on_matrix_cores(k):
    """A raw bf16 activation with one block per lane and at most two row slots per workgroup (K above
    10240, at most 1024 blocks) is rotated on the matrix cores.  Block counts that leave the last
    wavefront of a row part-filled (353, 700 and 1000 blocks), three sign masks, and one-hot activations
    (x' of a one-hot x is exactly +-1, so y is a column of W_deq)."""
    n = 37
    g = workloads.generator(k, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    x = workloads.activation(1, k, g, DEV, torch.bfloat16)[0].contiguous()
    for mask in (0, 0xFFFFFFFF, otq.sign_mask_from_seed(k)):
        say(f"[gemv mfma rotation] {n}x{k} mask={mask:#x}")
        packed, scales = tqa.quantize(W, sign_mask=mask)
        y = tqa.gemv(packed, scales, x, sign_mask=mask)
        yr, a = otq.gemv_rows_o64(packed.cpu().numpy(), u16(scales), x.float().cpu().numpy(), mask)
        assert assert_within(f32np(y), yr, a, what=f"gemv {n}x{k} mask {mask:#x}") < 1e-4
    Wd = otq.dequantize_o64(packed.cpu().numpy(), u16(scales), mask)
    for j in (0, 31, k // 2 + 5, k - 1):
        e = torch.zeros(k, dtype=torch.bfloat16, device=DEV)
        e[j] = 1.0
        np.testing.assert_allclose(f32np(tqa.gemv(packed, scales, e, sign_mask=mask)), Wd[:, j], rtol=1e-5,
                                   atol=1e-7)


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


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("k", [32, 96])
def test_gemm_one_hot_rows_rotated_domain_bound(k, xdtype):
    """One-hot activation rows at M = 16 (MFMA path): the rotated-domain bound holds.

    The kernels multiply q = d * c[idx] by x' = (1/sqrt 32) H D x, so the
    rounding of their operands is bounded by sum_k |q_k x'_k|.  For a one-hot
    x that sum can be far larger than sum_k |W_deq[n,k] x_k| (the 32 products
    of one block cancel down to a single weight), so the original-domain
    1e-3 bound is not guaranteed here.  Operand rounding per product:
    bf16 x' 2^-8 and bf16 weights 2^-8 + 2^-11 (fp16 centroids times the
    scale, rounded once); float32 x' through the three-pass hi/lo split, at
    most 2^-13.  Plus float32 accumulation over K.
    """
    m, n = 16, 37
    g = workloads.generator(31 * k + (xdtype == torch.float32), DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    vals = workloads.activation(1, m, g, DEV, torch.bfloat16)[0].float()
    X = torch.zeros(m, k, device=DEV, dtype=torch.float32)
    cols = torch.arange(m, device=DEV) * 7 % k
    X[torch.arange(m, device=DEV), cols] = vals
    X = X.to(xdtype)
    packed, scales = tqa.quantize(W)
    say(f"[gemm] one-hot M={m} K={k} x'={xdtype}")
    Y = f32np(tqa.gemm(packed, scales, tqa.rotate(X, dtype=xdtype)))
    Xh = X.float().cpu().numpy().astype(np.float64)
    yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), Xh)
    q = otq.rotated_weights_f64(packed.cpu().numpy(), u16(scales))
    xr = otq.rotate_f64(Xh.reshape(m, k // 32, 32), otq.DEFAULT_SIGN_MASK).reshape(m, k)
    rot = np.abs(xr) @ np.abs(q).T                         # sum_k |q_k x'_k|
    per_product = 2.0 ** -7 + 2.0 ** -10 if xdtype == torch.bfloat16 else 2.0 ** -13
    bound = (per_product + k * 2.0 ** -23) * rot
    err = np.abs(Y - yr)
    bad = err > bound
    assert not bad.any(), (f"{bad.sum()} outside the rotated-domain bound; worst ratio "
                           f"{float((err / np.maximum(rot, 1e-300)).max())!r}")
    assert np.all(rot >= a * (1 - 1e-12))                  # the rotated sum dominates the original one


@pytest.mark.gpu
def test_gemm_workspace_reused_across_shapes():
    """One workspace serves split-K calls of different shapes in turn: a call with few row tiles writes its
    partial sums where a later, taller call keeps per-tile counters only if the layout let them overlap, so
    the taller call must still be exact (and the shorter one after it)."""
    m = 16
    ws = torch.zeros(tqa.workspace_bytes("gemm", 8192, 14336, 64), dtype=torch.uint8, device=DEV)
    for n, k in ((517, 4096), (4100, 4096), (300, 8192), (8192, 14336), (517, 4096)):
        g = workloads.generator(n + k, DEV)
        W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
        X = workloads.activation(m, k, g, DEV, torch.bfloat16)
        packed, scales = tqa.quantize(W)
        say(f"[gemm] shared workspace M={m} {n}x{k}")
        Y = tqa.gemm(packed, scales, tqa.rotate(X, dtype=torch.bfloat16), workspace=ws)
        rows = np.unique(np.linspace(0, n - 1, 256).astype(int))
        yr, a = otq.gemm_o64(packed.cpu().numpy()[rows], u16(scales)[rows], X.float().cpu().numpy())
        assert_within(f32np(Y)[:, rows], yr, a, what=f"gemm shared workspace {n}x{k}")
        # every call leaves the per-tile counters (the first 64 KiB) at zero for the next one
        torch.cuda.synchronize()
        assert int(ws[:65536].view(torch.int32).count_nonzero()) == 0


@pytest.mark.parametrize("m", [1, 2, 3, 16, 17, 64])
@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float32])
def test_gemm_padded_row_strides(m, xdtype):
    """Activation rows and output rows with leading dimensions above K and N (slices of wider buffers): every
    path (VALU rows, the persistent MFMA kernel with K split over workgroups at K = 8192, the float32 hi/lo
    MFMA kernel) reads and writes through them, and the padding columns of the output stay untouched."""
    n, k = 96, 8192
    g = workloads.generator(3000 + m, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    X = workloads.activation(m, k, g, DEV, torch.bfloat16)
    packed, scales = tqa.quantize(W)
    xr_full = torch.zeros((m, k + 64), dtype=xdtype, device=DEV)
    xr = xr_full[:, :k]
    xr.copy_(tqa.rotate(X, dtype=xdtype))
    y_full = torch.full((m, n + 40), 12345.0, dtype=torch.float32, device=DEV)
    y = y_full[:, :n]
    say(f"[gemm] padded strides M={m} x'={xdtype} ldx={xr.stride(0)} ldy={y.stride(0)}")
    tqa.gemm(packed, scales, xr, out=y)
    torch.cuda.synchronize()
    assert torch.all(y_full[:, n:] == 12345.0)
    yr, a = otq.gemm_o64(packed.cpu().numpy(), u16(scales), X.float().cpu().numpy())
    assert_within(f32np(y), yr, a, what=f"gemm padded M={m} {xdtype}")


def test_rotate_padded_rows_and_given_outputs():
    """Rotation through padded input and output row strides, into a given output (written in place), and of
    a single vector into a given 1-D output: bit-exact against the oracle."""
    g = workloads.generator(6, DEV)
    x = workloads.activation(5, 2048, g, DEV, torch.bfloat16)
    ref = otq.rotate_f32(x.float().cpu().numpy().reshape(5, -1, 32), otq.DEFAULT_SIGN_MASK).reshape(5, -1)
    x_full = torch.zeros((5, 2048 + 96), dtype=torch.bfloat16, device=DEV)
    x_full[:, :2048] = x
    out_full = torch.full((5, 2048 + 32), 9.0, dtype=torch.float32, device=DEV)
    say("[rotate] padded rows into a given output")
    r = tqa.rotate(x_full[:, :2048], out=out_full[:, :2048])
    torch.cuda.synchronize()
    assert r.data_ptr() == out_full.data_ptr()
    np.testing.assert_array_equal(out_full[:, :2048].cpu().numpy(), ref)
    assert torch.all(out_full[:, 2048:] == 9.0)
    v_out = torch.empty(2048, dtype=torch.float32, device=DEV)
    r1 = tqa.rotate(x[2].contiguous(), out=v_out)
    torch.cuda.synchronize()
    assert r1.data_ptr() == v_out.data_ptr()
    np.testing.assert_array_equal(v_out.cpu().numpy(), ref[2])


def test_gemm_split_k_graph_replays():
    """Split-K GEMMs (M = 16 and M = 32 at K = 14336: sums and per-tile counters in the workspace) captured in
    a HIP graph and replayed several times, with other library work between the replays: every replay equals
    the eager result bit for bit, since each call leaves the counters at zero for the next."""
    n, k = 1024, 14336
    g = workloads.generator(4242, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    packed, scales = tqa.quantize(W)
    xs = [tqa.rotate(workloads.activation(m, k, g, DEV, torch.bfloat16), dtype=torch.bfloat16) for m in (16, 32)]
    ys = [torch.empty((x.shape[0], n), dtype=torch.float32, device=DEV) for x in xs]
    ws = torch.zeros(tqa.workspace_bytes("gemm", n, k, 32), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 65536                                   # the split path is taken
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ref = [tqa.gemm(packed, scales, x, workspace=ws).clone() for x in xs]
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            for x, y in zip(xs, ys):
                tqa.gemm(packed, scales, x, out=y, workspace=ws)
        for rep in range(4):
            say(f"[gemm] split-K graph replay {rep}")
            for y in ys:
                y.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            for y, r in zip(ys, ref):
                assert torch.equal(y, r), f"replay {rep}"
            tqa.gemm(packed, scales, xs[1], workspace=ws)       # eager work on the same workspace between replays
            torch.cuda.synchronize()
    assert int(ws[:65536].view(torch.int32).count_nonzero()) == 0
    X0 = xs[0].float().cpu().numpy()                            # x' itself: the oracle's product of rotated rows
    q = otq.rotated_weights_f64(packed.cpu().numpy()[:64], u16(scales)[:64])
    yr = X0.astype(np.float64) @ q.T
    a = np.abs(X0.astype(np.float64)) @ np.abs(q).T
    assert np.all(np.abs(f32np(ref[0])[:, :64] - yr) <= 1e-2 * a)   # bf16 operands: within 2^-7 of sum |q x'|


def test_gemm_split_k_on_two_streams():
    """The binding keeps one zero-filled workspace per stream: split-K GEMMs issued on two streams without
    synchronizing between them give the results of the same calls made one after the other."""
    n, k, m = 2048, 14336, 16
    g = workloads.generator(4343, DEV)
    Ws = [workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16) for _ in range(2)]
    qs = [tqa.quantize(W) for W in Ws]
    x = tqa.rotate(workloads.activation(m, k, g, DEV, torch.bfloat16), dtype=torch.bfloat16)
    ref = [tqa.gemm(p, sc, x) for p, sc in qs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    say("[gemm] split-K on two streams")
    for it in range(3):
        for i, (st, (p, sc)) in enumerate(zip(streams, qs)):
            with torch.cuda.stream(st):
                outs[i].append(tqa.gemm(p, sc, x))
    torch.cuda.synchronize()
    for i in range(2):
        for y in outs[i]:
            assert torch.equal(y, ref[i])


@pytest.mark.parametrize("n,k", [(300, 4096), (1000, 14336)])
def test_gemv_prerotated_bf16(n, k):
    """A pre-rotated activation in bf16 (as tq_rotate rounds it): the product is exact for that x', so it is
    checked in the rotated domain against the float64 q . x' within 1e-3 of sum |q x'|."""
    g = workloads.generator(5100 + n, DEV)
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    x = workloads.activation(1, k, g, DEV, torch.bfloat16)[0].contiguous()
    packed, scales = tqa.quantize(W)
    xr = tqa.rotate(x, dtype=torch.bfloat16)
    say(f"[gemv] pre-rotated bf16 x' {n}x{k}")
    y = tqa.gemv(packed, scales, xr, rotated=True)
    torch.cuda.synchronize()
    q = otq.rotated_weights_f64(packed.cpu().numpy(), u16(scales))
    xv = xr.float().cpu().numpy().astype(np.float64)
    yr = q @ xv
    a = np.abs(q) @ np.abs(xv)
    assert np.all(np.abs(f32np(y) - yr) <= 1e-3 * a)
    # the same x' as float32 gives the same product up to float32 rounding
    y32 = tqa.gemv(packed, scales, xr.float().contiguous(), rotated=True)
    torch.cuda.synchronize()
    assert np.all(np.abs(f32np(y32) - f32np(y)) <= 1e-5 * a)
