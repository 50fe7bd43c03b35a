"""Full-size parity on sampled outputs, in the launch configurations the benchmark times.

The decode layers of the Llama-3-8B, 27B (hidden 5120 / intermediate 17408) and
Llama-3-70B shapes, with the q|k|v and gate|up row groups concatenated as one
launch sees them:

* TQ4_1S quantize: packed nibbles and fp16 scales of sampled rows bit-exact
  against the oracle's canonical float32 quantizer;
* the fused GEMV with a bf16 activation (rotation fused, as benchmarked):
  sampled y within |dy| <= 1e-3 * sum_k |W_deq[n,k] x[k]| of the float64 oracle
  on the GPU's own packed weights;
* tq_gemm at M = 4, 16, 32, 64 on pre-rotated bf16 activations (8B q|k|v, o,
  gate|up, down: the split-K path at K = 4096 and the two-tile instantiation
  at M = 32 included);
* dequantization to float32 and bf16 at full size, at ragged shapes whose
  last wavefront is partial, and across the launch split at 2^30 blocks;
* NVFP4 and MXFP6 quantize + GEMV (M = 1 and 8) on the 27B MLP shapes, codes
  and block scales of sampled rows bit-exact.  The NVFP4 tensor scale depends
  on the whole tensor: its amax is taken on the host from the full weight and
  handed to the oracle as one extra row, so that the oracle applies its own
  definition to the same maximum.

The 70B shapes are drawn as the 70B workload draws them: N(0, 1/K) times the
layer's std drift U(0.5, 2) (one layer per shape).

Sampled rows: the first two, the middle, the last and twelve seeded ones.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa
from oracle import blockfp as obf
from oracle import tq4_1s as otq
import workloads
from gpu_helpers import say, u16, f32np, assert_within

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

TQ_SHAPES = [
    ("8B q|k|v", 6144, 4096), ("8B o", 4096, 4096), ("8B gate|up", 28672, 4096), ("8B down", 4096, 14336),
    ("27B q|k|v", 7168, 5120), ("27B gate|up", 34816, 5120), ("27B down", 5120, 17408),
    ("70B q|k|v", 10240, 8192), ("70B o", 8192, 8192), ("70B gate|up", 57344, 8192), ("70B down", 8192, 28672),
]


def sample_rows(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = {0, min(1, n - 1), n // 2, n - 1}
    rows.update(int(r) for r in rng.integers(0, n, 12))
    return np.array(sorted(rows))


def _weight(n, k, seed, variant="gauss"):
    g = workloads.generator(seed, DEV)
    if variant == "t4":
        return workloads.student_t4_weight(n, k, g, DEV, torch.bfloat16)
    return workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)


LLAMA70B_MEMBERS = {"70B q|k|v": ["q", "k", "v"], "70B o": ["o"], "70B gate|up": ["gate", "up"], "70B down": ["down"]}


def _weight_of(label, n, k, seed):
    """The 70B groups from the 70B workload's own draw (per-layer drift), the others N(0, 1/K) or t4."""
    if label in LLAMA70B_MEMBERS:
        layer = seed % workloads.LLAMA70B_LAYERS
        W = torch.cat([workloads.llama70b_weight(t, layer, DEV) for t in LLAMA70B_MEMBERS[label]], dim=0)
        assert tuple(W.shape) == (n, k)
        return W
    return _weight(n, k, seed, "t4" if n % 3 == 0 else "gauss")


@pytest.mark.parametrize("label,n,k", TQ_SHAPES, ids=[s[0] for s in TQ_SHAPES])
def test_tq4_full_size_quantize_and_fused_gemv(label, n, k):
    seed = n * 131 + k
    W = _weight_of(label, n, k, seed)
    x = workloads.activation(1, k, workloads.generator(seed + 1, DEV), DEV, torch.bfloat16)[0].contiguous()
    say(f"[full] {label} {n}x{k} quantize + gemv(bf16 x, fused rotation)")
    packed, scales = tqa.quantize(W)
    y = tqa.gemv(packed, scales, x)
    torch.cuda.synchronize()
    rows = sample_rows(n, seed)
    idx = torch.as_tensor(rows, device=DEV)
    Wh = W.index_select(0, idx).float().cpu().numpy()
    op, osc = otq.quantize_o32(Wh)
    gp = packed.index_select(0, idx).cpu().numpy()
    gs = u16(scales.index_select(0, idx))
    np.testing.assert_array_equal(gs, osc, err_msg=f"scales {label}")
    np.testing.assert_array_equal(gp, op, err_msg=f"packed {label}")
    yr, a = otq.gemv_rows_o64(gp, gs, x.float().cpu().numpy())
    worst = assert_within(f32np(y)[rows], yr, a, what=f"gemv {label}")
    assert worst < 1e-4
    y2 = tqa.gemv(packed, scales, x)
    assert torch.equal(y, y2), f"{label}: a second launch differs"


@pytest.mark.parametrize("m", [4, 16, 32, 64])
@pytest.mark.parametrize("label,n,k", TQ_SHAPES[:4], ids=[s[0] for s in TQ_SHAPES[:4]])
def test_tq4_full_size_gemm(label, n, k, m):
    seed = n + k + m
    W = _weight(n, k, seed)
    X = workloads.activation(m, k, workloads.generator(seed + 1, DEV), DEV, torch.bfloat16)
    say(f"[full] {label} {n}x{k} gemm M={m}")
    packed, scales = tqa.quantize(W)
    Y = tqa.gemm(packed, scales, tqa.rotate(X, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    rows = sample_rows(n, seed)
    idx = torch.as_tensor(rows, device=DEV)
    yr, a = otq.gemm_o64(packed.index_select(0, idx).cpu().numpy(), u16(scales.index_select(0, idx)),
                         X.float().cpu().numpy())
    assert_within(f32np(Y)[:, rows], yr, a, what=f"gemm {label} M={m}")


def _host_amax(W: torch.Tensor) -> np.float32:
    best = np.float32(0)
    for r0 in range(0, W.shape[0], 4096):
        best = max(best, np.abs(W[r0:r0 + 4096].float().cpu().numpy()).max())
    return np.float32(best)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
@pytest.mark.parametrize("label,n,k", [("27B gate|up", 34816, 5120), ("27B down", 5120, 17408)],
                         ids=["27B gate|up", "27B down"])
def test_blockfp_full_size(fmt, label, n, k):
    seed = n * 7 + k + (0 if fmt == "nvfp4" else 1)
    g = workloads.generator(seed, DEV)
    W = workloads.add_outliers(workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.float32), 0.001, 20.0, g)
    W = W.to(torch.bfloat16)
    say(f"[full] {fmt} {label} {n}x{k} quantize + gemm M=1, 8")
    codes, bs, ts = tqa.blockfp_quantize(fmt, W)
    torch.cuda.synchronize()
    rows = sample_rows(n, seed)
    idx = torch.as_tensor(rows, device=DEV)
    Wh = W.index_select(0, idx).float().cpu().numpy()
    if fmt == "nvfp4":
        extra = np.zeros((1, k), np.float32)
        extra[0, 0] = _host_amax(W)
        oc, osb, ost = obf.nvfp4_quantize_o32(np.concatenate([Wh, extra]))
        oc, osb = oc[:-1], osb[:-1]
        assert np.float32(ts.cpu().numpy()[0]).view(np.uint32) == np.float32(ost).view(np.uint32)
        Wd = obf.nvfp4_dequantize_o64(oc, osb, ost)
    else:
        oc, osb = obf.mxfp6_quantize_o32(Wh)
        Wd = obf.mxfp6_dequantize_o64(oc, osb)
    np.testing.assert_array_equal(bs.index_select(0, idx).cpu().numpy(), osb, err_msg=f"{fmt} block scales")
    np.testing.assert_array_equal(codes.index_select(0, idx).cpu().numpy(), oc, err_msg=f"{fmt} codes")
    for m in (1, 8):
        X = workloads.activation(m, k, workloads.generator(seed + m, DEV), DEV, torch.bfloat16)
        Y = tqa.blockfp_gemm(fmt, codes, bs, ts, X)
        torch.cuda.synchronize()
        yr, a = obf.gemm_deq_o64(Wd, X.float().cpu().numpy())
        assert_within(f32np(Y)[:, rows], yr, a, what=f"{fmt} {label} M={m}")


def _check_dequant_rows(packed, scales, Wd32, Wdb, rows, what):
    """Sampled rows of the float32 output against the float64 definition (4e-7 * sum|q| per block, the
    float32 rounding of a 32-term butterfly), and the bf16 output equal to the RNE of the float32 one."""
    idx = torch.as_tensor(rows, device=DEV)
    p = packed.index_select(0, idx).cpu().numpy()
    sc = u16(scales.index_select(0, idx))
    ref = otq.dequantize_o64(p, sc)
    q = otq.rotated_weights_f64(p, sc)
    bound = 4e-7 * np.repeat(np.abs(q).reshape(len(rows), -1, 32).sum(-1), 32, axis=1) + 1e-30
    got = f32np(Wd32.index_select(0, idx))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements outside the bound"
    np.testing.assert_array_equal(Wdb.index_select(0, idx).float().cpu().numpy(),
                                  Wd32.index_select(0, idx).bfloat16().float().cpu().numpy(), err_msg=what)


@pytest.mark.parametrize("n,k", [(28672, 4096), (4097, 4096), (65, 96), (3, 32), (1, 14336)])
def test_dequantize_full_size_and_ragged(n, k):
    """Full-size and ragged shapes: 65 x 96 and 3 x 32 end on a partial wavefront of blocks (the output
    goes through LDS one wavefront of blocks at a time)."""
    seed = n * 3 + k
    W = _weight(n, k, seed, "t4" if n % 2 else "gauss")
    packed, scales = tqa.quantize(W)
    say(f"[full] dequantize {n}x{k} float32 + bf16")
    Wd32 = tqa.dequantize(packed, scales)
    Wdb = tqa.dequantize(packed, scales, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.arange(n) if n <= 128 else sample_rows(n, seed)
    _check_dequant_rows(packed, scales, Wd32, Wdb, rows, f"dequantize {n}x{k}")
    if n * k <= (1 << 24):              # small enough to compare every element on the device
        assert torch.equal(Wdb, Wd32.bfloat16())


def test_dequantize_across_the_launch_split():
    """N x K with more than 2^30 blocks is dequantized in launches of 2^30 / (K/32) rows: rows on both sides of
    the split (and the last one) are checked.  Random nibbles and scales (the quantizer is not needed to
    exercise the split): 1048579 x 32768, 21.5 GB packed and scales, 68.7 GB of bf16 output."""
    n, k = (1 << 20) + 3, 32768
    split = (1 << 30) // (k // 32)
    assert split == 1 << 20
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    say(f"[full] dequantize across the launch split {n}x{k}")
    packed = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=DEV, generator=g)
    scales = (torch.rand((n, k // 16), device=DEV, generator=g) * 0.1 + 1e-3).half().view(torch.int16)
    Wdb = tqa.dequantize(packed, scales, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.array([0, 1, split - 2, split - 1, split, split + 1, n - 1])
    idx = torch.as_tensor(rows, device=DEV)
    p = packed.index_select(0, idx)
    sc = scales.index_select(0, idx)
    del packed, scales
    Wd32 = tqa.dequantize(p, sc)           # the same rows through one launch
    got = Wdb.index_select(0, idx)
    del Wdb
    torch.cuda.empty_cache()
    _check_dequant_rows(p, sc, Wd32, got, np.arange(len(rows)), "dequantize across the split")
