"""The library's calls captured in a HIP graph and replayed: every replay must equal the eager result bit for
bit, with other library work (on the same buffers and workspaces) between the replays.  Covers the fused
GEMV (raw bf16 and pre-rotated fp32 activations), quantize, dequantize, the NVFP4 quantizer (its partial
maxima in a workspace that nothing clears), the block-float product, and decode attention (split partials
in a workspace)."""

import pytest
import torch

import dequant_gemv_tq_amd as tqa
import workloads
from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _replay(capture, outputs, between, reps=3):
    """Eager run, capture, then `reps` replays (outputs poisoned before each) compared with the eager run."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        capture()
        torch.cuda.synchronize()
        ref = [o.clone() for o in outputs]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            capture()
        for rep in range(reps):
            for o in outputs:
                if o.is_floating_point():
                    o.fill_(float("nan"))
                else:
                    o.fill_(0x5A)
            graph.replay()
            torch.cuda.synchronize()
            for o, r in zip(outputs, ref):
                assert torch.equal(o, r), f"replay {rep}"
            between()
            torch.cuda.synchronize()


def test_gemv_quantize_dequantize_replays():
    g = workloads.generator(7001, DEV)
    n, k = 3000, 4096
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    x = workloads.activation(1, k, g, DEV, torch.bfloat16)[0].contiguous()
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((n, k // 16), dtype=torch.int16, device=DEV)
    tqa.quantize(W, out=(packed, scales))
    xr = tqa.rotate(x)
    y1 = torch.empty(n, dtype=torch.float32, device=DEV)
    y2 = torch.empty(n, dtype=torch.float32, device=DEV)
    Wd = torch.empty((n, k), dtype=torch.bfloat16, device=DEV)
    p2 = torch.empty_like(packed)
    s2 = torch.empty_like(scales)

    def capture():
        tqa.quantize(W, out=(p2, s2))
        tqa.gemv(packed, scales, x, out=y1)
        tqa.gemv(packed, scales, xr, rotated=True, out=y2)
        tqa.dequantize(packed, scales, dtype=torch.bfloat16, out=Wd)

    say("[graphs] quantize / gemv / dequantize")
    _replay(capture, [p2, s2, y1, y2, Wd], lambda: tqa.gemv(p2, s2, x))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp6"])
def test_blockfp_replays(fmt):
    g = workloads.generator(7002, DEV)
    n, k = 700, 5120
    W = workloads.normal_weight(n, k, k ** -0.5, g, DEV, torch.bfloat16)
    X = workloads.activation(8, k, g, DEV, torch.bfloat16)
    codes, bs, ts = tqa.blockfp_quantize(fmt, W)
    need = tqa.workspace_bytes(f"{fmt}_quantize", n, k)
    qws = torch.zeros(max(need, 4), dtype=torch.uint8, device=DEV)
    c2, b2 = torch.empty_like(codes), torch.empty_like(bs)
    t2 = torch.empty_like(ts) if ts is not None else None
    Y = torch.empty((8, n), dtype=torch.float32, device=DEV)

    def capture():
        tqa.blockfp_quantize(fmt, W, out=(c2, b2, t2), workspace=qws if fmt == "nvfp4" else None)
        tqa.blockfp_gemm(fmt, codes, bs, ts, X, out=Y)

    say(f"[graphs] {fmt} quantize / gemm")
    outs = [c2, b2, Y] + ([t2] if t2 is not None else [])
    _replay(capture, outs, lambda: tqa.blockfp_quantize(fmt, X.repeat(4, 1)[:, :k].contiguous(),
                                                         workspace=qws if fmt == "nvfp4" else None))


def test_attention_replays():
    g = workloads.generator(7003, DEV)
    B, Hq, Hkv, T = 3, 16, 4, 900
    K = torch.randn((B, Hkv, T, 128), generator=g, device=DEV).to(torch.bfloat16)
    V = torch.randn((B, Hkv, T, 128), generator=g, device=DEV).to(torch.bfloat16)
    kc, ks = tqa.kv_quantize_k(K)
    vp, vn = tqa.kv_quantize_v(V)
    q = torch.randn((B, Hq, 128), generator=g, device=DEV).to(torch.bfloat16)
    lengths = torch.tensor([900, 1, 513], dtype=torch.int32, device=DEV)
    ws = torch.zeros(tqa.attn_workspace_bytes(B, Hq, T), dtype=torch.uint8, device=DEV)
    o = torch.empty((B, Hq, 128), dtype=torch.float32, device=DEV)
    kc2, ks2 = torch.empty_like(kc), torch.empty_like(ks)

    def capture():
        tqa.kv_quantize_k(K, out=(kc2, ks2))
        tqa.attn_decode(q, lengths, kc, ks, vp, vn, out=o, workspace=ws)

    def between():
        tqa.attn_decode(q[:2].contiguous(), lengths[:2].contiguous(), kc[:2].contiguous(), ks[:2].contiguous(),
                        vp[:2].contiguous(), vn[:2].contiguous(), workspace=ws)

    say("[graphs] kv encode / attention")
    _replay(capture, [kc2, ks2, o], between)
