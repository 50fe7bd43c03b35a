"""tq_attn_decode_noalloc (the allocation-free variant of tq_attn_decode) against tq_attn_decode, through
the C ABI: two calls in a row, the second with a smaller problem, each output identical to the one the
workspace entry point gives for the same inputs (the same kernels; the partials only live elsewhere)."""

import ctypes

import pytest
import torch

import dequant_gemv_tq_amd as tqa

pytestmark = pytest.mark.gpu

BF16 = 1


def _cache(B, Hkv, T, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    K = torch.randn((B, Hkv, T, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, T, 128), generator=g, device="cuda").to(torch.bfloat16)
    return tqa.kv_quantize_k(K) + tqa.kv_quantize_v(V)


def _both(B, Hq, Hkv, T, lengths, seed):
    L = tqa.lib()
    kc, ks, vp, vn = _cache(B, Hkv, T, seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    sign = tqa.kv_sign_from_seed(0)
    o_ref = torch.full((B, Hq, 128), float("nan"), device="cuda")
    o_new = torch.full((B, Hq, 128), float("nan"), device="cuda")
    ws_bytes = L.tq_attn_workspace_bytes(B, Hq, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.tq_attn_decode(P(q), BF16, B, Hq, Hkv, 128, T, P(lens), P(kc), P(ks), P(vp), P(vn), sign, P(o_ref), P(ws),
                          ws_bytes, s)
    assert st == 0
    st = L.tq_attn_decode_noalloc(P(q), BF16, B, Hq, Hkv, 128, T, P(lens), P(kc), P(ks), P(vp), P(vn), sign, P(o_new),
                                  s)
    assert st == 0
    torch.cuda.synchronize()
    return o_ref, o_new


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    # first call: 8 sequences (ragged lengths, empty ones included), GQA 4, T_max 2048
    o_ref, o_new = _both(8, 32, 8, 2048, [2048, 1, 0, 1000, 2047, 256, 257, 1500], seed=11)
    assert torch.equal(o_new, o_ref)
    assert not torch.isnan(o_new).any()
    # second call on the same device right after: a smaller problem (3 sequences, GQA 4, 2 cache heads)
    o_ref, o_new = _both(3, 8, 2, 600, [600, 17, 300], seed=12)
    assert torch.equal(o_new, o_ref)
    assert not torch.isnan(o_new).any()


def test_noalloc_rejects_problems_beyond_its_scratch():
    L = tqa.lib()
    sign = tqa.kv_sign_from_seed(0)
    g = ctypes.c_void_p(0x10000)
    # 64 x 32 query heads x 32768 tokens need 34 MB of partials, more than the 8 MiB the array holds
    assert L.tq_attn_workspace_bytes(64, 32, 32768) > (8 << 20)
    st = L.tq_attn_decode_noalloc(g, BF16, 64, 32, 8, 128, 32768, g, g, g, g, g, sign, g,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 2                     # TQ_ESHAPE, before anything launches


def test_noalloc_under_graph_capture():
    """The allocation-free call captured in a HIP graph (what it is for) and replayed several times, with an
    eager call of another shape on the same device between the replays: every replay gives the result of the
    workspace entry point."""
    L = tqa.lib()
    B, Hq, Hkv, T = 4, 16, 4, 1500
    kc, ks, vp, vn = _cache(B, Hkv, T, 21)
    g = torch.Generator(device="cuda")
    g.manual_seed(22)
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    lens = torch.tensor([1500, 3, 700, 257], dtype=torch.int32, device="cuda")
    sign = tqa.kv_sign_from_seed(0)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    ws_bytes = L.tq_attn_workspace_bytes(B, Hq, T)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    o_ref = torch.empty((B, Hq, 128), device="cuda")
    cur = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.tq_attn_decode(P(q), BF16, B, Hq, Hkv, 128, T, P(lens), P(kc), P(ks), P(vp), P(vn), sign, P(o_ref),
                            P(ws), ws_bytes, cur()) == 0
    o = torch.empty_like(o_ref)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # one eager call first: the array's device address is looked up outside the capture
        assert L.tq_attn_decode_noalloc(P(q), BF16, B, Hq, Hkv, 128, T, P(lens), P(kc), P(ks), P(vp), P(vn), sign,
                                        P(o), cur()) == 0
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            assert L.tq_attn_decode_noalloc(P(q), BF16, B, Hq, Hkv, 128, T, P(lens), P(kc), P(ks), P(vp), P(vn),
                                            sign, P(o), cur()) == 0
        for rep in range(3):
            o.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), f"replay {rep}"
            o_ref2, o_new2 = _both(2, 8, 2, 400, [400, 99], seed=30 + rep)   # other shapes, same array
            assert torch.equal(o_new2, o_ref2)
