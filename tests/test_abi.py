"""The C ABI library loads, exports every symbol include/tq.h declares, and
rejects bad arguments before launching anything (CPU only: no compute calls)."""

import ctypes
import os
import re

import numpy as np
import pytest

import dequant_gemv_tq_amd as tqa
from oracle import codebook as cb
from oracle import tq4_1s as otq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

EINVAL, ESHAPE, EALIGN, EDTYPE = 1, 2, 3, 4
F32, BF16, F16 = 0, 1, 2
GOOD = 0x10000          # a 64 KiB-aligned fake device address: never dereferenced by a rejected call


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_what_the_binding_knows():
    assert sorted(tqa.EXPORTED) == _declared()


def test_library_exports_every_declared_symbol():
    L = tqa.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_abi_version_and_status_strings():
    L = tqa.lib()
    assert L.tq_abi_version() == 3
    for s in range(6):
        assert L.tq_status_str(s)
    assert b"unknown" in L.tq_status_str(99)


def test_codebook_matches_oracle_bit_exactly():
    c, m = tqa.codebook()
    np.testing.assert_array_equal(c, cb.tq4_codebook_f32())
    np.testing.assert_array_equal(m, cb.tq4_midpoints_f32())


def test_sign_mask_matches_oracle_splitmix():
    for seed in (0, 1, 42, 2 ** 63 + 5):
        assert tqa.sign_mask_from_seed(seed) == otq.sign_mask_from_seed(seed)
    assert tqa.default_sign_mask() == otq.DEFAULT_SIGN_MASK == tqa.DEFAULT_SIGN_MASK


def test_kv_sign_words_match_oracle_splitmix():
    from oracle import kv as okv
    for seed in (0, 3, 2 ** 64 - 1):
        assert list(tqa.kv_sign_from_seed(seed)) == okv.kv_sign_words(seed)
    assert tqa.lib().tq_kv_sign_from_seed(0, None) == EINVAL


def _p(v):
    return ctypes.c_void_p(v)


@pytest.mark.parametrize("args,expect", [
    ((None, F32, 4, 64, 64, 0, _p(GOOD), _p(GOOD), None), EINVAL),          # null W
    ((_p(GOOD), F32, 4, 64, 64, 0, None, _p(GOOD), None), EINVAL),          # null packed
    ((_p(GOOD), F32, 0, 64, 64, 0, _p(GOOD), _p(GOOD), None), EINVAL),      # N = 0
    ((_p(GOOD), F32, 4, -32, 64, 0, _p(GOOD), _p(GOOD), None), EINVAL),     # K < 0
    ((_p(GOOD), F32, 4, 48, 48, 0, _p(GOOD), _p(GOOD), None), ESHAPE),      # K % 32
    ((_p(GOOD), F32, 4, 64, 32, 0, _p(GOOD), _p(GOOD), None), EINVAL),      # ldw < K
    ((_p(GOOD), F16, 4, 64, 64, 0, _p(GOOD), _p(GOOD), None), EDTYPE),      # fp16 weights
    ((_p(GOOD + 4), F32, 4, 64, 64, 0, _p(GOOD), _p(GOOD), None), EALIGN),  # W misaligned
    ((_p(GOOD), F32, 4, 64, 66, 0, _p(GOOD), _p(GOOD), None), EALIGN),      # ldw*4 % 16
    ((_p(GOOD), F32, 4, 64, 64, 0, _p(GOOD + 8), _p(GOOD), None), EALIGN),  # packed misaligned
    ((_p(GOOD), F32, 4, 64, 64, 0, _p(GOOD), _p(GOOD + 2), None), EALIGN),  # scales misaligned
])
def test_quantize_rejects(args, expect):
    assert tqa.lib().tq_quantize(*args) == expect
    assert tqa.lib().tq_quantize_rsf(*args) == expect


def test_other_calls_reject_before_launch():
    L = tqa.lib()
    g = _p(GOOD)
    # gemv
    assert L.tq_gemv(g, g, 8, 64, 0, None, F32, 1, g, None) == EINVAL
    assert L.tq_gemv(g, g, 8, 50, 0, g, F32, 1, g, None) == ESHAPE
    assert L.tq_gemv(g, g, 8, 131072 + 32, 0, g, F32, 1, g, None) == ESHAPE
    assert L.tq_gemv(g, g, 8, 64, 0, g, F16, 1, g, None) == EDTYPE           # rotated x: fp32 or bf16
    assert L.tq_gemv(g, g, 8, 64, 0, g, F16, 0, g, None) == EDTYPE
    assert L.tq_gemv(g, g, 8, 64, 0, _p(GOOD + 4), F32, 1, g, None) == EALIGN
    assert L.tq_gemv(g, g, 8, 64, 0, g, F32, 1, _p(GOOD + 2), None) == EALIGN
    # gemm
    assert L.tq_gemm(g, g, 8, 64, 0, g, BF16, 64, g, 8, None, 0, None) == EINVAL
    assert L.tq_gemm(g, g, 8, 64, 257, g, BF16, 64, g, 8, None, 0, None) == ESHAPE
    assert L.tq_gemm(g, g, 8, 64, 16, g, F16, 64, g, 8, None, 0, None) == EDTYPE
    assert L.tq_gemm(g, g, 8, 64, 4, g, BF16, 60, g, 8, None, 0, None) == EINVAL     # ldx < K
    assert L.tq_gemm(g, g, 8, 64, 4, g, BF16, 64, g, 4, None, 0, None) == EINVAL     # ldy < N
    # a launch that splits K needs its workspace: missing, short or misaligned is rejected
    need = L.tq_workspace_bytes(5, 4096, 14336, 16)
    assert need > 0
    assert L.tq_gemm(g, g, 4096, 14336, 16, g, BF16, 14336, g, 4096, None, 0, None) == EINVAL
    assert L.tq_gemm(g, g, 4096, 14336, 16, g, BF16, 14336, g, 4096, g, need - 4, None) == EINVAL
    assert L.tq_gemm(g, g, 4096, 14336, 16, g, BF16, 14336, g, 4096, _p(GOOD + 16), need, None) == EALIGN
    assert L.tq_blockfp_gemm(1, g, g, g, 4096, 14336, 16, g, BF16, 14336, g, 4096, None, 0, None) == EINVAL
    # rotate / dequantize
    assert L.tq_rotate(g, F32, 2, 40, 40, 0, g, F32, 40, None) == ESHAPE
    assert L.tq_rotate(g, F16, 2, 64, 64, 0, g, F32, 64, None) == EDTYPE
    assert L.tq_dequantize(g, g, 2, 64, 0, None, F32, 64, None) == EINVAL
    assert L.tq_dequantize(g, g, 2, 64, 0, g, F16, 64, None) == EDTYPE
    # block float
    W4 = 4096                                                                     # TQ_NVFP4_WORKSPACE_BYTES
    assert L.tq_blockfp_quantize(3, g, F32, 2, 64, g, g, g, g, W4, None) == EINVAL
    assert L.tq_blockfp_quantize(1, g, F32, 2, 64, g, g, None, g, W4, None) == EINVAL   # NVFP4 needs tensor_scale
    assert L.tq_blockfp_quantize(1, g, F32, 2, 64, g, g, g, None, W4, None) == EINVAL   # ... and a workspace
    assert L.tq_blockfp_quantize(1, g, F32, 2, 64, g, g, g, g, W4 - 4, None) == EINVAL  # ... of the full size
    assert L.tq_blockfp_quantize(1, g, F32, 2, 64, g, g, g, _p(GOOD + 2), W4, None) == EALIGN
    assert L.tq_blockfp_quantize(1, g, F32, 2, 40, g, g, g, g, W4, None) == ESHAPE
    assert L.tq_blockfp_quantize(2, g, F32, 2, 48, g, g, None, None, 0, None) == ESHAPE   # MXFP6 needs K % 32
    assert L.tq_blockfp_quantize(2, g, F16, 2, 64, g, g, None, None, 0, None) == EDTYPE
    # workspace sizes: NVFP4 quantization, the split-K GEMMs and decode attention take one
    smax = ctypes.c_size_t(-1).value
    assert L.tq_workspace_bytes(6, 17408, 5120, 0) == W4
    for op in (1, 2, 3, 4, 7, 9, 10):
        assert L.tq_workspace_bytes(op, 4096, 4096, 16) == 0
    for op in (5, 8):
        assert L.tq_workspace_bytes(op, 4096, 14336, 2) == 0                  # M <= 2: the VALU kernel
        assert L.tq_workspace_bytes(op, 4096, 14336, 64) > 0                  # K in several ranges
        assert L.tq_workspace_bytes(op, 4096, 14336, 0) == smax
    assert L.tq_workspace_bytes(11, 2, 32, 1000) == L.tq_attn_workspace_bytes(2, 32, 1000)
    assert L.tq_workspace_bytes(11, 0, 32, 1000) == smax
    assert L.tq_workspace_bytes(99, 1, 1, 1) == smax
    assert tqa.workspace_bytes("nvfp4_quantize", 8, 64) == W4
    # the plain streaming-read helper
    assert L.tq_stream_read(None, 64, g, None) == EINVAL
    assert L.tq_stream_read(g, 0, g, None) == EINVAL
    assert L.tq_stream_read(g, 72, g, None) == ESHAPE
    assert L.tq_stream_read(_p(GOOD + 8), 64, g, None) == EALIGN
    assert L.tq_stream_read(g, 64, _p(GOOD + 2), None) == EALIGN
    for fn in (L.tq_blockfp_quantize, L.tq_blockfp_quantize_rsf):
        assert fn(3, g, F32, 2, 64, g, g, g, g, W4, None) == EINVAL
        assert fn(1, g, F32, 2, 64, g, g, None, g, W4, None) == EINVAL
        assert fn(1, g, F32, 2, 64, g, g, g, None, W4, None) == EINVAL
        assert fn(1, g, F32, 2, 40, g, g, g, g, W4, None) == ESHAPE
        assert fn(2, g, F32, 2, 48, g, g, None, None, 0, None) == ESHAPE
        assert fn(2, g, F16, 2, 64, g, g, None, None, 0, None) == EDTYPE
        assert fn(2, _p(GOOD + 4), F32, 2, 64, g, g, None, None, 0, None) == EALIGN     # W: 16 B
        assert fn(1, g, F32, 2, 64, _p(GOOD + 4), g, g, g, W4, None) == EALIGN        # codes: 8 B
    assert L.tq_blockfp_gemm(1, g, g, g, 8, 64, 4097, g, F32, 64, g, 8, None, 0, None) == ESHAPE   # M <= 4096
    assert L.tq_blockfp_gemm(1, g, g, g, 8, 32800, 1, g, F32, 32800, g, 8, None, 0, None) == ESHAPE  # K <= 32768
    assert L.tq_blockfp_gemm(2, g, g, None, 8, 48, 1, g, F32, 64, g, 8, None, 0, None) == ESHAPE     # K % 32
    assert L.tq_blockfp_gemm(2, g, g, None, 8, 64, 1, g, F16, 64, g, 8, None, 0, None) == EDTYPE
    assert L.tq_blockfp_gemm(1, _p(GOOD + 8), g, g, 8, 64, 1, g, F32, 64, g, 8, None, 0, None) == EALIGN   # NVFP4 codes: 16 B
    assert L.tq_blockfp_gemm(2, _p(GOOD + 4), g, None, 8, 64, 1, g, F32, 64, g, 8, None, 0, None) == EALIGN  # MXFP6 codes: 8 B
    # int8 transcode and GEMV
    assert L.tq_transcode_q8(g, g, 8, 64, 0, None, g, None) == EINVAL
    assert L.tq_transcode_q8(g, g, 8, 48, 0, g, g, None) == ESHAPE
    assert L.tq_transcode_q8(g, g, 8, 64, 0, _p(GOOD + 8), g, None) == EALIGN      # codes: 16 B
    assert L.tq_transcode_q8(g, g, 8, 64, 0, g, _p(GOOD + 1), None) == EALIGN      # scales: 2 B
    assert L.tq_q8_gemv(g, g, 0, 64, g, F32, g, None) == EINVAL
    assert L.tq_q8_gemv(g, g, 8, 40, g, F32, g, None) == ESHAPE
    assert L.tq_q8_gemv(g, g, 8, 32768 + 32, g, F32, g, None) == ESHAPE
    assert L.tq_q8_gemv(g, g, 8, 64, g, F16, g, None) == EDTYPE
    assert L.tq_q8_gemv(g, g, 8, 64, _p(GOOD + 8), BF16, g, None) == EALIGN      # x: 16 B
    assert L.tq_quantize(g, F32, 1, (1 << 31) + 32, (1 << 31) + 32, 0, g, g, None) == ESHAPE   # K <= 2^31
    # turbo4 KV cache and decode attention
    sg = tqa.kv_sign_from_seed(0)
    assert L.tq_kv_quantize_k(g, F32, 0, 128, g, g, None) == EINVAL
    assert L.tq_kv_quantize_k(g, F32, 4, 100, g, g, None) == ESHAPE
    assert L.tq_kv_quantize_k(g, F16, 4, 128, g, g, None) == EDTYPE
    assert L.tq_kv_quantize_k(g, F32, 4, 128, _p(GOOD + 8), g, None) == EALIGN    # codes: 16 B
    assert L.tq_kv_quantize_v(g, F32, 4, 128, None, g, g, None) == EINVAL        # sign words
    assert L.tq_kv_quantize_v(g, F32, 4, 64, sg, g, g, None) == ESHAPE           # head dim 128 only
    assert L.tq_kv_quantize_v(g, BF16, 4, 128, sg, _p(GOOD + 4), g, None) == EALIGN   # packed: 8 B
    assert L.tq_kv_dequantize_v(g, g, 4, 128, sg, _p(GOOD + 4), None) == EALIGN       # out: 16 B
    assert L.tq_attn_workspace_bytes(2, 32, 1000) == 2 * 32 * 4 * 130 * 4
    assert L.tq_attn_workspace_bytes(0, 32, 1000) == 0
    ws = L.tq_attn_workspace_bytes(1, 32, 512)
    args = lambda **kw: [kw.get("q", g), kw.get("qt", BF16), kw.get("B", 1), kw.get("Hq", 32), kw.get("Hkv", 8),
                         kw.get("d", 128), kw.get("T", 512), g, g, g, g, g, sg, g, kw.get("ws", g),
                         kw.get("wsb", ws), None]
    assert L.tq_attn_decode(*args(Hq=12)) == ESHAPE                  # Hq % Hkv
    assert L.tq_attn_decode(*args(Hq=128, Hkv=8)) == ESHAPE          # G = 16
    assert L.tq_attn_decode(*args(d=64)) == ESHAPE
    assert L.tq_attn_decode(*args(wsb=ws - 4)) == EINVAL             # workspace too small
    assert L.tq_attn_decode(*args(T=0)) == EINVAL
    big = L.tq_attn_workspace_bytes(1, 32, 1 << 31)
    assert L.tq_attn_decode(*args(T=1 << 31, wsb=big)) == ESHAPE      # T_max > INT32_MAX
    assert L.tq_attn_decode(*args(qt=F16)) == EDTYPE
    assert L.tq_attn_decode(*args(q=_p(GOOD + 8))) == EALIGN
    # decode attention without a workspace: the same checks, and problems beyond its scratch array
    nargs = lambda **kw: [kw.get("q", g), kw.get("qt", BF16), kw.get("B", 1), kw.get("Hq", 32), kw.get("Hkv", 8),
                          kw.get("d", 128), kw.get("T", 512), g, g, g, g, g, sg, g, None]
    assert L.tq_attn_decode_noalloc(*nargs(q=None)) == EINVAL
    assert L.tq_attn_decode_noalloc(*nargs(Hq=12)) == ESHAPE
    assert L.tq_attn_decode_noalloc(*nargs(B=64, T=32768)) == ESHAPE          # 34 MB of partials > 8 MiB
    assert L.tq_attn_decode_noalloc(*nargs(qt=F16)) == EDTYPE
    assert L.tq_attn_decode_noalloc(*nargs(q=_p(GOOD + 8))) == EALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        tqa.quantize(w)
    with pytest.raises(ValueError):
        tqa.gemv(torch.zeros(4, 32, dtype=torch.uint8), torch.zeros(4, 4, dtype=torch.int16), torch.zeros(64))


def test_binding_checks_tensor_shapes_before_any_call():
    """Mis-shaped, strided or mistyped weight tensors are refused by the binding itself (CPU tensors:
    the shape check comes first, so nothing reaches libtq)."""
    import torch
    N, K = 8, 64
    packed = torch.zeros(N, K // 2, dtype=torch.uint8)
    scales = torch.zeros(N, K // 16, dtype=torch.int16)
    x = torch.zeros(K)
    with pytest.raises(ValueError, match="scales: shape"):
        tqa.gemv(packed, torch.zeros(N, K // 32, dtype=torch.int16), x)
    with pytest.raises(ValueError, match="scales: dtype"):
        tqa.gemv(packed, torch.zeros(N, K // 16, dtype=torch.int32), x)
    with pytest.raises(ValueError, match="packed: dtype"):
        tqa.gemv(packed.to(torch.int8), scales, x)
    with pytest.raises(ValueError, match="packed must be contiguous"):
        tqa.gemv(torch.zeros(N, K, dtype=torch.uint8)[:, ::2], scales, x)
    with pytest.raises(ValueError, match="packed must be a 2-D"):
        tqa.dequantize(torch.zeros(N * K // 2, dtype=torch.uint8), scales)
    with pytest.raises(ValueError, match="GPU tensor"):          # well-formed, but on the CPU
        tqa.gemv(packed, scales, x)
    with pytest.raises(ValueError, match="scales: shape"):
        tqa.gemm(packed, scales[:, :2].contiguous(), torch.zeros(4, K))
    with pytest.raises(ValueError, match="scales: shape"):
        tqa.transcode_q8(packed, scales[:4])
    with pytest.raises(ValueError, match="q8_scales: shape"):
        tqa.q8_gemv(torch.zeros(N, K, dtype=torch.int8), torch.zeros(N, K // 16, dtype=torch.int16), x)
    with pytest.raises(ValueError, match="block_scales: shape"):
        tqa.blockfp_gemm("nvfp4", torch.zeros(N, K // 2, dtype=torch.uint8), torch.zeros(N, K // 32, dtype=torch.uint8),
                         torch.ones(1), x)
    with pytest.raises(ValueError, match="tensor scale"):
        tqa.blockfp_gemm("nvfp4", torch.zeros(N, K // 2, dtype=torch.uint8), torch.zeros(N, K // 16, dtype=torch.uint8),
                         None, x)
    with pytest.raises(ValueError, match="codes: shape"):
        tqa.blockfp_gemm("mxfp6", torch.zeros(N, 3 * K // 4 + 1, dtype=torch.uint8),
                         torch.zeros(N, K // 32, dtype=torch.uint8), None, x)
