"""GPU parity of the turbo4 KV cache and its decode attention against the CPU oracle (through the C ABI).

* key encode (q8_0 rows) and value encode (turbo4): bit-exact against the oracle's canonical float32 order
  (ragged counts, bf16 and float32, sign words, edge vectors);
* value decode: within float32 rounding of the float64 decode;
* decode attention: |do| <= 1e-3 * sum_t p_t (nn_t / 128) sum_j |c[idx_tj]| (the largest magnitude an output
  coordinate's terms reach) against the oracle on the GPU's own cache bytes, for GQA groups 1, 2, 4, 8, ragged
  lengths (0, 1, split boundaries, T_max), bf16 and float32 queries, and the Llama-3-8B head layout at 8K tokens.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa
from oracle import kv as okv
import workloads
from gpu_helpers import say, u16, f32np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def _rand(shape, seed, dtype, scale=1.0):
    g = workloads.generator(seed, DEV)
    return (torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) * scale).to(dtype)


@pytest.mark.parametrize("n,d", [(1, 128), (7, 32), (1000, 128), (33, 96)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_quantize_k_bit_exact(n, d, dtype):
    K = _rand((n, d), 10 + n + d, dtype, 0.7)
    say(f"[kv k] n={n} d={d} {dtype}")
    codes, scales = tqa.kv_quantize_k(K)
    torch.cuda.synchronize()
    oc, os_ = okv.q8_0_quantize_o32(K.float().cpu().numpy())
    np.testing.assert_array_equal(u16(scales), os_)
    np.testing.assert_array_equal(codes.cpu().numpy(), oc)


def test_kv_encode_into_given_outputs():
    K = _rand((3, 2, 50, D), 15, torch.bfloat16)
    kc, ks = tqa.kv_quantize_k(K)
    vp, vn = tqa.kv_quantize_v(K)
    out_k = (torch.full_like(kc, 7), torch.full_like(ks, 7))
    out_v = (torch.full_like(vp, 7), torch.full_like(vn, 7))
    say("[kv] encode into given outputs")
    tqa.kv_quantize_k(K, out=out_k)
    tqa.kv_quantize_v(K, out=out_v)
    torch.cuda.synchronize()
    assert torch.equal(out_k[0], kc) and torch.equal(out_k[1], ks)
    assert torch.equal(out_v[0], vp) and torch.equal(out_v[1], vn)


def _edge_vectors():
    V = np.zeros((8, D), np.float32)
    V[1, 17] = -3.25                                     # a single spike
    V[2, :] = 1.0                                        # a constant vector
    V[3, :] = np.linspace(-2, 2, D)
    V[4, :64] = 1e4                                      # norm above fp16's range: saturates at 65504
    V[5, :] = 1e-6                                       # tiny norm (fp16 subnormal)
    V[6, ::2] = 0.5
    V[6, 1::2] = -0.5
    V[7, 5] = 2.0 ** -24                                 # norm at fp16's smallest subnormal
    return V


@pytest.mark.parametrize("n", [1, 9, 4099])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_turbo4_encode_bit_exact(n, dtype):
    V = _rand((n, D), 20 + n, dtype)
    for seed in (0, 5):
        sign = tqa.kv_sign_from_seed(seed)
        say(f"[turbo4 encode] n={n} {dtype} seed={seed}")
        packed, norms = tqa.kv_quantize_v(V, sign)
        torch.cuda.synchronize()
        op, on = okv.turbo4_quantize_o32(V.float().cpu().numpy(), okv.kv_sign_words(seed))
        np.testing.assert_array_equal(u16(norms), on)
        np.testing.assert_array_equal(packed.cpu().numpy(), op)


def test_turbo4_encode_edge_vectors_and_sign_words():
    V = torch.from_numpy(_edge_vectors()).to(DEV)
    for words in ([0, 0, 0, 0], [0xFFFFFFFF] * 4, okv.kv_sign_words(9)):
        sign = (tqa.ctypes.c_uint32 * 4)(*words)
        say(f"[turbo4 encode] edge vectors, words={[hex(w) for w in words]}")
        packed, norms = tqa.kv_quantize_v(V, sign)
        torch.cuda.synchronize()
        op, on = okv.turbo4_quantize_o32(V.cpu().numpy(), words)
        np.testing.assert_array_equal(u16(norms), on)
        np.testing.assert_array_equal(packed.cpu().numpy(), op)


def test_turbo4_decode():
    V = _rand((2048, D), 30, torch.float32)
    packed, norms = tqa.kv_quantize_v(V)
    out = tqa.kv_dequantize_v(packed, norms)
    torch.cuda.synchronize()
    ref = okv.turbo4_dequantize_o64(packed.cpu().numpy(), u16(norms))
    nn = okv.fp16_bits_to_f32(u16(norms)).astype(np.float64)
    cabs = np.abs(okv.codebook.tq4_codebook_f32().astype(np.float64)[okv.turbo4_indices(packed.cpu().numpy())])
    bound = (nn / D * cabs.sum(1))[:, None]
    err = np.abs(f32np(out) - ref)
    assert np.all(err <= 1e-6 * bound), float((err / bound).max())


def _cache(B, T, Hkv, seed, dtype=torch.bfloat16):
    K = _rand((B, Hkv, T, D), seed, dtype)
    V = _rand((B, Hkv, T, D), seed + 1, dtype)
    kc, ks = tqa.kv_quantize_k(K)
    vp, vn = tqa.kv_quantize_v(V)
    return kc, ks, vp, vn


def _check_attn(q, lengths, cache, label):
    kc, ks, vp, vn = cache
    say(f"[attn] {label} q={tuple(q.shape)} {q.dtype} lengths={lengths.tolist()} T_max={kc.shape[2]}")
    o = tqa.attn_decode(q, lengths, kc, ks, vp, vn)
    torch.cuda.synchronize()
    ref, bound = okv.attn_decode_o64(q.float().cpu().numpy(), lengths.cpu().numpy(), kc.cpu().numpy(), u16(ks),
                                     vp.cpu().numpy(), u16(vn))
    got = f32np(o)
    err = np.abs(got - ref)
    lim = 1e-3 * bound[..., None]
    bad = err > lim
    assert not bad.any(), f"{label}: {bad.sum()} outside; worst ratio {(err / np.maximum(lim, 1e-300)).max()}"
    worst = float((err / np.maximum(bound[..., None], 1e-300)).max())
    say(f"[attn] {label}: worst |do| / bound = {worst:.2e}")
    return o, worst


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 8), (32, 8), (64, 8), (12, 3)])
@pytest.mark.parametrize("qdtype", [torch.bfloat16, torch.float32])
def test_attn_decode_groups_and_lengths(Hq, Hkv, qdtype):
    B, T = 5, 600
    cache = _cache(B, T, Hkv, 40 + Hq)
    q = _rand((B, Hq, D), 50 + Hq, qdtype, 2.0)
    lengths = torch.tensor([600, 1, 256, 257, 513], dtype=torch.int32, device=DEV)
    _, worst = _check_attn(q, lengths, cache, f"Hq={Hq} Hkv={Hkv}")
    assert worst < 1e-4


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 4)])
@pytest.mark.parametrize("spread", ["tiny", "large", "mixed"])
def test_attn_decode_value_norm_range(Hq, Hkv, spread):
    """Value sums on the matrix cores (four or more query heads per cache head) take fp16 weights scaled per
    wavefront by a power of two: value norms of about 1e-4 everywhere, about 1e4 everywhere, and spread
    over ten decades within one 256-token chunk stay within the bound."""
    B, T = 2, 700
    V = _rand((B, Hkv, T, D), 91, torch.float32)
    if spread == "tiny":
        V = V * 1e-5
    elif spread == "large":
        V = V * 1e3
    else:
        g = torch.Generator(device=DEV)
        g.manual_seed(92)
        V = V * torch.pow(10.0, torch.rand((B, Hkv, T, 1), generator=g, device=DEV) * 10.0 - 7.0)
    K = _rand((B, Hkv, T, D), 90, torch.bfloat16)
    kc, ks = tqa.kv_quantize_k(K)
    vp, vn = tqa.kv_quantize_v(V.to(torch.bfloat16).contiguous())
    q = _rand((B, Hq, D), 93, torch.bfloat16, 1.5)
    lengths = torch.tensor([700, 301], dtype=torch.int32, device=DEV)
    _, worst = _check_attn(q, lengths, (kc, ks, vp, vn), f"norms {spread} Hq={Hq} Hkv={Hkv}")
    assert worst < 1e-4


def test_attn_decode_zero_length_and_peaked_scores():
    B, T, Hq, Hkv = 3, 300, 32, 8
    kc, ks, vp, vn = _cache(B, T, Hkv, 60)
    q = _rand((B, Hq, D), 61, torch.bfloat16, 40.0)      # large scores: nearly one-hot softmax
    lengths = torch.tensor([0, 300, 17], dtype=torch.int32, device=DEV)
    o, _ = _check_attn(q, lengths, (kc, ks, vp, vn), "peaked")
    assert not o[0].any()
    # repeat runs are bit-identical
    o2 = tqa.attn_decode(q, lengths, kc, ks, vp, vn)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)


def test_attn_decode_llama8b_heads_8k():
    """The Llama-3-8B attention layout (32 query heads, 8 cache heads, head dim 128) at 8K cached tokens."""
    B, T, Hq, Hkv = 2, 8192, 32, 8
    cache = _cache(B, T, Hkv, 70)
    q = _rand((B, Hq, D), 71, torch.bfloat16, 1.5)
    lengths = torch.tensor([8192, 3001], dtype=torch.int32, device=DEV)
    _, worst = _check_attn(q, lengths, cache, "llama8b 8K")
    assert worst < 1e-4


def test_attn_decode_many_splits_32k():
    """32768 cached tokens: 128 splits per sequence in the combine (its split loop in groups of eight), with a
    ragged second sequence (20001 tokens: a partial last split)."""
    B, T, Hq, Hkv = 2, 32768, 8, 2
    cache = _cache(B, T, Hkv, 80)
    q = _rand((B, Hq, D), 81, torch.bfloat16, 1.5)
    lengths = torch.tensor([32768, 20001], dtype=torch.int32, device=DEV)
    _, worst = _check_attn(q, lengths, cache, "32K tokens")
    assert worst < 1e-4


def test_kv_encode_rejects_malformed_outputs():
    """Given outputs of the wrong dtype, shape or layout are refused before anything launches (a strided
    view would otherwise be written as if dense)."""
    K = _rand((2, 3, 40, D), 16, torch.bfloat16)
    kc, ks = tqa.kv_quantize_k(K)
    vp, vn = tqa.kv_quantize_v(K)
    with pytest.raises(ValueError, match="dtype"):
        tqa.kv_quantize_k(K, out=(kc.to(torch.int16), ks))
    with pytest.raises(ValueError, match="contiguous"):
        wide = torch.empty((2, 3, 40, 2 * D), dtype=torch.int8, device=DEV)
        tqa.kv_quantize_k(K, out=(wide[..., :D], ks))
    with pytest.raises(ValueError, match="shape"):
        tqa.kv_quantize_k(K, out=(kc, ks[..., :2].contiguous()))
    with pytest.raises(ValueError, match="contiguous"):
        wide = torch.empty((2, 3, 40, D), dtype=torch.uint8, device=DEV)
        tqa.kv_quantize_v(K, out=(wide[..., :D // 2], vn))
    with pytest.raises(ValueError, match="dtype"):
        tqa.kv_quantize_v(K, out=(vp, vn.to(torch.float32)))
    torch.cuda.synchronize()
