"""Pins for the oracle's turbo4 / q8_0 KV cache and its decode attention (CPU only).

Independent anchors used here:
* the codebook's own distortion: a rotated Gaussian vector's coordinates are
  close to N(0, 1), so the relative squared error of turbo4 must be close to
  D_16 (any slip in the rotation, its inverse, the signs or the norm breaks
  this by orders of magnitude);
* closed forms: a single spike a e_j decodes to c_11 * a e_j; the decoded
  norm is nn * ||c[idx]|| / sqrt(d) (the rotation is orthogonal);
* brute-force nearest centroids and fp16 rounding of the norm in float64;
* attention: explicit Python loops on tiny inputs, one cached token gives
  its value vector, a zero query gives the mean, tokens past the length are
  ignored, the bound covers every output coordinate;
* planted mistakes (signs left out of the decode, a wrong head mapping, a
  wrong score scale) fail.
"""

import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import kv
from oracle import q8
from oracle import tq4_1s as tq

C32 = cb.tq4_codebook_f32()
D = kv.HEAD_DIM


def _v(n, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((n, D)) * scale).astype(np.float32)


def test_sign_words_follow_splitmix64():
    a, b = tq.splitmix64(7, 2)
    w = kv.kv_sign_words(7)
    assert w == [a & 0xFFFFFFFF, a >> 32, b & 0xFFFFFFFF, b >> 32]
    s = kv.kv_sign_vector(w)
    assert s[0] == (-1.0 if a & 1 else 1.0) and s[64] == (-1.0 if b & 1 else 1.0) and s[127] == (-1.0 if b >> 63 else 1.0)


def test_turbo4_distortion_matches_the_codebook():
    V = _v(4096, 1, 0.3)
    p, n = kv.turbo4_quantize_o32(V)
    Vh = kv.turbo4_dequantize_o64(p, n)
    rel = ((Vh - V) ** 2).sum(1).mean() / (V.astype(np.float64) ** 2).sum(1).mean()
    d16 = cb.distortion([float(c) for c in C32])
    assert abs(rel - d16) < 0.05 * d16


def test_turbo4_single_spike_closed_form():
    rng = np.random.default_rng(2)
    V = np.zeros((40, D), np.float32)
    js = rng.integers(0, D, 40)
    amps = (rng.uniform(0.01, 50, 40) * rng.choice([-1, 1], 40)).astype(np.float32)
    V[np.arange(40), js] = amps
    p, n = kv.turbo4_quantize_o32(V)
    Vh = kv.turbo4_dequantize_o64(p, n)
    nn = tq.fp16_bits_to_f32(n).astype(np.float64)
    want = np.zeros((40, D))
    want[np.arange(40), js] = np.sign(amps) * nn * float(C32[11])
    np.testing.assert_allclose(Vh, want, rtol=0, atol=1e-12 * np.abs(amps).max())


def test_turbo4_norm_indices_and_decoded_length():
    V = _v(512, 3, 2.0)
    p, n, u, idx = kv.turbo4_quantize_o32(V, return_parts=True)
    norm64 = np.sqrt((V.astype(np.float64) ** 2).sum(1))
    nn = tq.fp16_bits_to_f32(n).astype(np.float64)
    # fp16 rounding of the norm: within half an fp16 ulp (plus the float32 sum's rounding)
    ulp = 2.0 ** (np.floor(np.log2(norm64)) - 10)
    assert np.all(np.abs(nn - norm64) <= 0.5 * ulp * (1 + 1e-5))
    # indices: nearest centroid of u / nn by brute force, away from float32 rounding of a midpoint
    t = u.astype(np.float64) / nn[:, None]
    dist = np.abs(t[..., None] - C32.astype(np.float64))
    near = dist.argmin(axis=-1)
    srt = np.sort(dist, axis=-1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-5
    assert clear.mean() > 0.99 and np.array_equal(idx[clear], near[clear])
    # u is H D w: the unnormalised rotation keeps sum u^2 = d * ||w||^2
    np.testing.assert_allclose((u.astype(np.float64) ** 2).sum(1), D * norm64 ** 2, rtol=1e-5)
    # the decode is an orthogonal map of c / sqrt(d), scaled by the norm
    Vh = kv.turbo4_dequantize_o64(p, n)
    cn = np.sqrt((C32.astype(np.float64)[kv.turbo4_indices(p)] ** 2).sum(1))
    np.testing.assert_allclose(np.sqrt((Vh ** 2).sum(1)), nn * cn / math.sqrt(D), rtol=1e-12)


def test_q8_0_keys():
    K = _v(64, 4, 0.5)
    codes, s = kv.q8_0_quantize_o32(K)
    dd = tq.fp16_bits_to_f32(s).astype(np.float64)
    blocks = K.astype(np.float64).reshape(64, 4, 32)
    c = codes.astype(np.float64).reshape(64, 4, 32)
    top = np.take_along_axis(c, np.abs(blocks).argmax(-1)[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.abs(c * dd[..., None] - blocks) <= 0.5 * dd[..., None] * (1 + 1e-6))


def _cache(B, T, Hkv, seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    kc, ks = kv.q8_0_quantize_o32(K.reshape(-1, D))
    vp, vn = kv.turbo4_quantize_o32(V.reshape(-1, D))
    return (kc.reshape(B, Hkv, T, D), ks.reshape(B, Hkv, T, D // 32), vp.reshape(B, Hkv, T, D // 2),
            vn.reshape(B, Hkv, T))


def _attn_loops(q, lengths, kc, ks, vp, vn):
    """The definition with explicit loops (float64, math.exp)."""
    B, Hq, _ = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(lengths[b])
        for h in range(Hq):
            g = h // G
            qc, dq = q8.quantize_act_q8(q[b, h])
            s = []
            for t in range(L):
                tot = 0.0
                for blk in range(D // 32):
                    isum = 0
                    for i in range(32):
                        isum += int(qc[32 * blk + i]) * int(kc[b, g, t, 32 * blk + i])
                    tot += float(dq[blk]) * float(tq.fp16_bits_to_f32(ks[b, g, t, blk:blk + 1])[0]) * isum
                s.append(tot / math.sqrt(D))
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            vh = kv.turbo4_dequantize_o64(vp[b, g, :L], vn[b, g, :L])
            for t in range(L):
                o[b, h] += e[t] / sum(e) * vh[t]
    return o


def test_attention_against_explicit_loops():
    B, T, Hq, Hkv = 2, 6, 4, 2
    cache = _cache(B, T, Hkv, 5)
    q = np.random.default_rng(6).standard_normal((B, Hq, D)).astype(np.float32) * 2
    lengths = np.array([3, 6])
    o, bound = kv.attn_decode_o64(q, lengths, *cache)
    np.testing.assert_allclose(o, _attn_loops(q, lengths, *cache), rtol=0, atol=1e-12)
    assert np.all(np.abs(o) <= bound[..., None] * (1 + 1e-12))


def test_attention_closed_forms():
    B, T, Hq, Hkv = 1, 9, 8, 2
    kc, ks, vp, vn = _cache(B, T, Hkv, 7)
    q = np.random.default_rng(8).standard_normal((B, Hq, D)).astype(np.float32)
    vh = kv.turbo4_dequantize_o64(vp.reshape(-1, D // 2), vn.reshape(-1)).reshape(B, Hkv, T, D)
    # one cached token: the output is its value vector
    o, _ = kv.attn_decode_o64(q, np.array([1]), kc, ks, vp, vn)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], vh[0, h // 4, 0], rtol=0, atol=1e-12)
    # a zero query: equal scores, the mean of the values
    o, _ = kv.attn_decode_o64(np.zeros_like(q), np.array([T]), kc, ks, vp, vn)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], vh[0, h // 4, :].mean(0), rtol=0, atol=1e-12)
    # tokens past the length are ignored
    o1, _ = kv.attn_decode_o64(q, np.array([5]), kc, ks, vp, vn)
    kc2, ks2, vp2, vn2 = kc.copy(), ks.copy(), vp.copy(), vn.copy()
    kc2[:, :, 5:] = 99
    vp2[:, :, 5:] = 0xAB
    o2, _ = kv.attn_decode_o64(q, np.array([5]), kc2, ks2, vp2, vn2)
    assert np.array_equal(o1, o2)
    # a zero length gives zeros
    o, _ = kv.attn_decode_o64(q, np.array([0]), kc, ks, vp, vn)
    assert not o.any()


def _fails(*tests):
    for t in tests:
        try:
            t()
        except AssertionError:
            return True
    return False


def test_mistake_decode_without_signs_is_caught(monkeypatch):
    real = kv.turbo4_dequantize_o64
    monkeypatch.setattr(kv, "turbo4_dequantize_o64", lambda p, n, words=None, c=None: real(p, n, [0, 0, 0, 0], c))
    assert _fails(test_turbo4_distortion_matches_the_codebook, test_turbo4_single_spike_closed_form)


def test_mistake_wrong_head_mapping_is_caught(monkeypatch):
    real = kv.attn_decode_o64

    def wrong(q, lengths, kc, ks, vp, vn, words=None, c=None):
        # cache head h % Hkv instead of h // G
        Hq, Hkv = q.shape[1], kc.shape[1]
        perm = np.array([h % Hkv for h in range(Hq)])
        o = np.zeros((q.shape[0], Hq, D))
        bd = np.zeros((q.shape[0], Hq))
        for h in range(Hq):
            oo, bb = real(q[:, h:h + 1], lengths, kc[:, perm[h]:perm[h] + 1], ks[:, perm[h]:perm[h] + 1],
                          vp[:, perm[h]:perm[h] + 1], vn[:, perm[h]:perm[h] + 1], words, c)
            o[:, h], bd[:, h] = oo[:, 0], bb[:, 0]
        return o, bd

    monkeypatch.setattr(kv, "attn_decode_o64", wrong)
    assert _fails(test_attention_against_explicit_loops, test_attention_closed_forms)


@pytest.mark.parametrize("wrong", [lambda d: 1.0, lambda d: 1.0 / d])
def test_mistake_wrong_score_scale_is_caught(monkeypatch, wrong):
    """Scores not divided by sqrt(d), or divided by d: the explicit loops disagree."""
    monkeypatch.setattr(kv, "score_scale", wrong)
    assert _fails(test_attention_against_explicit_loops)
