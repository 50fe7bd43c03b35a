"""Pins for the oracle's RSF-lite TQ4_1S quantizer (CPU only).

Independent anchors used here:
* a float64 recomputation of every candidate's error: the chosen scale is
  the float64 minimiser except within float32 rounding of a tie, and never
  worse than the plain quantizer's scale;
* a constructed half whose rotated values lie exactly on the lattice of a
  non-base candidate: the search must find it with zero error;
* the plain quantizer is reproduced where the multiplier-1 candidate wins;
* planted mistakes (keeping the worst candidate, dropping the base) fail.
"""

import numpy as np

from oracle import codebook as cb
from oracle import rsf
from oracle import tq4_1s as tq

C32 = cb.tq4_codebook_f32()
C64 = C32.astype(np.float64)
M32 = cb.tq4_midpoints_f32(C32)


def _halves_and_choice(W):
    packed, scales, wr, err = rsf.quantize_rsf_o32(W, return_parts=True)
    n, nb, _ = wr.shape
    idx = tq.unpack_nibbles(packed).reshape(n, nb, 2, 16)
    d = tq.fp16_bits_to_f32(scales).astype(np.float64).reshape(n, nb, 2)
    return wr.reshape(n, nb, 2, 16).astype(np.float64), idx, d


def _err64(h, d, idx):
    return ((h - d[..., None] * C64[idx]) ** 2).sum(axis=-1)


def test_choice_is_the_float64_minimum_and_never_worse_than_plain():
    rng = np.random.default_rng(0)
    W = np.concatenate([rng.standard_normal((16, 512)) * 0.02,
                        rng.standard_t(4, (16, 512)) * 0.02]).astype(np.float32)
    h, idx, d = _halves_and_choice(W)
    chosen = _err64(h, d, idx)
    # plain quantizer's error
    p0, s0 = tq.quantize_o32(W)
    i0 = tq.unpack_nibbles(p0).reshape(idx.shape)
    d0 = tq.fp16_bits_to_f32(s0).astype(np.float64).reshape(d.shape)
    plain = _err64(h, d0, i0)
    assert np.all(chosen <= plain * (1 + 1e-5) + 1e-30)
    # every candidate, recomputed in float64 with brute-force nearest centroids
    best = np.full(chosen.shape, np.inf)
    for j in rsf.ORDER:
        dj = tq.fp16_sat((d0.astype(np.float32) * rsf.multiplier(j)).astype(np.float32)).astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = np.where(dj[..., None] > 0, h / dj[..., None], 0.0)
        ij = np.abs(t[..., None] - C64).argmin(axis=-1)
        best = np.minimum(best, _err64(h, dj, ij))
    assert np.all(chosen <= best * (1 + 1e-5) + 1e-30)
    # and the search pays: a few percent less squared error on these weights
    assert chosen.sum() < 0.99 * plain.sum()


def test_exact_lattice_fit_of_a_non_base_candidate_is_found():
    """Rotated halves built as fl(t * c[k_i]) for an fp16 t that equals a non-base candidate of
    their own plain scale (fp16 of the half's RMS): the search returns scale t, indices k_i and
    zero error, while the plain scale does not fit exactly."""
    rng = np.random.default_rng(1)
    found = 0
    for _ in range(4000):
        k = rng.integers(0, 16, 16)
        t = np.float16(rng.uniform(0.05, 0.2))
        h = (np.float32(t) * C32[k]).astype(np.float32)
        ss = rsf._pairwise_sum16((h * h).astype(np.float32))
        d0 = tq.fp16_sat(np.sqrt((ss * np.float32(0.0625)).astype(np.float32))).astype(np.float32)
        hits = [j for j in rsf.ORDER[1:] if tq.fp16_sat((d0 * rsf.multiplier(j)).astype(np.float32)) == t]
        if not hits or np.float16(d0) == t:
            continue
        d, idx, err = rsf.search_halves(h[None], np.array([d0], np.float32), C32, M32)
        assert d[0] == t and np.array_equal(idx[0], k.astype(np.uint8)) and err[0] == 0.0
        found += 1
        if found >= 5:
            break
    assert found >= 5


def test_plain_quantizer_reproduced_where_base_wins():
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    packed, scales = rsf.quantize_rsf_o32(W)
    p0, s0 = tq.quantize_o32(W)
    same = scales == s0
    i1 = tq.unpack_nibbles(packed).reshape(32, 16, 16)
    i0 = tq.unpack_nibbles(p0).reshape(32, 16, 16)
    assert same.any() and (~same).any()
    assert np.array_equal(i1[same], i0[same])
    assert np.array_equal(rsf.quantize_rsf_o32(np.zeros((2, 64), np.float32))[1], np.zeros((2, 4), np.uint16))


def _fails(*tests):
    for t in tests:
        try:
            t()
        except AssertionError:
            return True
    return False


def test_mistake_keeping_the_worst_candidate_is_caught(monkeypatch):
    real = rsf.half_error_f32
    monkeypatch.setattr(rsf, "half_error_f32", lambda *a: -real(*a))
    assert _fails(test_choice_is_the_float64_minimum_and_never_worse_than_plain)


def test_mistake_dropping_the_base_candidate_is_caught(monkeypatch):
    monkeypatch.setattr(rsf, "ORDER", (-1, 1, -2, 2, -3, 3, -4, 4))
    assert _fails(test_choice_is_the_float64_minimum_and_never_worse_than_plain,
                  test_plain_quantizer_reproduced_where_base_wins)
