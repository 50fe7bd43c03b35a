"""Pins for the oracle's RSF-lite TQ4_1S quantizer (CPU only).

Independent anchors used here (TQ4_1S half-block scales, then the NVFP4 and
MXFP6 block scales, whose grids the tests enumerate from the field layouts):
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


# ---------------------------------------------------------------------------
# block-float formats
# ---------------------------------------------------------------------------

from oracle import blockfp  # noqa: E402


def _grid(ebits, mbits, bias, drop_top=False):
    """Non-negative values of a sign-magnitude float format, in code order, from its field layout."""
    vals = []
    for e in range(1 << ebits):
        for m in range(1 << mbits):
            if e == 0:
                vals.append(m / (1 << mbits) * 2.0 ** (1 - bias))
            else:
                vals.append((1 + m / (1 << mbits)) * 2.0 ** (e - bias))
    return np.array(vals[:-1] if drop_top else vals)


E2M1_GRID = _grid(2, 1, 1)                      # 0 .. 6
E3M2_GRID = _grid(3, 2, 3)                      # 0 .. 28
E4M3_GRID = _grid(4, 3, 7, drop_top=True)       # 0 .. 448 (S.1111.111 is NaN)


def _nearest_code(a, grid):
    """Nearest grid index to |a| (float64), ties to the even index, saturating at the top."""
    a = np.minimum(np.abs(np.asarray(a, np.float64)), grid[-1])
    d = np.abs(a[..., None] - grid)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(len(grid)), len(grid) + 1)
    even = np.where(cand % 2 == 0, cand, len(grid) + 1).min(axis=-1)
    return np.where(even <= len(grid), even, cand.min(axis=-1))


def _signed_nearest(x, grid):
    return np.sign(x) * grid[_nearest_code(x, grid)]


def _weights(seed, n=24, k=256):
    rng = np.random.default_rng(seed)
    return np.concatenate([rng.standard_normal((n // 2, k)) * 0.02,
                           rng.standard_t(4, (n - n // 2, k)) * 0.02]).astype(np.float32)


def _nv_block_err64(W, packed, sb, st):
    deq = blockfp.nvfp4_dequantize_o64(packed, sb, st)
    return ((deq - W.astype(np.float64)) ** 2).reshape(W.shape[0], -1, 16).sum(axis=-1)


def test_nvfp4_choice_is_the_float64_minimum_and_never_worse_than_plain():
    W = _weights(10)
    packed, sb, st = rsf.nvfp4_quantize_rsf_o32(W)
    p0, sb0, st0 = blockfp.nvfp4_quantize_o32(W)
    assert st == st0
    chosen = _nv_block_err64(W, packed, sb, st)
    plain = _nv_block_err64(W, p0, sb0, st0)
    assert np.all(chosen <= plain * (1 + 1e-5) + 1e-30)
    # every candidate scale (plain scale times 1 + j/16, re-rounded to E4M3), brute force in float64
    blocks = W.astype(np.float64).reshape(W.shape[0], -1, 16)
    base = E4M3_GRID[sb0]
    best = np.full(chosen.shape, np.inf)
    for j in range(-4, 5):
        eff = E4M3_GRID[_nearest_code(base * (1 + j / 16), E4M3_GRID)] * float(st)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = np.where(eff[..., None] > 0, blocks / eff[..., None], 0.0)
        deq = _signed_nearest(t, E2M1_GRID) * eff[..., None]
        best = np.minimum(best, ((deq - blocks) ** 2).sum(axis=-1))
    assert np.all(chosen <= best * (1 + 1e-5) + 1e-30)
    assert chosen.sum() < 0.95 * plain.sum()


def test_nvfp4_plain_reproduced_where_base_wins_and_zero_tensor():
    W = _weights(11)
    packed, sb, st = rsf.nvfp4_quantize_rsf_o32(W)
    p0, sb0, _ = blockfp.nvfp4_quantize_o32(W)
    same = sb == sb0
    assert same.any() and (~same).any()
    c1 = np.stack([packed & 15, packed >> 4], -1).reshape(W.shape[0], -1, 16)
    c0 = np.stack([p0 & 15, p0 >> 4], -1).reshape(W.shape[0], -1, 16)
    assert np.array_equal(c1[same], c0[same])
    z = rsf.nvfp4_quantize_rsf_o32(np.zeros((2, 32), np.float32))
    assert not z[0].any() and not z[1].any() and z[2] == 0


def test_mxfp6_clipped_outlier_takes_the_next_exponent():
    """A block holding one value 31.5 * 2^e (others 0): the plain exponent e clips it to 28 * 2^e
    (error 3.5 * 2^e); exponent e + 1 rounds it to 16 * 2^(e+1) = 32 * 2^e (error 0.5 * 2^e)."""
    k = 64
    W = np.zeros((3, k), np.float32)
    for r, (e, pos) in enumerate([(0, 5), (-10, 31), (6, 0)]):
        W[r, pos] = np.float32(31.5 * 2.0 ** e)
        W[r, 32 + pos] = np.float32(-1.5 * 2.0 ** e)       # a second block that is exact at its own e
    codes, byte = rsf.mxfp6_quantize_rsf_o32(W)
    c0, byte0 = blockfp.mxfp6_quantize_o32(W)
    deq = blockfp.mxfp6_dequantize_o64(codes, byte)
    for r, (e, pos) in enumerate([(0, 5), (-10, 31), (6, 0)]):
        assert byte[r, 0] == byte0[r, 0] + 1
        assert deq[r, pos] == 32 * 2.0 ** e and not np.delete(deq[r, :32], pos).any()
        assert byte[r, 1] == byte0[r, 1] and deq[r, 32 + pos] == -1.5 * 2.0 ** e
    assert np.array_equal(blockfp.mxfp6_dequantize_o64(c0, byte0)[0, 5], 28.0)


def test_mxfp6_choice_is_the_float64_minimum_and_never_worse_than_plain():
    W = _weights(12)
    codes, byte = rsf.mxfp6_quantize_rsf_o32(W)
    c0, byte0 = blockfp.mxfp6_quantize_o32(W)
    blocks = W.astype(np.float64).reshape(W.shape[0], -1, 32)
    err = lambda c, b: ((blockfp.mxfp6_dequantize_o64(c, b).reshape(blocks.shape) - blocks) ** 2).sum(-1)
    chosen, plain = err(codes, byte), err(c0, byte0)
    assert np.all(chosen <= plain * (1 + 1e-6))
    best = np.full(chosen.shape, np.inf)
    for j in (-1, 0, 1):
        s = 2.0 ** (byte0.astype(np.float64) - 127 + j)
        deq = _signed_nearest(blocks / s[..., None], E3M2_GRID) * s[..., None]
        best = np.minimum(best, ((deq - blocks) ** 2).sum(-1))
    assert np.all(chosen <= best * (1 + 1e-6))
    assert np.all(np.abs(byte.astype(int) - byte0) <= 1) and chosen.sum() < plain.sum()


def test_mistake_keeping_the_worse_block_candidate_is_caught(monkeypatch):
    def keep_worse(best, cand):
        if best is None:
            return cand
        take = cand[0] > best[0]
        return (np.where(take, cand[0], best[0]), np.where(take, cand[1], best[1]),
                np.where(take[..., None], cand[2], best[2]))

    monkeypatch.setattr(rsf, "_keep_better", keep_worse)
    assert _fails(test_nvfp4_choice_is_the_float64_minimum_and_never_worse_than_plain)
    assert _fails(test_mxfp6_choice_is_the_float64_minimum_and_never_worse_than_plain,
                  test_mxfp6_clipped_outlier_takes_the_next_exponent)


def test_mistake_dropping_the_block_base_candidate_is_caught(monkeypatch):
    monkeypatch.setattr(rsf, "ORDER", (-1, 1, -2, 2, -3, 3, -4, 4))
    monkeypatch.setattr(rsf, "MX_ORDER", (-1, 1))
    assert _fails(test_nvfp4_choice_is_the_float64_minimum_and_never_worse_than_plain,
                  test_nvfp4_plain_reproduced_where_base_wins_and_zero_tensor)
    assert _fails(test_mxfp6_choice_is_the_float64_minimum_and_never_worse_than_plain)
