"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each.

Each case monkeypatches one oracle function with a wrong variant (a dropped
term, a misplaced sign matrix, a swapped index or operand) and re-runs pin
tests from the other oracle test modules; at least one must fail.
"""

import numpy as np
import pytest

from oracle import tq4_1s as tq
from oracle import blockfp as bf
import test_oracle_quantize as tqz
import test_oracle_rotation as trot
import test_oracle_blockfp as tbf


def _fails(*tests):
    for t in tests:
        try:
            t()
        except AssertionError:
            return True
    return False


def test_d_after_h_is_caught(monkeypatch):
    real = tq.rotate_f32

    def wrong(blocks, sign_mask):       # D applied after the transform instead of before
        w = np.asarray(blocks, np.float32)
        flip = ((int(sign_mask) >> np.arange(32)) & 1).astype(bool)
        u = tq.fwht32_f32(w) * tq.S32
        return np.where(flip, -u, u).astype(np.float32)

    monkeypatch.setattr(tq, "rotate_f32", wrong)
    assert _fails(tqz.test_single_spike_closed_form_bit_exact, tqz.test_nibble_order_and_scale_slots)
    monkeypatch.setattr(tq, "rotate_f32", real)


def test_missing_normalisation_is_caught(monkeypatch):
    monkeypatch.setattr(tq, "S32", np.float32(1.0))
    assert _fails(tqz.test_single_spike_closed_form_bit_exact, tqz.test_reconstruction_error_near_codebook_distortion)


def test_swapped_nibbles_are_caught(monkeypatch):
    monkeypatch.setattr(tq, "pack_nibbles", lambda idx: (np.asarray(idx, np.uint8)[:, 1::2] | (np.asarray(idx, np.uint8)[:, 0::2] << 4)).astype(np.uint8))
    assert _fails(tqz.test_single_spike_closed_form_bit_exact, tqz.test_nibble_order_and_scale_slots)


def test_non_strict_threshold_is_caught(monkeypatch):
    real = tq.quantize_o32

    def wrong(W, sign_mask=tq.DEFAULT_SIGN_MASK, centroids32=None, return_parts=False):
        out = real(W, sign_mask, centroids32, return_parts=True)
        packed, scales, wr, dd, idx = out
        # off-by-one: count thresholds at or below (index shifted up by one)
        idx = np.minimum(idx.astype(np.int64) + 1, 15).astype(np.uint8)
        packed = tq.pack_nibbles(idx)
        return (packed, scales, wr, dd, idx) if return_parts else (packed, scales)

    monkeypatch.setattr(tq, "quantize_o32", wrong)
    assert _fails(tqz.test_single_spike_closed_form_bit_exact, tqz.test_brute_force_nearest_on_tiny_blocks)


def test_transposed_hadamard_product_is_caught(monkeypatch):
    real = tq.hadamard
    monkeypatch.setattr(tq, "hadamard", lambda n=32: real(n)[::-1])   # rows permuted
    assert _fails(trot.test_hadamard_definition, trot.test_rotation_is_orthogonal_and_inverts)


def test_nvfp4_wrong_tensor_scale_is_caught(monkeypatch):
    monkeypatch.setattr(bf, "E4M3_MAX", 240.0)                        # e.g. the E4M3FNUZ max
    assert _fails(tbf.test_nvfp4_closed_form_scales)


def test_mxfp6_wrong_emax_is_caught(monkeypatch):
    monkeypatch.setattr(bf, "E3M2_EMAX", 2)
    assert _fails(tbf.test_mxfp6_closed_form_scale)


def test_gemm_deq_transposed_product_is_caught(monkeypatch):
    real = bf.gemm_deq_o64

    def wrong(W_deq, X):                # W_deq used untransposed (a square-only mistake)
        Xa = np.atleast_2d(np.asarray(X, dtype=np.float64))
        Wt = np.asarray(W_deq).reshape(W_deq.shape[1], W_deq.shape[0])
        return Xa @ Wt, np.abs(Xa) @ np.abs(Wt)

    monkeypatch.setattr(bf, "gemm_deq_o64", wrong)
    assert _fails(tbf.test_gemm_deq_tiny_explicit_loop,
                  lambda: tbf.test_gemm_deq_one_hot_selects_columns("nvfp4"))
    monkeypatch.setattr(bf, "gemm_deq_o64", real)


def test_gemm_deq_dropped_abs_is_caught(monkeypatch):
    def wrong(W_deq, X):                # the tolerance scale without absolute values
        Xa = np.atleast_2d(np.asarray(X, dtype=np.float64))
        return Xa @ W_deq.T, np.abs(Xa @ W_deq.T)

    monkeypatch.setattr(bf, "gemm_deq_o64", wrong)
    assert _fails(tbf.test_gemm_deq_zero_weights_and_scale_bounds, tbf.test_gemm_deq_tiny_explicit_loop)
