"""Shared helpers for the GPU parity tests (host-side conversions and input builders)."""

import sys

import numpy as np
import torch

from oracle import codebook as ocb
from oracle import tq4_1s as otq

C32 = ocb.tq4_codebook_f32()
M32 = ocb.tq4_midpoints_f32(C32)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def f32np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def assert_within(y_gpu, y_ref, a_ref, rel=1e-3, what=""):
    """|y_gpu - y_ref| <= rel * A elementwise (A = sum |W_deq x|)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    bound = rel * a_ref
    bad = err > bound
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {i}: "
                             f"gpu={y_gpu.ravel()[i]!r} ref={y_ref.ravel()[i]!r} A={a_ref.ravel()[i]!r}")
    return float((err / np.maximum(a_ref, 1e-300)).max())


def edge_rows(K: int) -> np.ndarray:
    """Rows exercising zeros, saturation, subnormal scales, spikes and exact rotated zeros."""
    rows = []
    rows.append(np.zeros(K, np.float32))
    r = np.zeros(K, np.float32); r[:32] = 1e6; rows.append(r)                 # fp16 saturation
    r = np.zeros(K, np.float32); r[5] = 1e-6; rows.append(r)                  # subnormal fp16 scale
    r = np.zeros(K, np.float32); r[K - 1] = -3.25; rows.append(r)             # spike in the last block
    h = otq.hadamard()
    d = otq.sign_vector(otq.DEFAULT_SIGN_MASK)
    r = np.zeros(K, np.float32)
    r[:32] = (d * h[:, 3] * 0.25).astype(np.float32)                          # rotates to a single spike
    rows.append(r)
    r = np.full(K, -0.0, np.float32); rows.append(r)                          # negative zeros
    r = np.full(K, 2.0 ** -130, np.float32); rows.append(r)                   # fp32 subnormal inputs
    return np.stack(rows)


def tie_rows(K: int = 64, want: int = 6, seed: int = 0) -> np.ndarray:
    """Rows in which some rotated value equals a threshold fl(d * m_k) exactly.

    Built on the CPU with the oracle: a block whose first half carries a few
    fixed values plus one swept element; the swept value is stepped over
    consecutive floats near m_k * d * sqrt(32) until the oracle's rotated value
    lands exactly on the threshold.  Returns float32 rows [n, K].
    """
    rng = np.random.default_rng(seed)
    found = []
    tries = 0
    while len(found) < want and tries < 200:
        tries += 1
        k = int(rng.choice([0, 1, 2, 3, 4, 5, 6, 8, 9, 10, 11, 12, 13, 14]))
        j = int(rng.integers(0, 16))
        base = np.zeros(32, np.float64)
        base[:16] = rng.normal(size=16)
        # move the input along R^-1 e_j: only rotated element j changes (up to rounding)
        dirv = otq.inverse_rotate_f64(np.eye(32)[j], otq.DEFAULT_SIGN_MASK)
        for _ in range(6):                         # fixed point: the scale depends on the swept value
            _, _, wr, dd, _ = otq.quantize_o32(base[None, :].astype(np.float32), return_parts=True)
            target = float(np.float32(dd[0, 0, 0] * M32[k]))
            base = base + (target - float(wr[0, 0, j])) * dirv
        step = np.arange(-4096, 4096, dtype=np.float64) * 2e-8 * abs(target)
        cand = (base[None, :] + np.outer(step, dirv)).astype(np.float32)
        _, _, wr2, dd2, _ = otq.quantize_o32(cand, return_parts=True)
        thr = (dd2[:, 0, 0].astype(np.float32) * M32[k]).astype(np.float32)
        hit = np.flatnonzero(wr2[:, 0, j] == thr)
        if hit.size:
            found.append(cand[hit[0]])
    if len(found) < want:
        raise RuntimeError(f"constructed only {len(found)} exact threshold ties")
    rows = np.zeros((len(found), K), np.float32)
    for i, b in enumerate(found):
        rows[i, :32] = b
        rows[i, 32:64] = b[::-1]
    return rows
