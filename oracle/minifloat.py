"""Small floating-point formats (E2M1, E3M2, E4M3fn, E8M0), float64 definitions.

Test infrastructure only (see the package docstring).

The pages name NVFP4 (llm-compressor page, "NVFP4 + FP8 双格式支持"; the
quantizer-tool page, "目前能实现的部分功能") and MXFP6 (quantizer-tool page,
"MXFP6 的未来") but define no bit layouts.  The element formats here follow
their public definitions (OCP Microscaling spec v1.0 for E2M1/E3M2/E8M0;
the OCP 8-bit float spec for E4M3 in its "fn" variant: no infinities,
S.1111.111 is NaN):

============  ====  ========  =====  ==============  ===============
format        bits  exp bias  man    max finite      smallest > 0
============  ====  ========  =====  ==============  ===============
E2M1          4     1         1      6.0             0.5 (subnormal)
E3M2          6     3         2      28.0            0.0625 (subn.)
E4M3fn        8     7         3      448.0           2^-9 (subnormal)
E8M0          8     127       0      2^127           2^-127 (no sign)
============  ====  ========  =====  ==============  ===============

Encoding is round-to-nearest, ties to the even code, with saturation to
the largest finite magnitude ("satfinite").  The encoder below is the plain
definition: enumerate the representable magnitudes from the bit layout, find
the nearest, and break an exact tie towards the code whose last bit is 0.
The sign bit is copied from the input (so -0.0 and small negatives that
round to zero encode as negative zero).
"""

import numpy as np


class Format:
    """A sign-magnitude binary float format with subnormals and no inf/NaN use."""

    def __init__(self, name: str, ebits: int, mbits: int, bias: int, nan_codes=()):
        self.name = name
        self.ebits = ebits
        self.mbits = mbits
        self.bias = bias
        self.bits = 1 + ebits + mbits
        self.sign_bit = 1 << (ebits + mbits)
        self.nan_codes = set(nan_codes)
        mags = []
        for code in range(self.sign_bit):
            if code in self.nan_codes:
                continue
            mags.append((code, self.decode_magnitude(code)))
        self._codes = np.array([c for c, _ in mags], dtype=np.int64)
        self._mags = np.array([m for _, m in mags], dtype=np.float64)
        order = np.argsort(self._mags, kind="stable")
        self._codes = self._codes[order]
        self._mags = self._mags[order]
        self.max = float(self._mags[-1])

    def decode_magnitude(self, code: int) -> float:
        """Value of a non-negative code from its exponent and mantissa fields."""
        e = (code >> self.mbits) & ((1 << self.ebits) - 1)
        m = code & ((1 << self.mbits) - 1)
        if e == 0:
            return (m / (1 << self.mbits)) * 2.0 ** (1 - self.bias)
        return (1.0 + m / (1 << self.mbits)) * 2.0 ** (e - self.bias)

    def decode(self, codes) -> np.ndarray:
        """Codes (integers) -> float64 values; NaN codes decode to NaN."""
        codes = np.asarray(codes, dtype=np.int64)
        mag_code = codes & (self.sign_bit - 1)
        table = np.array([self.decode_magnitude(c) for c in range(self.sign_bit)])
        for c in self.nan_codes:
            table[c] = np.nan
        v = table[mag_code]
        return np.where(codes & self.sign_bit, -v, v)

    def encode(self, x) -> np.ndarray:
        """float64-exact inputs -> codes, RNE with ties to even code, satfinite."""
        x = np.asarray(x, dtype=np.float64)
        neg = np.signbit(x)
        a = np.minimum(np.abs(x), self.max)
        hi = np.searchsorted(self._mags, a, side="left")          # first mag >= a
        hi = np.minimum(hi, len(self._mags) - 1)
        lo = np.maximum(hi - 1, 0)
        m_hi = self._mags[hi]
        m_lo = self._mags[lo]
        c_hi = self._codes[hi]
        c_lo = self._codes[lo]
        d_hi = m_hi - a
        d_lo = a - m_lo
        exact = m_hi == a
        pick_hi = exact | (d_hi < d_lo) | ((d_hi == d_lo) & ((c_hi & 1) == 0))
        code = np.where(pick_hi, c_hi, c_lo)
        return (code | np.where(neg, self.sign_bit, 0)).astype(np.uint8)


E2M1 = Format("e2m1", 2, 1, 1)
E3M2 = Format("e3m2", 3, 2, 3)
E4M3FN = Format("e4m3fn", 4, 3, 7, nan_codes=(0x7F,))


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale byte b -> 2^(b - 127) (b = 255 is NaN)."""
    b = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, (b - 127).astype(np.int64))
    return np.where(b == 255, np.nan, v)
