"""OCP FP8 E4M3 ("fn" variant) decode and round-to-nearest-even encode, in numpy.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark; never by the library or its binding.

The pages store the latent cache as ``torch.float8_e4m3fn`` bytes with a
per-tensor ``k_scale`` or per-token x 128-channel-group scales
(flashinfer_mla_sparse_sm90.py, module docstring and ``forward_mqa``). The
"fn" variant is the OCP 8-bit E4M3 format: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits, no infinities, the two codes S.1111.111 are NaN, and
the largest finite magnitude is 1.75 * 2**8 = 448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_code(b: int) -> float:
    """Value of one E4M3FN byte, straight from the field definition."""
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                       # subnormal: m * 2**-3 * 2**(1-7)
        mag = m * 2.0 ** -9
    else:                            # normal: (1 + m/8) * 2**(e-7)
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


DECODE_TABLE = np.array([decode_code(b) for b in range(256)], dtype=np.float64)

# the 127 non-negative finite values, codes 0x00..0x7E, in increasing order
_POS_VALUES = DECODE_TABLE[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0)


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_rne(y: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3FN codes, round to nearest with ties to the even
    code, magnitudes at or beyond 448 saturated to 448, NaN -> 0x7F (sign kept).

    Nearest is decided by exact comparison in float64 of |y| against the two
    neighbouring representable values (all differences are exact there)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    sign = np.signbit(y).astype(np.uint8) << 7
    out = np.zeros(y.shape, dtype=np.uint8)

    nan = np.isnan(a)
    sat = (~nan) & (a >= E4M3_MAX)
    mid = (~nan) & (~sat)

    am = a[mid]
    hi = np.searchsorted(_POS_VALUES, am, side="left")      # _POS[hi-1] < am <= _POS[hi]
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = am - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - am
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(am == _POS_VALUES[hi], hi, code)          # exact hit
    out[mid] = code.astype(np.uint8)
    out[sat] = 0x7E
    out[nan] = 0x7F
    return out | sign
