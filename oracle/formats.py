"""Number formats of the compressed caches, decoded and encoded in fp64.

Test infrastructure only: nothing in the product path imports this package.

Storage formats named by the pages (DeepSeek-V4 reviews):
  * main KV entry: the non-RoPE dims in FP8, the 64 RoPE dims in BF16
    (ricardokevins.github.io review, "CSA 与 HCA", closing stability box;
    yeyulingfeng.com digest, section 二).
  * indexer QK path in FP4, MXFP4 (ricardokevins.github.io review,
    "FP4 QAT、可恢复 rollout" section; digest section 二).

The pages do not define the bit layouts.  The readings used here:
  * FP8 is OCP E4M3FN (bias 7, no infinities, 0x7F/0xFF are NaN, max 448),
    encoded round-to-nearest-even and saturating at +-448, with no scale.
  * Every encoder keeps the sign of its input, so negative values that round
    to zero become -0 (IEEE convention).
  * BF16 is the upper half of an IEEE binary32, encoded round-to-nearest-even.
  * MXFP4 is OCP MX v1.0: blocks of 32 E2M1 elements sharing one E8M0 scale
    2**(floor(log2(amax)) - 2); elements round-to-nearest-even, clamped to
    +-6; element 2j sits in the low nibble of byte j.

Every encoder works by enumerating the representable values and picking the
nearest one (ties to the even code), so it can be checked by eye.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- E4M3FN


def decode_e4m3fn(codes) -> np.ndarray:
    """uint8 codes -> fp64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    sub = (man / 8.0) * 2.0 ** -6
    nor = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    mag = np.where(exp == 0, sub, nor)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


_E4M3_POS = decode_e4m3fn(np.arange(0, 127))  # codes 0..126: 0 .. 448, ascending


def _nearest_even(table: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of an ascending table; ties go to the even index.

    Assumes a >= table[0] and a <= table[-1].
    """
    hi = np.searchsorted(table, a, side="left")
    hi = np.clip(hi, 1, len(table) - 1)
    lo = hi - 1
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(a <= table[0], 0, idx)
    return idx


def encode_e4m3fn(x) -> np.ndarray:
    """fp64 -> uint8 E4M3FN codes, round-to-nearest-even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    idx = _nearest_even(_E4M3_POS, a)
    code = idx.astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


# ---------------------------------------------------------------- BF16


def decode_bf16(codes) -> np.ndarray:
    """uint16 codes -> fp64."""
    c = np.asarray(codes).astype(np.uint32)
    shape = c.shape
    c = np.ascontiguousarray(c.reshape(-1) << np.uint32(16))
    return c.view(np.float32).astype(np.float64).reshape(shape)


_BF16_POS = decode_bf16(np.arange(0, 0x7F80, dtype=np.uint32))  # +0 .. max finite


def encode_bf16(x) -> np.ndarray:
    """fp64 -> uint16 BF16 codes, round-to-nearest-even (finite inputs only)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > _BF16_POS[-1]):
        raise ValueError("bf16 overflow")
    idx = _nearest_even(_BF16_POS, a)
    code = idx.astype(np.uint32)
    return np.where(np.signbit(x), code | 0x8000, code).astype(np.uint16)


# ---------------------------------------------------------------- MXFP4

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def decode_e2m1(nibbles) -> np.ndarray:
    n = np.asarray(nibbles).astype(np.int64)
    mag = E2M1_VALUES[n & 7]
    return np.where((n >> 3) & 1, -mag, mag)


def decode_e8m0(codes) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    v = np.exp2(c.astype(np.float64) - 127.0)
    return np.where(c == 255, np.nan, v)


def unpack_nibbles(packed) -> np.ndarray:
    """[..., n/2] uint8 -> [..., n] nibbles; element 2j is the low nibble of byte j."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_nibbles(nib) -> np.ndarray:
    n = np.asarray(nib).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def decode_mxfp4(packed, scales) -> np.ndarray:
    """packed [..., D/2] uint8 + scales [..., D/32] uint8 -> fp64 [..., D]."""
    vals = decode_e2m1(unpack_nibbles(packed))
    sc = decode_e8m0(scales)
    D = vals.shape[-1]
    vals = vals.reshape(vals.shape[:-1] + (D // 32, 32)) * sc[..., None]
    return vals.reshape(vals.shape[:-2] + (D,))


def mxfp4_scale_exponent(amax) -> np.ndarray:
    """Shared exponent of a block: floor(log2(amax)) - 2, clamped to [-127, 127].

    2 is the exponent of the largest E2M1 magnitude (6 = 1.5 * 2**2).  A block of
    zeros takes the smallest scale.
    """
    amax = np.asarray(amax, dtype=np.float64)
    frac, e = np.frexp(np.where(amax > 0, amax, 1.0))  # amax = frac * 2**e, frac in [0.5, 1)
    fl = e.astype(np.int64) - 1                         # floor(log2(amax))
    E = np.where(amax > 0, fl - 2, -127)
    return np.clip(E, -127, 127)


def encode_mxfp4(x):
    """fp64 [..., D] (D % 32 == 0) -> (packed [..., D/2] uint8, scales [..., D/32] uint8)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 32:
        raise ValueError("MXFP4 needs a multiple of 32 elements")
    blocks = x.reshape(x.shape[:-1] + (D // 32, 32))
    E = mxfp4_scale_exponent(np.abs(blocks).max(axis=-1))
    scaled = blocks / np.exp2(E.astype(np.float64))[..., None]
    a = np.minimum(np.abs(scaled), 6.0)
    code = _nearest_even(E2M1_VALUES, a).astype(np.uint8)
    code = np.where(np.signbit(scaled), code | 8, code).astype(np.uint8)
    code = code.reshape(x.shape)
    return pack_nibbles(code), (E + 127).astype(np.uint8)
