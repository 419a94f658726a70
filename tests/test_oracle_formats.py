"""Pins of the oracle's codecs against published format tables and torch's casts."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_formats.txt")


def _golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            kind, code, val = line.split()
            rows.append((kind, int(code, 0), float(val)))
    return rows


def test_e2m1_e8m0_e4m3_tables():
    for kind, code, val in _golden():
        if kind == "e2m1":
            got = F.decode_e2m1(code)
        elif kind == "e8m0":
            got = F.decode_e8m0(code)
        else:
            got = F.decode_e4m3fn(code)
        assert got == val and np.signbit(got) == np.signbit(val), (kind, code)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = F.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(size=20000) * s for s in (1e-3, 0.1, 1, 10, 100)])
    x = x[np.abs(x) < 440].astype(np.float32)
    # midpoints between neighbouring codes are ties: torch rounds them to even
    pos = F.decode_e4m3fn(np.arange(0, 127))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.encode_e4m3fn(x.astype(np.float64))
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    assert F.encode_e4m3fn(np.array([1000.0, -1e9, 448.0, 464.0]))[:4].tolist() == \
        [0x7E, 0xFE, 0x7E, 0x7E]


def test_bf16_roundtrip_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.normal(size=50000) * np.exp(rng.normal(size=50000) * 5)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.encode_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(F.decode_bf16(ref), back.astype(np.float64))


def test_mxfp4_scale_rule():
    # amax in [2^e, 2^(e+1)) -> shared exponent e - 2 (E2M1's top exponent is 2)
    for e in range(-10, 10):
        for frac in (1.0, 1.3, 1.999):
            assert F.mxfp4_scale_exponent(frac * 2.0 ** e) == e - 2
    assert F.mxfp4_scale_exponent(0.0) == -127


def test_mxfp4_hand_example():
    blk = np.zeros(32)
    blk[:8] = [6, -3, 0.5, 1.25, 1.75, 5.0, -0.25, 2.5]   # amax 6 -> E = 0
    codes, scales = F.encode_mxfp4(blk)
    nib = F.unpack_nibbles(codes)
    # 1.25 and 1.75, 5.0, -0.25 and 2.5 are ties: even mantissa wins
    assert nib[:8].tolist() == [7, 8 | 5, 1, 2, 4, 6, 8 | 0, 4]
    assert scales.tolist() == [127]
    assert np.array_equal(F.decode_mxfp4(codes, scales)[:8], [6, -3, 0.5, 1, 2, 4, 0, 2])
    # element 2j is the low nibble of byte j
    assert codes[0] == (7 | ((8 | 5) << 4))


def test_mxfp4_roundtrip_and_clamp():
    rng = np.random.default_rng(3)
    nib = rng.integers(0, 16, size=(64, 128)).astype(np.uint8)
    nib[:, ::32] = 7                      # block max magnitude 6 -> exponent round-trips
    sc = rng.integers(100, 140, size=(64, 4)).astype(np.uint8)
    codes = F.pack_nibbles(nib)
    x = F.decode_mxfp4(codes, sc)
    c2, s2 = F.encode_mxfp4(x)
    assert np.array_equal(s2, sc)
    assert np.array_equal(F.decode_mxfp4(c2, s2), x)   # -0 and +0 may swap codes
    # beyond 6 * 2^E clamps to 6 * 2^E (only 7.99.. can appear after the scale rule)
    blk = np.full(32, 7.9)
    c3, s3 = F.encode_mxfp4(blk)
    assert s3[0] == 127 and np.all(F.decode_mxfp4(c3, s3) == 6.0)


def test_mxfp4_products_are_exact_quarters():
    """E2M1 x E2M1 products are multiples of 1/4 below 36, so a block's dot
    product is an exact small integer multiple of 1/4."""
    rng = np.random.default_rng(4)
    a = F.decode_e2m1(rng.integers(0, 16, size=(1000, 32)))
    b = F.decode_e2m1(rng.integers(0, 16, size=(1000, 32)))
    dots = (a * b).sum(axis=1)
    assert np.all(dots * 4 == np.round(dots * 4))
    assert np.max(np.abs(dots)) <= 32 * 36
