"""Pins of the oracle's number formats (BF16, FP8 E4M3, FP4 E2M1).

Formats: *The 4-bitter Lesson*, section "Baseline: A starting recipe with stable
training dynamics" (16-value blocks, FP8 E4M3 block scale, FP32 tensor scale);
FP4 E2M1 and E4M3 as defined by the OCP MX v1.0 and OCP OFP8 specifications.
"""

import math

import numpy as np
import pytest
import torch

from oracle import formats as F


# ---------------------------------------------------------------- E2M1

def _e2m1_from_fields(code: int) -> float:
    """E2M1 value from its bit fields (bias 1): s.ee.m"""
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_decode_all_codes():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = F.e2m1_decode(np.arange(16, dtype=np.uint8))
    for c in range(16):
        assert got[c] == _e2m1_from_fields(c)
        assert abs(got[c]) == grid[c & 7]
        assert math.copysign(1.0, got[c]) == (-1.0 if c & 8 else 1.0)


def test_e2m1_encode_grid_identity_and_ties():
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)
    assert (F.e2m1_encode(grid) == np.arange(8)).all()
    assert (F.e2m1_encode(-grid[1:]) == np.arange(1, 8) | 8).all()
    # midpoints go to the even code (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2, 3.5 -> 4, 5 -> 4)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert F.e2m1_encode(mids).tolist() == [0, 2, 2, 4, 4, 6, 6]
    # just above / below each midpoint
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    assert F.e2m1_encode(up).tolist() == [1, 2, 3, 4, 5, 6, 7]
    assert F.e2m1_encode(dn).tolist() == [0, 1, 2, 3, 4, 5, 6]
    # saturation and signed zero
    assert F.e2m1_encode(np.array([6.5, 1e30, -1e30, -0.0, -0.1], np.float32)).tolist() == [7, 7, 15, 8, 8]


def test_e2m1_encode_is_nearest_on_dense_sweep():
    """Property: the decoded code is a nearest grid magnitude; on a tie it is the even code."""
    v = np.concatenate([np.linspace(-8, 8, 400_001, dtype=np.float32),
                        np.random.default_rng(1).standard_normal(100_000).astype(np.float32) * 3])
    c = F.e2m1_encode(v)
    dec = np.abs(F.e2m1_decode(c))
    a = np.abs(v.astype(np.float64))
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    d_all = np.abs(a[:, None] - grid[None, :])
    d_min = d_all.min(axis=1)
    assert (np.abs(a - dec) == d_min).all()
    ties = (d_all == d_min[:, None]).sum(axis=1) > 1
    assert ((c[ties] & 1) == 0).all()
    assert ((c >> 3) == np.signbit(v)).all()


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_all_codes():
    v = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(v).sum() == 2 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    fin = v[np.isfinite(v)]
    assert len(fin) == 254 and fin.max() == 448.0 and fin.min() == -448.0
    assert v[0x7E] == 448.0
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    assert v[0x08] == 2.0 ** -6          # smallest normal
    assert v[0x38] == 1.0                # exponent field 7 = bias
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()      # codes 0..0x7E strictly increasing
    assert (v[0x80:0xFF] == -pos[:0x7F]).all()


def test_e4m3_encode_matches_torch_cast():
    """torch.float8_e4m3fn is an open-source RNE cast to OCP E4M3FN (NaN above 464);
    on [0, 464] it and the oracle must agree bit for bit."""
    tab = F.e4m3_finite_nonneg().astype(np.float32)
    mids = ((tab[1:].astype(np.float64) + tab[:-1]) / 2).astype(np.float32)
    pts = np.concatenate([tab, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                          np.linspace(0, 464, 2_000_001, dtype=np.float32),
                          (2.0 ** np.random.default_rng(2).uniform(-12, 9, 500_000)).astype(np.float32),
                          np.array([464.0, 2.0 ** -10, 2.0 ** -30, 1e-45], np.float32)])
    pts = pts[(pts >= 0) & (pts <= 464)]
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(pts)
    assert (got == ref).all()


def test_e4m3_encode_saturates():
    big = np.array([448.0, 460.0, 464.0, 480.0, 1e6, 3.4e38], np.float32)
    assert (F.e4m3_encode(big) == 0x7E).all()


# ---------------------------------------------------------------- BF16 and FP32 helpers

def test_bf16_rne_matches_torch_cast():
    r = np.random.default_rng(3)
    x = (r.standard_normal(500_000) * 10.0 ** r.integers(-40, 38, 500_000)).astype(np.float32)
    bits = r.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, bits[np.isfinite(bits)], np.array([3.4028235e38, -0.0, 1e-45, np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    with np.errstate(invalid="ignore"):
        got = F.f32_to_bf16_bits(x)
    assert (got == ref).all()
    back = F.bf16_bits_to_f32(got[:1000])
    assert (F.f32_to_bf16_bits(back) == got[:1000]).all()


def test_f32_ops_are_ieee_single():
    """The FP64-then-round helpers equal numpy's native binary32 arithmetic."""
    r = np.random.default_rng(4)
    a = (r.standard_normal(300_000) * 2.0 ** r.integers(-60, 60, 300_000)).astype(np.float32)
    b = (r.standard_normal(300_000) * 2.0 ** r.integers(-60, 60, 300_000)).astype(np.float32)
    b[b == 0] = 1
    with np.errstate(all="ignore"):
        assert (F.f32_div(a, b).view(np.uint32) == (a / b).view(np.uint32)).all()
        assert (F.f32_mul(a, b).view(np.uint32) == (a * b).view(np.uint32)).all()


@pytest.mark.parametrize("bad", [np.nan])
def test_e2m1_rejects_nan(bad):
    with pytest.raises(ValueError):
        F.e2m1_encode(np.array([bad], np.float32))
