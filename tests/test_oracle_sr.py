"""Pins of the oracle's stochastic rounding: the Philox4x64-10 generator against
numpy's own Philox bit generator (an independent implementation of the same
published bijection), the E2M1 stochastic rounding rule against exact rational
arithmetic and exhaustive counts over all 2^24 uniforms, and the quantiser with
stochastic rounding against its round-to-nearest counterpart (same block scales,
codes one grid step apart at most, unbiased on average).

*The 4-bitter Lesson*, section "Why is the NVFP4 pretraining recipe not
sufficient for RL?": the pretraining recipe rounds gradients stochastically so
that their quantisation is unbiased on average.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import philox as P

GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_philox_matches_numpy_bit_generator(seed):
    """numpy's Philox (4x64, 10 rounds) advances its 256-bit counter before each
    block of four outputs: with counter c its first outputs are philox(c + 1)."""
    r = np.random.default_rng(seed)
    key = [int(k) for k in r.integers(0, 2 ** 63, 2, dtype=np.int64)]
    for _ in range(4):
        c = [int(v) for v in r.integers(0, 2 ** 62, 4, dtype=np.int64)]
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(c, dtype=np.uint64))
        raw = [int(v) for v in bg.random_raw(8)]
        assert raw[:4] == list(P.philox4x64_scalar((c[0] + 1, c[1], c[2], c[3]), key))
        assert raw[4:] == list(P.philox4x64_scalar((c[0] + 2, c[1], c[2], c[3]), key))
        vec = P.philox4x64(c[0] + 1, c[1], c[2], c[3], key[0], key[1])
        assert [int(w) for w in vec] == raw[:4]


def test_uniform24_layout():
    """Element (row, pos) reads half (pos & 1) of word (pos >> 1) & 3 of the block
    for counter (pos >> 3, row, stream, 0), key (seed, 0)."""
    seed = 0x5EED
    rows = np.array([0, 3, 3, 7])
    pos = np.array([0, 5, 13, 8])
    u = P.uniform24(rows, pos, 1, seed)
    for i in range(4):
        w = P.philox4x64_scalar((int(pos[i]) >> 3, int(rows[i]), 1, 0), (seed, 0))[(int(pos[i]) >> 1) & 3]
        half = (w >> 32) if pos[i] & 1 else (w & 0xFFFFFFFF)
        assert u[i] == half >> 8


def test_sr_on_grid_values_are_exact():
    vals = np.array([0.0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -6, 7.5, -100.0], np.float32)
    want = np.array([0, 1, 2, 3, 4, 5, 6, 7, 9, 15, 7, 15], np.uint8)
    for u in (0, 1, 1 << 23, (1 << 24) - 1):
        assert np.array_equal(F.e2m1_encode_sr(vals, np.full(len(vals), u, np.uint32)), want)
    # -0.0 keeps its sign, as in round-to-nearest
    assert F.e2m1_encode_sr(np.array([-0.0], np.float32), np.array([5], np.uint32))[0] == 8


def test_sr_decision_exact_rational():
    r = synth.rng(21)
    v = (r.uniform(-7, 7, 4000)).astype(np.float32)
    v[:50] = r.uniform(-1e-6, 1e-6, 50).astype(np.float32)   # tiny values between 0 and 0.5
    u = r.integers(0, 1 << 24, 4000).astype(np.uint32)
    got = F.e2m1_encode_sr(v, u)
    for i in range(len(v)):
        a = min(abs(Fraction(float(v[i]))), Fraction(6))
        j = max(k for k in range(8) if GRID[k] <= a)
        up = j < 7 and Fraction(int(u[i]), 1 << 24) < (a - GRID[j]) / (GRID[j + 1] - GRID[j])
        want = (8 if np.signbit(v[i]) else 0) | (j + int(up))
        assert got[i] == want, (v[i], u[i])


@pytest.mark.parametrize("v", [0.3, 1.2, 2.75, 5.125, 0.25, 1e-7])
def test_sr_up_probability_over_all_uniforms(v):
    """Over all 2^24 uniforms, the number that round up is ceil(frac * 2^24), where
    frac is the exact position of |v| between its grid neighbours."""
    u = np.arange(1 << 24, dtype=np.uint32)
    codes = F.e2m1_encode_sr(np.full(1 << 24, v, np.float32), u)
    a = Fraction(float(np.float32(v)))
    j = max(k for k in range(8) if GRID[k] <= a)
    frac = (a - GRID[j]) / (GRID[j + 1] - GRID[j])
    n_up = int(np.count_nonzero(codes == j + 1))
    want = -((-frac * (1 << 24)).numerator // (-frac * (1 << 24)).denominator) if frac else 0
    assert n_up == want and np.count_nonzero(codes == j) == (1 << 24) - n_up


def test_sr_vs_nearest_away_from_ties():
    """With the uniform at exactly 1/2 stochastic rounding rounds up iff the
    position between the neighbours exceeds 1/2: the nearest-value rounding
    except at ties."""
    r = synth.rng(5)
    v = r.uniform(-6.5, 6.5, 20000).astype(np.float32)
    sr = F.e2m1_encode_sr(v, np.full(len(v), 1 << 23, np.uint32))
    rne = F.e2m1_encode(v)
    a = np.abs(v).astype(np.float64)
    tie = np.isin(a, [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert np.array_equal(sr[~tie], rne[~tie])


def test_quantize_sr_keeps_scales_and_moves_codes_one_step():
    x = synth.activations(64, 256, 9)
    q = Q.quantize_rows(x)
    s = Q.quantize_rows(x, sr_seed=123)
    assert np.array_equal(q.scales, s.scales) and np.array_equal(q.G, s.G)
    mag_q, mag_s = q.codes & 7, s.codes & 7
    assert np.abs(mag_q.astype(int) - mag_s.astype(int)).max() <= 1
    assert not np.array_equal(q.codes, s.codes)
    assert np.array_equal(Q.quantize_rows(x, sr_seed=123).codes, s.codes)       # deterministic per seed
    assert not np.array_equal(Q.quantize_rows(x, sr_seed=124).codes, s.codes)
    # the column form draws from its own stream: its codes are not the rows' codes transposed
    c, _ = Q.quantize_cols(x.T.copy(), np.array([0, 256]), sr_seed=123)
    r = Q.quantize_rows(x, sr_seed=123)
    assert np.array_equal(c.scales, Q.quantize_cols(x.T.copy(), np.array([0, 256]))[0].scales)
    assert not np.array_equal(c.codes, r.codes)


def test_quantize_sr_is_unbiased_on_average():
    """The mean of the dequantised values over 200 seeds approaches the
    pre-rounding value v * sf * G (E2M1 saturation aside), well inside the
    standard error of the mean, while round-to-nearest has a fixed bias."""
    x = synth.activations(8, 64, 4, outlier_frac=0.0)
    q = Q.quantize_rows(x)
    sfv = F.e4m3_decode(q.scales).astype(np.float64) * q.G_block
    S = Q.tensor_scales(q.amax)[0][0]
    sf = F.e4m3_decode(q.scales).astype(np.float32)
    inv = np.where(q.scales > 0, F.f32_div(np.float32(S), np.where(q.scales > 0, sf, 1)), 0).astype(np.float32)
    v = F.f32_mul(x.reshape(8, 4, 16), inv[:, :, None])        # the quantiser's own fp32(x * fp32(S / sf))
    target = (np.minimum(np.abs(v), 6.0) * np.sign(v) * sfv[:, :, None]).reshape(8, 64)
    acc = np.zeros_like(target)
    n = 200
    for seed in range(n):
        acc += Q.quantize_rows(x, sr_seed=seed).dequant()
    mean = acc / n
    gap = sfv.repeat(16, axis=1) * 2.0      # largest grid gap times the block scale bounds the spread
    assert np.all(np.abs(mean - target) <= 5 * gap / np.sqrt(n) + 1e-12)
    bias_sr = np.abs(mean - target).mean()
    bias_rne = np.abs(q.dequant() - target).mean()
    assert bias_sr < 0.25 * bias_rne
