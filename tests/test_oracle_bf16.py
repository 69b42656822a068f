"""Pins of the oracle's BF16 pieces: the BF16 dequantisation of NVFP4 tensors
(the operands of the dequantized backward), the column layout of the BF16
weight-gradient operands, the unquantised BF16 layer and the BF16 backward.

*The 4-bitter Lesson*, section "Improving Gradient Stability": the dequantized
backward runs the backward GEMMs on BF16 operands that hold DQ(Q(.)) of the very
tensors the forward used, for weights and activations; the conservative
baseline (section "Why is the NVFP4 pretraining recipe not sufficient for
RL?") keeps the backward in BF16 on the unquantised tensors.

The pins do not reuse the oracle's arithmetic: exact rational arithmetic with a
rounding routine written here, the exact FP64 dequantisation where the BF16
value must be exact, brute-force per-token loops for the layer, and the adjoint
identity <dY, f(D)> = <grad, D> that defines the gradients of a bilinear map.
"""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import moe
from oracle import nvfp4 as Q
from oracle import pipeline as P


def _round_sig(x: Fraction, bits: int) -> Fraction:
    """x rounded to `bits` significant bits, ties to even (normal range only)."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    scaled = a * (1 << (bits - 1))          # in [2^(bits-1), 2^bits)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * Fraction(n, 1 << (bits - 1)) * (Fraction(2) ** e)


def test_dequantize_bf16_worked_examples():
    """G = fp32(1/3) = 11184811 * 2^-25.
    code 6.0 (0b0111) with scale 448 (0x7E): 2688 * G = 896.0000267...; FP32 keeps
    896 (the excess is 0.44 of an FP32 ulp there) and BF16 holds 896 exactly.
    code 0.5 (0b0001) with scale 1.0 (0x38): 0.5 * G is exact in FP32,
    0.16666667163...; its mantissa 1.0101010|1010... rounds up to 1.0101011, so
    the BF16 value is 1.3359375 * 2^-3 = 0.1669921875.  code -1.5 (0b1011) with
    the smallest subnormal scale 2^-9 (0x01) and G = 1: -1.5 * 2^-9 exactly."""
    G = np.float32(1) / np.float32(3)
    assert float(G) == 11184811 * 2.0 ** -25
    codes = np.zeros((1, 32), np.uint8)
    codes[0, 0], codes[0, 16], codes[0, 17] = 7, 1, 11
    t = Q.NVFP4(codes, np.array([[0x7E, 0x38]], np.uint8), np.array([G]),
                np.full((1, 2), G, np.float32), np.array([1.0], np.float32))
    v = Q.dequantize_bf16(t)
    assert v[0, 0] == 896.0
    assert v[0, 16] == 0.1669921875
    # -1.5 * G = -(0.5 + 2^-26): a quarter of an FP32 ulp above 0.5, so FP32 (and BF16) hold -0.5
    assert v[0, 17] == -0.5
    assert not v[0, 1:16].any() and not v[0, 18:].any()
    t3 = Q.NVFP4(np.array([[11] + [0] * 15], np.uint8), np.array([[0x01]], np.uint8), np.array([1.0], np.float32),
                 np.full((1, 1), np.float32(1.0), np.float32), np.array([1.0], np.float32))
    assert Q.dequantize_bf16(t3)[0, 0] == -1.5 * 2.0 ** -9


@pytest.mark.parametrize("seed", [0, 1])
def test_dequantize_bf16_exact_rational(seed):
    """Every element equals the exact rational e2m1 * sf * G rounded once to 24
    significant bits (FP32) and then to 8 (BF16), with the rounding written here."""
    r = synth.rng(100 + seed)
    x = (r.standard_normal((6, 64)) * np.exp(r.uniform(-4, 4, (6, 1)))).astype(np.float32)
    q = Q.quantize_rows(x, "row")
    got = Q.dequantize_bf16(q)
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
            Fraction(6)]
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            c = int(q.codes[i, j])
            e2m1 = (-1 if c & 8 else 1) * mags[c & 7]
            sf = Fraction(float(F.e4m3_decode(np.array([q.scales[i, j // 16]]))[0]))
            exact = e2m1 * sf * Fraction(float(q.G_block[i, j // 16]))
            want = _round_sig(_round_sig(exact, 24), 8)
            assert Fraction(float(got[i, j])) == want, (i, j)


def test_dequantize_bf16_power_of_two_scale_is_exact():
    """With a power-of-two G the BF16 value is the exact dequantised value
    (e2m1 * sf has at most 6 significant bits)."""
    r = synth.rng(7)
    x = r.standard_normal((8, 128)).astype(np.float32)
    q = Q.quantize_rows(x)
    for G in (np.float32(1.0), np.float32(2.0 ** -7), np.float32(2.0 ** 5)):
        t = Q.NVFP4(q.codes, q.scales, np.array([G]), np.full_like(q.G_block, G), q.amax)
        exact = Q.dequantize(q.codes, q.scales, t.G_block)
        assert np.array_equal(Q.dequantize_bf16(t).astype(np.float64), exact)


def test_transpose_segments_feeds_per_expert_outer_products():
    """grouped_gemm_k over the column layouts equals, for every expert, the sum of
    the outer products of that expert's rows (explicit loops); padding adds
    nothing and an empty segment gives zeros."""
    r = synth.rng(3)
    off = np.array([0, 5, 5, 22, 40])
    A = r.standard_normal((40, 6))
    B = r.standard_normal((40, 3))
    At, po = moe.transpose_segments(A, off)
    Bt, po2 = moe.transpose_segments(B, off)
    assert np.array_equal(po, po2) and po.tolist() == [0, 16, 16, 48, 80]
    C = moe.grouped_gemm_k(At, Bt, po, 4)
    for e in range(4):
        ref = np.zeros((6, 3))
        for row in range(off[e], off[e + 1]):
            for a in range(6):
                for b in range(3):
                    ref[a, b] += A[row, a] * B[row, b]
        assert np.allclose(C[e], ref, rtol=1e-13, atol=1e-13)
    assert not C[1].any()


def test_transpose_batched_is_per_matrix_transpose():
    x = np.arange(2 * 4 * 3).reshape(8, 3)
    t = moe.transpose_batched(x, 2)
    for e in range(2):
        for i in range(4):
            for c in range(3):
                assert t[e * 3 + c, i] == x[e * 4 + i, c]


def test_bf16_layer_matches_per_token_loop():
    """The grouped, permuted BF16 layer equals a plain loop over tokens and their
    chosen experts: h = silu(x W_gate^T) * (x W_up^T) stored as BF16, y = h W2^T,
    out = sum_j w_j y_j."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg)
    T, H, E, I, k = cfg.T, cfg.H, cfg.E, cfg.I, cfg.k
    X, W13, W2 = d["X"][:40], d["W13"], d["W2"]
    f = P.moe_forward_bf16(X, d["logits"][:40], W13, W2, k)
    ids, w = moe.route_topk(d["logits"][:40], k)
    out = np.zeros((40, H))
    for t in range(40):
        for j in range(k):
            e = ids[t, j]
            g = W13[e, :I].astype(np.float64) @ X[t]
            u = W13[e, I:].astype(np.float64) @ X[t]
            h = P.bf16(g / (1 + np.exp(-g)) * u).astype(np.float64)
            y = F.f32(W2[e].astype(np.float64) @ h).astype(np.float64)
            out[t] += w[t, j] * y
    assert np.allclose(f["out"], out, rtol=1e-6, atol=1e-6 * np.abs(out).max())


@pytest.mark.parametrize("dequantized", [False, True])
def test_bf16_backward_is_adjoint_of_forward(dequantized):
    """Each gradient satisfies <dY, f(D)> = <grad, D> for the linear map f through
    which its operand enters the forward GEMM (random directions D)."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.k
    fwd = P.moe_forward(d["X"], d["logits"], d["W13"], d["W2"], k)
    perm = fwd["perm"]
    ops = P.backward_operands_bf16(d["X"], fwd["Hact_bf16"], d["W13"], d["W2"], fwd if dequantized else None)
    g = P.moe_backward_bf16(ops, d["dY2"], d["dY13"], perm)
    off = perm["offsets"]
    Xperm = ops["X"][perm["row_token"]]
    r = synth.rng(11)
    inner = lambda a, b: float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))
    dY2, dY13 = d["dY2"].astype(np.float64), d["dY13"].astype(np.float64)

    D = r.standard_normal(ops["Hact"].shape)
    lhs = inner(dY2, moe.grouped_gemm_m(D, ops["W2"], off, E, H))
    assert abs(lhs - inner(g["dHact"], D)) <= 1e-10 * abs(lhs)
    D = r.standard_normal(ops["W2"].shape)
    lhs = inner(dY2, moe.grouped_gemm_m(ops["Hact"], D, off, E, H))
    assert abs(lhs - inner(g["dW2"].reshape(E * H, I), D)) <= 1e-10 * abs(lhs)
    D = r.standard_normal(Xperm.shape)
    lhs = inner(dY13, moe.grouped_gemm_m(D, ops["W13"], off, E, 2 * I))
    assert abs(lhs - inner(g["dXperm"], D)) <= 1e-10 * abs(lhs)
    D = r.standard_normal(ops["W13"].shape)
    lhs = inner(dY13, moe.grouped_gemm_m(Xperm, D, off, E, 2 * I))
    assert abs(lhs - inner(g["dW13"].reshape(E * 2 * I, H), D)) <= 1e-10 * abs(lhs)
    if dequantized:
        # the operands are the forward's own NVFP4 values, not the BF16 tensors
        assert not np.array_equal(ops["W2"], d["W2"].reshape(E * H, I))
        assert np.array_equal(ops["Hact"], Q.dequantize_bf16(fwd["Hq"]))
