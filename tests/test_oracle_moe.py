"""Pins of the oracle's routing, permutation, grouped GEMMs, SwiGLU and combine
against brute force (Python sorting and loops), exact rational arithmetic
(fractions.Fraction), closed forms and special cases that reduce to a dense layer.

Method: *Low-Bit Precision Training*, section "What W4A4 GEMM Actually Changes"
(W4A4 expert GEMMs under dynamic expert routing); *miniTE news item*, section
"Development: Aligning Numerics, Then Making NVFP4 Fast" (grouped GEMMs);
*The 4-bitter Lesson*, section "Improving Gradient Stability" (y = x . DQ(Q(w))).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import moe
from oracle import nvfp4 as Q
from oracle import pipeline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- routing / permutation

def _brute_route(logits, k):
    T, E = logits.shape
    ids, ws = [], []
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        m = max(row)
        z = sum(math.exp(v - m) for v in row)
        ids.append(order)
        ws.append([math.exp(row[e] - m) / z for e in order])
    return np.array(ids), np.array(ws)


@pytest.mark.parametrize("T,E,k", [(37, 8, 2), (50, 5, 5), (64, 16, 1), (9, 3, 3)])
def test_route_matches_brute_force(T, E, k):
    lg = synth.rng(T * 100 + E).standard_normal((T, E)).astype(np.float32)
    lg[0, :] = 0.5                    # a full tie: lowest ids win
    lg[1, 1] = lg[1, 2] = lg[1].max() + 1
    ids, w = moe.route_topk(lg, k)
    bi, bw = _brute_route(lg, k)
    assert (ids == bi).all()
    assert np.allclose(w, bw, rtol=1e-13, atol=0)
    assert ids[0].tolist() == list(range(k))
    if k >= 2:
        assert ids[1, :2].tolist() == [1, 2]
    if k == E:
        assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def test_route_renorm():
    lg = synth.logits_softmax(20, 8, 1)
    _, w = moe.route_topk(lg, 3, renorm=True)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-14)


def _brute_permute(ids, E):
    T, k = ids.shape
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    rows.append((t, j))
    return rows


@pytest.mark.parametrize("T,E,k,seed", [(40, 6, 2, 0), (33, 4, 4, 1), (16, 9, 1, 2)])
def test_permute_matches_brute_force(T, E, k, seed):
    r = synth.rng(seed)
    ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[ids == E - 1] = 0 if k == 1 else ids[ids == E - 1]   # sometimes leave an expert empty
    p = moe.permute(ids, E)
    rows = _brute_permute(ids, E)
    assert p["row_token"].tolist() == [t for t, _ in rows]
    for r_, (t, j) in enumerate(rows):
        assert p["token_row"][t, j] == r_
    assert p["offsets"].tolist() == [0] + np.cumsum(np.bincount(ids.ravel(), minlength=E)).tolist()
    # bijection
    assert sorted(p["token_row"].ravel().tolist()) == list(range(T * k))
    pc = (np.diff(p["padded_offsets"]))
    assert ((pc % 16) == 0).all() and (pc >= np.diff(p["offsets"])).all() and (pc - np.diff(p["offsets"]) < 16).all()


def test_gather_and_quantize_commute_for_tensor_scale():
    """With every token routed at least once, the tensor amax of the gathered
    activations equals that of X, so quantise-then-gather == gather-then-quantise."""
    cfg = synth.CONFIGS["tiny"]
    X = synth.activations(cfg.T, cfg.H, cfg.seed)
    ids, _ = moe.route_topk(synth.router_logits(cfg), cfg.k)
    p = moe.permute(ids, cfg.E)
    a = pipeline.gather_rows(Q.quantize_rows(X), p["row_token"])
    b = Q.quantize_rows(X[p["row_token"]])
    assert (a.codes == b.codes).all() and (a.scales == b.scales).all() and (a.G == b.G).all()


# ---------------------------------------------------------------- GEMMs

def _rand_nvfp4(rows, K, seed, ngroups=1):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 16, (rows, K)).astype(np.uint8)
    sf = r.integers(0, 0x7F, (rows, K // 16)).astype(np.uint8)
    G = (r.uniform(0.5, 2.0, ngroups) * 2.0 ** r.integers(-8, 8, ngroups)).astype(np.float32)
    grp = np.arange(rows) * ngroups // rows
    return codes, sf, G, np.repeat(G[grp][:, None], K // 16, axis=1)


def _fp64_sum_bound(K, mass):
    """A-priori error bound of an FP64 dot product whose K products are exact:
    |computed - exact| <= K * 2^-53 * sum |a_k b_k| (to first order; the slack
    factor 1.01 covers the second-order term for K << 2^53)."""
    return Fraction(101, 100) * K * Fraction(1, 2 ** 53) * mass


def _frac_dequant(codes, sf, Gb):
    e2 = {c: Fraction(float(F.e2m1_decode(np.uint8(c)))) for c in range(16)}
    e4 = {c: Fraction(float(F.e4m3_decode(np.uint8(c)))) for c in range(0x7F)}
    rows, K = codes.shape
    return [[e2[int(codes[i, j])] * e4[int(sf[i, j // 16])] * Fraction(float(Gb[i, j // 16]))
             for j in range(K)] for i in range(rows)]


def test_grouped_gemm_m_exact_rational():
    E, N, K = 3, 5, 32
    off = [0, 4, 4, 11]
    ac, asf, aG, aGb = _rand_nvfp4(11, K, 1)
    bc, bsf, bG, bGb = _rand_nvfp4(E * N, K, 2, ngroups=E)
    C = moe.grouped_gemm_m(Q.dequantize(ac, asf, aGb), Q.dequantize(bc, bsf, bGb), off, E, N)
    A = _frac_dequant(ac, asf, aGb)
    B = _frac_dequant(bc, bsf, bGb)
    for e in range(E):
        for i in range(off[e], off[e + 1]):
            for n in range(N):
                exact = sum(A[i][kk] * B[e * N + n][kk] for kk in range(K))
                mass = sum(abs(A[i][kk] * B[e * N + n][kk]) for kk in range(K))
                assert abs(Fraction(C[i, n]) - exact) <= _fp64_sum_bound(K, mass)


def test_grouped_gemm_k_exact_rational_and_empty_expert():
    E, Nr, Mr = 3, 4, 3
    ko = [0, 16, 16, 48]
    ac, asf, _, aGb = _rand_nvfp4(Nr, 48, 3)
    bc, bsf, _, bGb = _rand_nvfp4(Mr, 48, 4)
    C = moe.grouped_gemm_k(Q.dequantize(ac, asf, aGb), Q.dequantize(bc, bsf, bGb), ko, E)
    A = _frac_dequant(ac, asf, aGb)
    B = _frac_dequant(bc, bsf, bGb)
    assert (C[1] == 0).all()
    for e in (0, 2):
        for i in range(Nr):
            for j in range(Mr):
                exact = sum(A[i][kk] * B[j][kk] for kk in range(ko[e], ko[e + 1]))
                mass = sum(abs(A[i][kk] * B[j][kk]) for kk in range(ko[e], ko[e + 1]))
                assert abs(Fraction(C[e, i, j]) - exact) <= _fp64_sum_bound(ko[e + 1] - ko[e], mass)


def test_grouped_gemm_single_expert_is_dense_and_identity_b():
    K = 64
    ac, asf, _, aGb = _rand_nvfp4(20, K, 5)
    Ah = Q.dequantize(ac, asf, aGb)
    # B = identity: code 2 (1.0) on the diagonal, 0 elsewhere, block scale 1.0 (0x38), G = 1
    bc = np.where(np.eye(K, dtype=bool), 2, 0).astype(np.uint8)
    bsf = np.full((K, K // 16), 0x38, np.uint8)
    Bh = Q.dequantize(bc, bsf, np.ones((K, K // 16), np.float32))
    C = moe.grouped_gemm_m(Ah, Bh, [0, 20], 1, K)
    assert (C == Ah).all()
    bc2, bsf2, _, bGb2 = _rand_nvfp4(7, K, 6)
    Bh2 = Q.dequantize(bc2, bsf2, bGb2)
    assert np.array_equal(moe.grouped_gemm_m(Ah, Bh2, [0, 20], 1, 7), Ah @ Bh2.T)


def test_all_unit_scales_give_quarter_integer_sums():
    """With every block scale 1.0 and G = 1, each element is a multiple of 0.5, so
    every dot product is an exact multiple of 0.25 (no rounding anywhere)."""
    r = np.random.default_rng(7)
    K = 256
    ac = r.integers(0, 16, (9, K)).astype(np.uint8)
    bc = r.integers(0, 16, (2 * 6, K)).astype(np.uint8)
    one = lambda n: np.full((n, K // 16), 0x38, np.uint8)
    Ah = Q.dequantize(ac, one(9), np.ones((9, K // 16), np.float32))
    Bh = Q.dequantize(bc, one(12), np.ones((12, K // 16), np.float32))
    C = moe.grouped_gemm_m(Ah, Bh, [0, 5, 9], 2, 6)
    assert (C * 4 == np.round(C * 4)).all()
    ints_a = F.e2m1_decode(ac) * 2
    ints_b = F.e2m1_decode(bc) * 2
    exact = [(ints_a[i].astype(np.int64) @ ints_b[(0 if i < 5 else 6) + n].astype(np.int64)) for i in range(9) for n in range(6)]
    assert (np.array(exact).reshape(9, 6) == C * 4).all()


# ---------------------------------------------------------------- SwiGLU and combine

def test_swiglu_identities():
    g = np.array([-30.0, -2.0, -0.5, 0.0, 0.5, 2.0, 30.0])
    # silu(g) - silu(-g) = g (since sigmoid(g) + sigmoid(-g) = 1)
    assert np.allclose(moe.silu(g) - moe.silu(-g), g, rtol=1e-15, atol=1e-15)
    # sigmoid(ln 3) = 3/4, so silu(ln 3) = 0.75 ln 3
    assert moe.silu(np.array([math.log(3.0)]))[0] == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    C = np.stack([g, np.arange(7.0)], axis=1)          # one gate column, one up column
    h = moe.swiglu(C)
    assert h[3, 0] == 0.0                               # silu(0) * u = 0
    assert h[0, 0] == pytest.approx(0.0, abs=1e-11)     # silu(-30) ~ -30 e^-30
    assert h[6, 0] == pytest.approx(30.0 * 6, rel=1e-12)


def test_combine_unpermute_linearity_and_loop():
    cfg = synth.CONFIGS["tiny"]
    lg = synth.router_logits(cfg)
    ids, w = moe.route_topk(lg, 1)
    p = moe.permute(ids, cfg.E)
    X = synth.activations(cfg.T, 16, 3)
    Y = X[p["row_token"]]
    assert (moe.combine(Y, p["token_row"], np.ones_like(w)) == X).all()       # k = 1, w = 1: un-permute
    ids, w = moe.route_topk(lg, 2)
    p = moe.permute(ids, cfg.E)
    Y = synth.activations(cfg.R, 16, 4).astype(np.float64)
    out = moe.combine(Y, p["token_row"], w)
    w2 = synth.rng(5).random(w.shape)
    assert np.allclose(moe.combine(Y, p["token_row"], 2 * w + 3 * w2),
                       2 * out + 3 * moe.combine(Y, p["token_row"], w2), rtol=1e-13, atol=1e-13)
    t = 7
    loop = sum(w[t, j] * Y[p["token_row"][t, j]] for j in range(2))
    assert np.allclose(out[t], loop, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- end to end

def test_single_expert_top1_layer_is_dense_w4a4_mlp():
    """E = 1, k = 1: the softmax weight is exactly 1 and the permutation is the
    identity, so the layer must equal a dense W4A4 SwiGLU MLP."""
    T, H, I = 48, 64, 32
    X = synth.activations(T, H, 40)
    W13 = synth.weights((1, 2 * I, H), 41)
    W13[0, I:] *= 30.0                     # up and gate with very different amax
    W2 = synth.weights((1, H, I), 42)
    lg = np.zeros((T, 1), np.float32)
    r = pipeline.moe_forward(X, lg, W13, W2, 1)
    assert (r["topk_w"] == 1.0).all() and (r["perm"]["row_token"] == np.arange(T)).all()
    xq = Q.quantize_rows(X).dequant()
    # gate and up are separate projections with a scale each (reading 9 of the quantiser)
    w13 = np.vstack([Q.quantize_rows(W13[0, :I]).dequant(), Q.quantize_rows(W13[0, I:]).dequant()])
    w2 = Q.quantize_rows(W2[0]).dequant()
    c = xq @ w13.T
    h = c[:, :I] / (1 + np.exp(-c[:, :I])) * c[:, I:]
    h16 = F.bf16_bits_to_f32(F.f32_to_bf16_bits(h.astype(np.float32)))
    y = Q.quantize_rows(h16).dequant() @ w2.T
    assert np.array_equal(r["out"], y.astype(np.float32))


def test_expert_parameter_accounting_footnote():
    """The three-projection expert (gate, up, down) reproduces the parameter counts of
    the footnote in *The 4-bitter Lesson* ("Why is the NVFP4 pretraining recipe not
    sufficient for RL?")."""
    with open(os.path.join(GOLDEN, "expert_params_footnote.json")) as f:
        g = json.load(f)
    per_expert = 3 * g["expert_matrix"][0] * g["expert_matrix"][1]
    assert round(per_expert / 1e6) == g["params_per_expert_millions"]
    per_layer = per_expert * (g["routed_experts"] + g["shared_experts"])
    assert round(per_layer / 1e9, 2) == g["params_per_layer_billions"]
    assert round(per_layer * g["moe_layers"] / 1e9) == g["total_expert_params_billions"]
