"""Pins of the oracle's NVFP4 quantiser against facts that do not depend on it:
hand-derived worked examples, the block-scale corner case over every BF16
magnitude, the rounding-error bound, round-trip identity on representable
tensors, and the power-of-two and sign symmetries of the format.

Format and recipe: *The 4-bitter Lesson*, sections "Baseline: A starting recipe
with stable training dynamics" (16-value blocks, E4M3 block scales, one FP32
tensor scale), "Why is the NVFP4 pretraining recipe not sufficient for RL?"
(per-tensor global scale for weights; per-token FP32 scale for activations) and
"Improving Gradient Stability" (footnote 6: clip(round(w/s), qmin, qmax)).
"""

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import nvfp4 as Q


def test_worked_example_unit_scales():
    """A = 2688 makes S = G = 1.  Block 0 holds the E2M1 midpoints (and 6), so its
    block scale is 6/6 * 1 = 1.0 (E4M3 0x38) and its codes are the ties-to-even
    roundings; block 1 holds A itself (scale 448 = 0x7E, 2688 -> 6, 1344 -> 3,
    448 -> 1)."""
    b0 = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, -6]
    b1 = [2688, 1344, 448, -2688, 0, -0.0, 224, 896] + [0] * 8
    q = Q.quantize_rows(np.array([b0 + b1], np.float32))
    assert q.G.tolist() == [1.0]
    assert q.scales.tolist() == [[0x38, 0x7E]]
    assert q.codes[0, :16].tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 8, 10, 10, 12, 12, 14, 14, 15]
    # 224/448 = 0.5 -> code 1, 896/448 = 2 -> code 4, -0.0 keeps its sign
    assert q.codes[0, 16:24].tolist() == [7, 5, 2, 15, 0, 8, 1, 4]
    assert q.packed()[0, :2].tolist() == [0x20, 0x42]


def test_worked_example_nontrivial_tensor_scale():
    """A = 1: S = 2688, G = fp32(1/2688).  The block holding 1 gets
    t = fp32(fp32(1/6) * 2688) = 448.00002 -> saturates to 448, inv = 2688/448 = 6,
    so 1 -> 6 (code 7) and 0.5 -> 3 (code 5).  A block with max 0.25 gets
    t = fp32(fp32(0.25/6) * 2688) = 112.000004 -> 112 (0x6E), inv = 24, 0.25 -> 6."""
    row = np.zeros((1, 32), np.float32)
    row[0, 0], row[0, 1] = 1.0, 0.5
    row[0, 16], row[0, 17] = 0.25, -0.0625
    q = Q.quantize_rows(row)
    assert q.G[0] == np.float32(1.0) / np.float32(2688.0)
    assert q.scales.tolist() == [[0x7E, 0x6E]]
    assert q.codes[0, :2].tolist() == [7, 5]
    # -0.0625 * 24 = -1.5 -> code 8|3
    assert q.codes[0, 16:18].tolist() == [7, 11]


def _all_positive_finite_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    return F.bf16_bits_to_f32(bits)


def test_tensor_amax_block_maps_to_448_and_6():
    """Every positive finite BF16 magnitude A, as the amax of its own scale group:
    if 2688/A is finite, its block scale is 448 and its code is 6; otherwise S = 1
    and the (tiny) element quantises to zero."""
    A = _all_positive_finite_bf16()
    x = np.zeros((len(A), 16), np.float32)
    x[:, 0] = A
    q = Q.quantize_rows(x, "row")
    finite = np.isfinite(np.float64(2688.0) / A.astype(np.float64)) & \
        (np.float64(2688.0) / A.astype(np.float64) < np.finfo(np.float32).max)
    assert finite.sum() > 31_000
    assert (q.scales[finite, 0] == 0x7E).all()
    assert (q.codes[finite, 0] == 7).all()
    assert (q.scales[~finite, 0] == 0).all() and (q.codes[~finite, 0] == 0).all()


def _error_bound_holds(x: np.ndarray, q: Q.NVFP4):
    """|x - x_hat| <= (half the E2M1 gap at |v| + max(0, |v| - 6) + 2^-19) * sf * G,
    where v = x / (sf * G) is the scaled element.  The 2^-19 term covers the three
    FP32 roundings (G, inv, v), each at most 2^-24 relative on |v| <= 6.4 and |q| <= 6."""
    rows, K = x.shape
    sfG = (F.e4m3_decode(q.scales).astype(np.float64) * q.G_block).repeat(16, axis=1)
    xh = q.dequant()
    err = np.abs(x.astype(np.float64) - xh)
    nz = sfG > 0
    v = np.zeros_like(err)
    v[nz] = np.abs(x.astype(np.float64)[nz]) / sfG[nz]
    a = np.minimum(v, 6.0)
    half_gap = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = (half_gap + np.maximum(0.0, v - 6.0) + 2.0 ** -19) * sfG
    ok_nz = (err[nz] <= bound[nz]).all()
    # zero-scale blocks dequantise to 0; their elements are below 6 * 2^-10 * G (t_b rounds to 0)
    Gb = q.G_block.astype(np.float64).repeat(16, axis=1)
    ok_z = (np.abs(x.astype(np.float64)[~nz]) <= 6 * 2.0 ** -10 * Gb[~nz] * (1 + 2.0 ** -20)).all()
    return ok_nz, ok_z, float(v.max())


@pytest.mark.parametrize("mode", ["tensor", "row"])
def test_error_bound_on_seeded_activations(mode):
    x = synth.activations(512, 2048, seed=11)
    q = Q.quantize_rows(x, mode)
    ok_nz, ok_z, vmax = _error_bound_holds(x, q)
    assert ok_nz and ok_z
    assert vmax <= 6.375 + 1e-6       # normal block scales keep |v| within 6 * (1 + 2^-4)


def test_error_bound_on_weights_and_wide_range():
    w = synth.weights((64, 1024), seed=12)
    q = Q.quantize_rows(w, "segment", nseg=4)
    assert all(_error_bound_holds(w, q)[:2])
    r = np.random.default_rng(13)
    x = (r.standard_normal((64, 256)) * 2.0 ** r.integers(-30, 30, (64, 1))).astype(np.float32)
    q = Q.quantize_rows(x, "row")
    assert all(_error_bound_holds(x, q)[:2])


def _representable_tensor(rows, K, j, seed):
    """codes x E4M3 scale x 2^j, every block containing a +-6 code and the tensor
    containing a block with scale 448, so that the quantiser's own A, S, G come
    out as exact powers of two and must reproduce the construction."""
    r = np.random.default_rng(seed)
    nb = K // 16
    codes = r.integers(0, 16, (rows, K)).astype(np.uint8)
    cb = codes.reshape(rows, nb, 16)
    cb[:, :, 0] = np.where(r.random((rows, nb)) < 0.5, 7, 15)     # a +-6 in every block
    sf = r.integers(1, 0x7F, (rows, nb)).astype(np.uint8)         # any finite non-zero scale
    sf[0, 0] = 0x7E
    zero_blk = r.random((rows, nb)) < 0.05
    zero_blk[0, 0] = False
    sf[zero_blk] = 0
    cb[zero_blk] &= 0x8                                           # +-0 in zero blocks
    codes = cb.reshape(rows, K)
    G = np.float32(2.0 ** j)
    x = (F.e2m1_decode(codes).reshape(rows, nb, 16) * F.e4m3_decode(sf)[:, :, None] * float(G))
    return x.reshape(rows, K).astype(np.float32), codes, sf, G


@pytest.mark.parametrize("j", [-12, 0, 7])
def test_round_trip_identity(j):
    x, codes, sf, G = _representable_tensor(64, 512, j, seed=20 + j)
    q = Q.quantize_rows(x)
    assert q.G[0] == G
    assert (q.scales == sf).all()
    assert (q.codes == codes).all()
    assert (q.dequant() == x.astype(np.float64)).all()


@pytest.mark.parametrize("j", [-20, -3, 5, 30])
def test_power_of_two_equivariance(j):
    x = synth.activations(256, 512, seed=30)
    q0 = Q.quantize_rows(x)
    q1 = Q.quantize_rows((x.astype(np.float64) * 2.0 ** j).astype(np.float32))
    assert (q0.codes == q1.codes).all() and (q0.scales == q1.scales).all()
    assert q1.G[0] == np.float32(q0.G[0] * 2.0 ** j)


def test_sign_symmetry():
    x = synth.activations(256, 512, seed=31)
    q0 = Q.quantize_rows(x)
    q1 = Q.quantize_rows(-x)
    assert (q1.codes == (q0.codes ^ 0x8)).all()
    assert (q0.scales == q1.scales).all() and (q0.G == q1.G).all()


def test_groups_are_independent():
    """Per-row scales (the per-token variant) equal quantising each row alone;
    per-segment scales equal quantising each segment alone."""
    x = synth.activations(48, 256, seed=32)
    qr = Q.quantize_rows(x, "row")
    for i in (0, 17, 47):
        qi = Q.quantize_rows(x[i:i + 1])
        assert (qi.codes == qr.codes[i:i + 1]).all() and qi.G[0] == qr.G[i]
    off = [0, 5, 5, 30, 48]
    qs = Q.quantize_rows(x, "segment", seg_offsets=off)
    for s in (0, 2, 3):
        qi = Q.quantize_rows(x[off[s]:off[s + 1]])
        assert (qi.codes == qs.codes[off[s]:off[s + 1]]).all() and qi.G[0] == qs.G[s]
    assert qs.G[1] == 1.0          # empty segment: A = 0 -> S = 1


def test_column_quantisation_is_row_quantisation_of_padded_transpose():
    x = synth.activations(70, 32, seed=33)
    off = np.array([0, 20, 20, 53, 70])
    qc, po = Q.quantize_cols(x, off)
    assert po.tolist() == [0, 32, 32, 80, 112]
    xt = np.zeros((32, 112), np.float32)
    xt[:, 0:20] = x[0:20].T
    xt[:, 32:65] = x[20:53].T
    xt[:, 80:97] = x[53:70].T
    qr = Q.quantize_rows(xt, amax=np.abs(x).max())
    assert (qc.codes == qr.codes).all() and (qc.scales == qr.scales).all()
    # padded columns (always fewer than 16 per segment) hold code 0
    assert (qc.codes[:, 20:32] == 0).all() and (qc.codes[:, 65:80] == 0).all() and (qc.codes[:, 97:] == 0).all()


def test_batched_column_quantisation():
    w = synth.weights((3 * 32, 48), seed=34)
    q = Q.quantize_cols_batched(w, 3)
    for e in range(3):
        qe = Q.quantize_rows(w[e * 32:(e + 1) * 32].T.copy())
        assert (q.codes[e * 48:(e + 1) * 48] == qe.codes).all() and q.G[e] == qe.G[0]


def test_pack_roundtrip():
    c = np.random.default_rng(5).integers(0, 16, (7, 64)).astype(np.uint8)
    p = Q.pack_codes(c)
    assert p.shape == (7, 32)
    assert (p[:, 0] == (c[:, 0] | (c[:, 1] << 4))).all()
    assert (Q.unpack_codes(p) == c).all()


def test_column_quantisation_with_segment_scales():
    """quantize_cols(scale_mode='segment'): every segment's columns equal the row
    quantisation of that segment's own padded transpose under its own tensor scale,
    composed from the per-tensor row quantiser (pinned above); an empty segment
    gets S = 1 and writes nothing."""
    x = synth.activations(70, 48, seed=35)
    x[20:53] *= 40.0                                  # a segment with a much larger amax
    off = np.array([0, 20, 20, 53, 70])
    qc, po = Q.quantize_cols(x, off, "segment")
    assert po.tolist() == [0, 32, 32, 80, 112]
    assert qc.G[1] == 1.0
    for s in (0, 2, 3):
        n = off[s + 1] - off[s]
        width = po[s + 1] - po[s]
        xt = np.zeros((48, width), np.float32)
        xt[:, :n] = x[off[s]:off[s + 1]].T
        qr = Q.quantize_rows(xt, amax=np.abs(x[off[s]:off[s + 1]]).max())
        assert (qc.codes[:, po[s]:po[s + 1]] == qr.codes).all()
        assert (qc.scales[:, po[s] // 16:po[s + 1] // 16] == qr.scales).all()
        assert qc.G[s] == qr.G[0] and (qc.G_block[:, po[s] // 16:po[s + 1] // 16] == qr.G[0]).all()
    assert qc.G[2] != qc.G[0]


def test_expert_weights_one_scale_per_projection():
    """Reading 9: gate, up and down of every expert are separate scale groups.  The
    stacked W13 [E, 2I, H] quantises exactly like its gate and up matrices quantised
    as separate tensors, and W2 like each expert's down matrix; the transposed W13
    of the data gradient holds the gate transpose in K [0, I) and the up transpose
    in [I, 2I), each with its own projection's scale (composed from the pinned
    per-tensor row quantiser)."""
    from oracle import pipeline as P
    E, I, H = 3, 32, 48
    W13 = synth.weights((E, 2 * I, H), seed=36)
    W13[:, I:] *= 100.0                               # up amax ~100x the gate's
    W2 = synth.weights((E, H, I), seed=37)
    w13, w2 = P.quantize_expert_weights(W13, W2)
    w2t, w13t = P.quantize_expert_weights_t(W13, W2)
    assert w13.G.shape == (2 * E,) and w2.G.shape == (E,) and w13t.G.shape == (2 * E,)
    for e in range(E):
        g = Q.quantize_rows(W13[e, :I])
        u = Q.quantize_rows(W13[e, I:])
        d = Q.quantize_rows(W2[e])
        r = slice(2 * I * e, 2 * I * e + I)
        assert (w13.codes[r] == g.codes).all() and (w13.scales[r] == g.scales).all() and w13.G[2 * e] == g.G[0]
        r = slice(2 * I * e + I, 2 * I * (e + 1))
        assert (w13.codes[r] == u.codes).all() and (w13.scales[r] == u.scales).all() and w13.G[2 * e + 1] == u.G[0]
        assert (w2.codes[H * e:H * (e + 1)] == d.codes).all() and w2.G[e] == d.G[0]
        assert w13.G[2 * e + 1] > 50 * w13.G[2 * e]
        gt = Q.quantize_rows(W13[e, :I].T.copy())
        ut = Q.quantize_rows(W13[e, I:].T.copy())
        rows = slice(H * e, H * (e + 1))
        assert (w13t.codes[rows, :I] == gt.codes).all() and (w13t.codes[rows, I:] == ut.codes).all()
        assert (w13t.scales[rows, :I // 16] == gt.scales).all() and (w13t.scales[rows, I // 16:] == ut.scales).all()
        assert w13t.G[2 * e] == gt.G[0] and w13t.G[2 * e + 1] == ut.G[0]
        assert (w13t.G_block[rows, :I // 16] == gt.G[0]).all() and (w13t.G_block[rows, I // 16:] == ut.G[0]).all()
        dt = Q.quantize_rows(W2[e].T.copy())
        assert (w2t.codes[I * e:I * (e + 1)] == dt.codes).all() and w2t.G[e] == dt.G[0]
        # the dequantised transposes equal the transposes of the forward's own values
        # only up to requantisation; their scales are the forward groups' scales
        assert w13t.G[2 * e] == w13.G[2 * e] and w13t.G[2 * e + 1] == w13.G[2 * e + 1]
