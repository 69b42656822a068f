"""Pins of the oracle's fully quantised backward (``pipeline.moe_backward``): every
gradient it returns is the adjoint of the forward grouped GEMM through which that
operand enters, taken on the backward's own dequantised NVFP4 operands, and those
operands are the re-quantised tensors the backward is defined on.

Method: *The 4-bitter Lesson*, section "Results" (case (a): the backward GEMMs
also in NVFP4) and section "Improving Gradient Stability" (a GEMM consumes
DQ(Q(.)) of its operands); the backward operands are re-quantised along their new
contraction dimension.

The identity <dY, f(D)> = <grad, D> for random directions D, with f the linear map
of the forward GEMM, holds exactly in real arithmetic; in FP64 it holds to about
1e-13 relative.  A transposed operand, a wrong expert or segment, a dropped padding
offset or a swapped pair of operands breaks it by O(1).
"""

import numpy as np
import pytest

import synth
from oracle import formats as F
from oracle import moe
from oracle import nvfp4 as Q
from oracle import pipeline as P


def _rows_of_cols(c: np.ndarray, off, po) -> np.ndarray:
    """The rows [R, C] behind a segment-column operand [C, Rpad] (padding dropped)."""
    E = len(off) - 1
    return np.vstack([c[:, po[e]:po[e] + off[e + 1] - off[e]].T for e in range(E)])


@pytest.mark.parametrize("cfg_name", ["tiny"])
def test_nvfp4_backward_is_adjoint_on_its_operands(cfg_name):
    cfg = synth.CONFIGS[cfg_name]
    d = synth.layer_inputs(cfg, with_grads=True)
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.k
    fwd = P.moe_forward(d["X"], d["logits"], d["W13"], d["W2"], k)
    perm = fwd["perm"]
    off = np.asarray(perm["offsets"], np.int64)
    g = P.moe_backward(d["X"], fwd["Hact_bf16"], d["W13"], d["W2"], d["dY2"], d["dY13"], perm)
    po = g["padded_offsets"]
    assert po.tolist() == Q.padded_offsets(off).tolist()
    inner = lambda a, b: float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))
    r = synth.rng(12)

    dY2 = g["dY2q"].dequant()
    dY13 = g["dY13q"].dequant()
    W2t, W13t = g["W2t"].dequant(), g["W13t"].dequant()          # [E*I, H], [E*H, 2I]
    W2 = moe.transpose_batched(W2t, E)                           # [E*H, I]
    W13 = moe.transpose_batched(W13t, E)                         # [E*2I, H]

    # dHact = dY2 . W2: adjoint of D -> D . W2_e^T (the down projection)
    D = r.standard_normal((cfg.R, I))
    lhs = inner(dY2, moe.grouped_gemm_m(D, W2, off, E, H))
    assert abs(lhs - inner(g["dHact"], D)) <= 1e-12 * abs(lhs)
    # dXperm = dY13 . W13: adjoint of D -> D . W13_e^T (gate and up)
    D = r.standard_normal((cfg.R, H))
    lhs = inner(dY13, moe.grouped_gemm_m(D, W13, off, E, 2 * I))
    assert abs(lhs - inner(g["dXperm"], D)) <= 1e-12 * abs(lhs)

    # weight gradients on the token-direction operands, read back as rows
    dY2r = _rows_of_cols(g["dY2c"].dequant(), off, po)
    Hr = _rows_of_cols(g["Hc"].dequant(), off, po)
    dY13r = _rows_of_cols(g["dY13c"].dequant(), off, po)
    Xr = _rows_of_cols(g["Xc"].dequant(), off, po)
    D = r.standard_normal((E * H, I))
    lhs = inner(dY2r, moe.grouped_gemm_m(Hr, D, off, E, H))
    assert abs(lhs - inner(g["dW2"].reshape(E * H, I), D)) <= 1e-12 * abs(lhs)
    D = r.standard_normal((E * 2 * I, H))
    lhs = inner(dY13r, moe.grouped_gemm_m(Xr, D, off, E, 2 * I))
    assert abs(lhs - inner(g["dW13"].reshape(E * 2 * I, H), D)) <= 1e-12 * abs(lhs)
    # the padding of every segment contributes nothing
    for c in (g["dY2c"], g["Hc"], g["dY13c"], g["Xc"]):
        for e in range(E):
            assert (c.codes[:, po[e] + off[e + 1] - off[e]:po[e + 1]] == 0).all()
            assert (c.scales[:, (po[e] + off[e + 1] - off[e] + 15) // 16:po[e + 1] // 16] == 0).all()


def test_nvfp4_backward_operands_are_the_requantised_tensors():
    """The operands the backward GEMMs consume: dY2 and dY13 quantised along their
    rows; their column forms, the SwiGLU output's and X's (gathered into expert
    order) quantised along the tokens of each expert with one tensor scale each (the
    forward's); the weights transposed per expert with the forward's scale groups.
    Checked against compositions of the separately pinned quantisers: rows of a
    column operand equal the row quantisation of each segment's transpose under the
    tensor's scale, and a quantised tensor dequantises within its error bound of
    the source."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    E, H, I = cfg.E, cfg.H, cfg.I
    fwd = P.moe_forward(d["X"], d["logits"], d["W13"], d["W2"], cfg.k)
    perm = fwd["perm"]
    off = np.asarray(perm["offsets"], np.int64)
    g = P.moe_backward(d["X"], fwd["Hact_bf16"], d["W13"], d["W2"], d["dY2"], d["dY13"], perm)
    po = g["padded_offsets"]
    Xperm = d["X"][perm["row_token"]]
    for name, src in (("dY2c", d["dY2"]), ("Hc", fwd["Hact_bf16"]), ("dY13c", d["dY13"]), ("Xc", Xperm)):
        c = g[name]
        A = np.abs(src).max()
        for e in range(E):
            n = off[e + 1] - off[e]
            if n == 0:
                continue
            xt = np.zeros((src.shape[1], po[e + 1] - po[e]), np.float32)
            xt[:, :n] = src[off[e]:off[e + 1]].T
            qr = Q.quantize_rows(xt, amax=A)
            assert (c.codes[:, po[e]:po[e + 1]] == qr.codes).all(), name
            assert (c.scales[:, po[e] // 16:po[e + 1] // 16] == qr.scales).all(), name
    # the weight operand dequantises close to the transposed BF16 weights
    W13t = g["W13t"]
    ref = moe.transpose_batched(d["W13"].reshape(E * 2 * I, H), E)
    err = np.abs(W13t.dequant() - ref)
    step = F.e4m3_decode(W13t.scales).astype(np.float64) * W13t.G_block
    # half the widest E2M1 gap (1) plus the largest clip term of a normal block scale (0.375)
    assert (err <= np.repeat(step, 16, axis=1) * 1.375 * (1 + 2.0 ** -20)).all()
