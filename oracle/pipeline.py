"""The whole expert-layer forward and backward, stage by stage.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The forward follows the order the pages imply for a W4A4 expert layer (*Low-Bit
Precision Training*, section "What W4A4 GEMM Actually Changes"; *miniTE news
item*, section "Development: Aligning Numerics, Then Making NVFP4 Fast"):
route, quantise activations, permute tokens by expert, grouped GEMM with gate
and up projections and SwiGLU, quantise the SwiGLU output, grouped GEMM with
the down projection, weighted combine back to token order.

The backward computes the two data-gradient and two weight-gradient grouped
GEMMs of the expert layer with every operand re-quantised to NVFP4 along its
new contraction dimension (the fully quantised recipe, case (a) of *The
4-bitter Lesson*, section "Results"), starting from upstream gradients dY2 (of
the down projection's output rows) and dY13 (of the gate/up output rows).

The BF16 variants (*The 4-bitter Lesson*, sections "Why is the NVFP4
pretraining recipe not sufficient for RL?" and "Improving Gradient Stability"):
``moe_forward_bf16`` is the unquantised layer (the comparison point for the
W4A4 forward); ``moe_backward_bf16`` computes the same four gradients with BF16
operands, either the unquantised tensors (the conservative baseline: the
backward differentiates x . w although the forward used Q(w)) or the BF16
dequantised values of the exact NVFP4 tensors of the forward ("dequantized
backward", applied to weights and activations).  The upstream gradients stay
BF16 in both.

Weights carry one FP32 scale per expert and projection (reading 9 of ``nvfp4``):
gate, up and down are separate scale groups, in the forward layout and in the
transposed layout of the data gradients.

Storage roundings of the GPU path are mirrored (SwiGLU output stored as BF16,
expert outputs as FP32), so these functions give an end-to-end oracle result.
Pins: the single-expert top-1 forward equals a dense W4A4 SwiGLU MLP, and every
gradient of ``moe_backward`` is the adjoint of its forward GEMM on the backward's
own dequantised operands (tests/test_oracle_moe.py, tests/test_oracle_backward.py).
End to end, the GPU pipeline agrees with this one only statistically: after an
intermediate tensor is re-quantised, an FP32-vs-FP64 accumulation difference
upstream can move an element across an FP4 rounding boundary.  The GPU tests
therefore compare every stage separately, each fed the GPU's own stage inputs, and
the whole layer only loosely.
"""

from __future__ import annotations

import numpy as np

from . import formats as F
from . import moe
from . import nvfp4 as Q


def gather_rows(t: Q.NVFP4, row_token: np.ndarray) -> Q.NVFP4:
    """Rows of an NVFP4 tensor in permuted order (codes, scales and the decode
    scale of each block travel with the row)."""
    rt = np.asarray(row_token, dtype=np.int64)
    return Q.NVFP4(t.codes[rt], t.scales[rt], t.G, t.G_block[rt], t.amax)


def quantize_expert_weights(W13: np.ndarray, W2: np.ndarray) -> tuple[Q.NVFP4, Q.NVFP4]:
    """Reading 9 of ``nvfp4``: one FP32 scale per expert and projection.  W13
    [E, 2I, H] holds gate_e then up_e: 2E row segments of I rows, group 2e the
    gate and 2e + 1 the up projection of expert e; W2 [E, H, I]: E segments."""
    E, I2, H = W13.shape
    W13q = Q.quantize_rows(np.asarray(W13, np.float32).reshape(E * I2, H), "segment", nseg=2 * E)
    W2q = Q.quantize_rows(np.asarray(W2, np.float32).reshape(E * H, I2 // 2), "segment", nseg=E)
    return W13q, W2q


def quantize_expert_weights_t(W13: np.ndarray, W2: np.ndarray) -> tuple[Q.NVFP4, Q.NVFP4]:
    """The data gradients' weight operands, transposed per expert and re-quantised
    along the new K, with the forward's scale groups (reading 9 of ``nvfp4``):
    W2^T [E*I, H] one scale per expert; W13^T [E*H, 2I] one scale per expert for
    K in [0, I) (gate) and one for [I, 2I) (up)."""
    E, I2, H = W13.shape
    W2t = Q.quantize_cols_batched(np.asarray(W2, np.float32).reshape(E * H, I2 // 2), E)
    W13t = Q.quantize_cols_batched(np.asarray(W13, np.float32).reshape(E * I2, H), E, "segment_halves")
    return W2t, W13t


def moe_forward(X: np.ndarray, logits: np.ndarray, W13: np.ndarray, W2: np.ndarray, k: int,
                renorm: bool = False, out_bf16: bool = False) -> dict:
    """X [T, H] (FP32 values of BF16 inputs), logits [T, E], W13 [E, 2I, H] with
    rows [gate_e; up_e], W2 [E, H, I].  Returns every stage's result."""
    X = np.asarray(X, np.float32)
    T, H = X.shape
    E, I2, _ = W13.shape
    I = I2 // 2
    ids, w = moe.route_topk(logits, k, renorm)
    perm = moe.permute(ids, E)
    Xq = Q.quantize_rows(X, "tensor")
    Xg = gather_rows(Xq, perm["row_token"])
    W13q, W2q = quantize_expert_weights(W13, W2)
    C1 = moe.grouped_gemm_m(Xg.dequant(), W13q.dequant(), perm["offsets"], E, I2)
    Hact = moe.swiglu(C1)
    Hact_bf16 = F.bf16_bits_to_f32(F.f32_to_bf16_bits(F.f32(Hact)))
    Hq = Q.quantize_rows(Hact_bf16, "tensor")
    Y = moe.grouped_gemm_m(Hq.dequant(), W2q.dequant(), perm["offsets"], E, H)
    Y32 = F.f32(Y)
    out = moe.combine(Y32, perm["token_row"], w)
    out = F.f32(out)
    if out_bf16:
        out = F.bf16_bits_to_f32(F.f32_to_bf16_bits(out))
    return dict(topk_ids=ids, topk_w=w, perm=perm, Xq=Xq, Xg=Xg, W13q=W13q, W2q=W2q,
                C1=C1, Hact=Hact, Hact_bf16=Hact_bf16, Hq=Hq, Y=Y32, out=out)


def bf16(x: np.ndarray) -> np.ndarray:
    """Values rounded to BF16 (nearest, ties to even), as float32."""
    return F.bf16_bits_to_f32(F.f32_to_bf16_bits(F.f32(x)))


def moe_forward_bf16(X: np.ndarray, logits: np.ndarray, W13: np.ndarray, W2: np.ndarray, k: int,
                     renorm: bool = False) -> dict:
    """The unquantised layer on BF16 values: same routing, permutation, SwiGLU
    and combine as ``moe_forward``, with the GEMMs on the BF16 operands."""
    X = np.asarray(X, np.float32)
    T, H = X.shape
    E, I2, _ = W13.shape
    I = I2 // 2
    ids, w = moe.route_topk(logits, k, renorm)
    perm = moe.permute(ids, E)
    Xperm = X[np.asarray(perm["row_token"], np.int64)]
    C1 = moe.grouped_gemm_m(Xperm, np.asarray(W13, np.float32).reshape(E * I2, H), perm["offsets"], E, I2)
    Hact = moe.swiglu(C1)
    Hact_bf16 = bf16(Hact)
    Y = moe.grouped_gemm_m(Hact_bf16, np.asarray(W2, np.float32).reshape(E * H, I), perm["offsets"], E, H)
    Y32 = F.f32(Y)
    out = F.f32(moe.combine(Y32, perm["token_row"], w))
    return dict(topk_ids=ids, topk_w=w, perm=perm, C1=C1, Hact=Hact, Hact_bf16=Hact_bf16, Y=Y32, out=out)


def backward_operands_bf16(X: np.ndarray, Hact_bf16: np.ndarray, W13: np.ndarray, W2: np.ndarray,
                           fwd: dict | None = None) -> dict:
    """The four BF16 operands of the backward that come from the forward: X, Hact,
    W13 and W2.  With ``fwd`` (the result of ``moe_forward``) they are the BF16
    dequantised values of the forward's NVFP4 tensors (reading 7 of ``nvfp4``);
    without it, the BF16 tensors themselves."""
    E, I2, H = W13.shape
    I = I2 // 2
    if fwd is None:
        return dict(X=np.asarray(X, np.float32), Hact=np.asarray(Hact_bf16, np.float32),
                    W13=np.asarray(W13, np.float32).reshape(E * I2, H),
                    W2=np.asarray(W2, np.float32).reshape(E * H, I))
    return dict(X=Q.dequantize_bf16(fwd["Xq"]), Hact=Q.dequantize_bf16(fwd["Hq"]),
                W13=Q.dequantize_bf16(fwd["W13q"]), W2=Q.dequantize_bf16(fwd["W2q"]))


def moe_backward_bf16(ops: dict, dY2: np.ndarray, dY13: np.ndarray, perm: dict) -> dict:
    """The four gradients of ``moe_backward`` with BF16 operands ``ops`` (from
    ``backward_operands_bf16``; X un-permuted, Hact in expert order) and BF16
    upstream gradients, FP64 accumulation.  The weight gradients contract over
    each expert's own rows, laid out as the column operands of the GPU path."""
    E = len(perm["offsets"]) - 1
    H = ops["X"].shape[1]
    I = ops["Hact"].shape[1]
    off = perm["offsets"]
    Xperm = ops["X"][np.asarray(perm["row_token"], np.int64)]
    W2t = moe.transpose_batched(ops["W2"], E)      # [E*I, H]
    W13t = moe.transpose_batched(ops["W13"], E)    # [E*H, 2I]
    dHact = moe.grouped_gemm_m(dY2, W2t, off, E, I)
    dXperm = moe.grouped_gemm_m(dY13, W13t, off, E, H)
    dY2c, po = moe.transpose_segments(np.asarray(dY2, np.float32), off)
    Hc, _ = moe.transpose_segments(ops["Hact"], off)
    dY13c, _ = moe.transpose_segments(np.asarray(dY13, np.float32), off)
    Xc, _ = moe.transpose_segments(Xperm, off)
    dW2 = moe.grouped_gemm_k(dY2c, Hc, po, E)
    dW13 = moe.grouped_gemm_k(dY13c, Xc, po, E)
    return dict(W2t=W2t, W13t=W13t, dHact=dHact, dXperm=dXperm, dY2c=dY2c, Hc=Hc, dY13c=dY13c, Xc=Xc,
                padded_offsets=po, dW2=dW2, dW13=dW13)


def moe_backward(X: np.ndarray, Hact_bf16: np.ndarray, W13: np.ndarray, W2: np.ndarray,
                 dY2: np.ndarray, dY13: np.ndarray, perm: dict) -> dict:
    """Data and weight gradients of both grouped GEMMs, all operands re-quantised
    along the new contraction dimension.

    dHact  [R, I]     = dY2_e  . W2_e          (contraction over H)
    dXperm [R, H]     = dY13_e . W13_e         (contraction over 2I)
    dW2    [E, H, I]  = dY2_e^T  . Hact_e      (contraction over expert e's tokens)
    dW13   [E, 2I, H] = dY13_e^T . Xperm_e
    """
    X = np.asarray(X, np.float32)
    E, I2, H = W13.shape
    I = I2 // 2
    off = perm["offsets"]
    Xperm = X[np.asarray(perm["row_token"], np.int64)]
    dY2q = Q.quantize_rows(dY2, "tensor")
    dY13q = Q.quantize_rows(dY13, "tensor")
    W2t, W13t = quantize_expert_weights_t(W13, W2)      # [E*I, H], [E*H, 2I]
    dHact = moe.grouped_gemm_m(dY2q.dequant(), W2t.dequant(), off, E, I)
    dXperm = moe.grouped_gemm_m(dY13q.dequant(), W13t.dequant(), off, E, H)
    dY2c, po = Q.quantize_cols(dY2, off)          # [H, Rpad]
    Hc, _ = Q.quantize_cols(Hact_bf16, off)        # [I, Rpad]
    dY13c, _ = Q.quantize_cols(dY13, off)         # [2I, Rpad]
    Xc, _ = Q.quantize_cols(Xperm, off)           # [H, Rpad]
    dW2 = moe.grouped_gemm_k(dY2c.dequant(), Hc.dequant(), po, E)
    dW13 = moe.grouped_gemm_k(dY13c.dequant(), Xc.dequant(), po, E)
    return dict(dY2q=dY2q, dY13q=dY13q, W2t=W2t, W13t=W13t, dHact=dHact, dXperm=dXperm,
                dY2c=dY2c, Hc=Hc, dY13c=dY13c, Xc=Xc, padded_offsets=po, dW2=dW2, dW13=dW13)
