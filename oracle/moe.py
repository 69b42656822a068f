"""Routing, permutation by expert, grouped expert GEMMs, SwiGLU and combine.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
------------------
*Low-Bit Precision Training*, section "What W4A4 GEMM Actually Changes": expert
routing concentrates activations; W4A4 quantises both GEMM operands and is
applied to the expert layers.  *miniTE news item*, sections "Background: Same
Weights Did Not Guarantee Same Policy" and "Development: Aligning Numerics,
Then Making NVFP4 Fast": the expert work runs as grouped GEMMs.  *The 4-bitter
Lesson*, section "Why is the NVFP4 pretraining recipe not sufficient for RL?"
(footnote 5): an expert holds three projection matrices.  *The 4-bitter Lesson*,
section "Improving Gradient Stability": the quantised product is
y = x . DQ(Q(w)), i.e. the GEMM consumes the dequantised operands.

Readings taken where the pages are silent:

* Router: top-k of the logits (larger first, ties to the lower expert id); the
  weight of a chosen expert is its probability under a softmax over all E
  experts, without renormalisation unless asked.
* Permutation: a stable counting sort of the T*k assignments by expert, so
  within one expert the rows are in increasing token order (and for one token,
  increasing slot j).  expert_offsets is the exclusive prefix sum of the counts.
* Expert FFN: the three projections are gate and up ([I, H] each) and down
  ([H, I]); the gate and up weights of expert e are stacked as rows
  [gate_e; up_e] of one [2I, H] matrix.  SwiGLU is h = silu(g) * u with
  silu(g) = g / (1 + exp(-g)).
* Combine: out[t] = sum over j = 0..k-1 of w[t, j] * Y[row of (t, j)].

All floating point here is FP64.
"""

from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- routing

def route_topk(logits: np.ndarray, k: int, renorm: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """logits [T, E] -> (topk_ids int32 [T, k], topk_w FP64 [T, k])."""
    lg = np.asarray(logits, dtype=np.float64)
    if np.isnan(lg).any():
        raise ValueError("NaN logits are outside the method's contract")
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # a stable sort of -logit keeps equal logits in increasing expert id
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    m = lg.max(axis=1, keepdims=True)
    e = np.exp(lg - m)
    p = e / e.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


def permute(topk_ids: np.ndarray, E: int) -> dict:
    """Stable counting sort of the flat assignments f = t*k + j by expert."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    if ((flat < 0) | (flat >= E)).any():
        raise ValueError("expert id out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    order = np.argsort(flat, kind="stable")          # row r holds assignment order[r]
    row_token = (order // k).astype(np.int64)
    token_row = np.empty(T * k, dtype=np.int64)
    token_row[order] = np.arange(T * k)
    padded = np.concatenate([[0], np.cumsum((counts + 15) // 16 * 16)]).astype(np.int64)
    return dict(counts=counts, offsets=offsets, padded_offsets=padded,
                row_token=row_token, token_row=token_row.reshape(T, k))


# ----------------------------------------------------------------------------- GEMMs

def grouped_gemm_m(A_hat: np.ndarray, B_hat: np.ndarray, offsets, E: int, N: int) -> np.ndarray:
    """Rows of expert e of A (rows [offsets[e], offsets[e+1])) times B_e^T where
    B_e is rows [e*N, (e+1)*N) of B.  A_hat [R, K], B_hat [E*N, K] (dequantised,
    FP64) -> C [R, N] FP64."""
    A_hat = np.asarray(A_hat, dtype=np.float64)
    B_hat = np.asarray(B_hat, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    C = np.zeros((A_hat.shape[0], N), dtype=np.float64)
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:
            C[a:b] = A_hat[a:b] @ B_hat[e * N:(e + 1) * N].T
    return C


def grouped_gemm_k(A_hat: np.ndarray, B_hat: np.ndarray, k_offsets, E: int) -> np.ndarray:
    """Per-expert contraction over that expert's K range only:
    C[e] = A[:, ko[e]:ko[e+1]] . B[:, ko[e]:ko[e+1]]^T.  A_hat [N, Kp],
    B_hat [M, Kp] -> C [E, N, M] FP64; an empty range gives zeros."""
    A_hat = np.asarray(A_hat, dtype=np.float64)
    B_hat = np.asarray(B_hat, dtype=np.float64)
    ko = np.asarray(k_offsets, dtype=np.int64)
    C = np.zeros((E, A_hat.shape[0], B_hat.shape[0]), dtype=np.float64)
    for e in range(E):
        a, b = ko[e], ko[e + 1]
        if b > a:
            C[e] = A_hat[:, a:b] @ B_hat[:, a:b].T
    return C


def transpose_segments(x: np.ndarray, seg_offsets) -> tuple[np.ndarray, np.ndarray]:
    """The column layout of a weight-gradient operand: x [R, C] -> [C, Rpad],
    segment s (rows [off[s], off[s+1])) in columns [po[s], po[s] + n_s) and
    zeros in the rest of its range padded to a multiple of 16.  Returns the
    matrix and the padded offsets po."""
    x = np.asarray(x)
    off = np.asarray(seg_offsets, dtype=np.int64)
    n = np.diff(off)
    po = np.concatenate([[0], np.cumsum((n + 15) // 16 * 16)]).astype(np.int64)
    out = np.zeros((x.shape[1], int(po[-1])), dtype=x.dtype)
    for s in range(len(n)):
        out[:, po[s]:po[s] + n[s]] = x[off[s]:off[s + 1]].T
    return out, po


def transpose_batched(x: np.ndarray, nbatch: int) -> np.ndarray:
    """x [nbatch*m, C] (nbatch matrices of m rows) -> [nbatch*C, m]: every matrix
    transposed in place in the stack (the data-gradient form of expert weights)."""
    x = np.asarray(x)
    R, C = x.shape
    m = R // nbatch
    return x.reshape(nbatch, m, C).transpose(0, 2, 1).reshape(nbatch * C, m)


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(C: np.ndarray) -> np.ndarray:
    """C [R, 2I] with gate columns first -> silu(gate) * up, [R, I]."""
    C = np.asarray(C, dtype=np.float64)
    I = C.shape[1] // 2
    return silu(C[:, :I]) * C[:, I:]


def combine(Y: np.ndarray, token_row: np.ndarray, topk_w: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * Y[token_row[t, j]]  (FP64)."""
    Y = np.asarray(Y, dtype=np.float64)
    tr = np.asarray(token_row, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T, k = tr.shape
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Y[tr[:, j]]
    return out
