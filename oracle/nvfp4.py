"""NVFP4 two-level block quantisation, written out step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix
------------------
*The 4-bitter Lesson*, section "Baseline: A starting recipe with stable training
dynamics": blocks of 16 values, one FP8 E4M3 scale per block, one FP32 scale per
tensor; the two scales together recover the higher-precision value.  Section
"Why is the NVFP4 pretraining recipe not sufficient for RL?" ("Baseline recipe"
paragraph): weights use the standard format with a single FP32 global scale.
Section "Improving Gradient Stability" (footnote 6): a quantiser is
clip(round(w/s), qmin, qmax); DQ denotes its inverse map back to real values.
*Low-Bit Precision Training*, section "What W4A4 GEMM Actually Changes":
activation quantisation uses per-tensor or per-token scaling.  *The 4-bitter
Lesson*, same "Baseline recipe" paragraph: the per-token variant gives each
token row its own FP32 scale computed across the hidden dimension.

Readings taken where the pages are silent (the plainest reading the rest
supports, used identically by the GPU path):

1. Tensor scale.  A = max|x| over the scale group.  The encode scale is
   S = fp32(2688 / A), 2688 = 6 * 448 being the largest E2M1 magnitude times the
   largest E4M3 value, so that the block holding A gets block scale 448 and
   that element the code for 6.  If A == 0 or 2688/A is not finite, S = 1.  The
   stored FP32 decode scale is G = fp32(1 / S).
2. Block scale.  For each 16-element block, a_b = max|x|,
   t_b = fp32(fp32(a_b / 6) * S), sf_b = E4M3(t_b) (nearest, ties to even,
   saturating at 448).
3. Elements.  inv_b = fp32(S / sf_b) (0 when sf_b == 0), v = fp32(x * inv_b),
   q = E2M1(v) (nearest, ties to even, saturating at 6, sign from v).
4. Dequantisation.  x_hat = e2m1(q) * sf_b * G, exact in FP64.
5. Packing.  Element 2i in the low nibble of byte i, element 2i+1 in the high
   nibble; one scale byte per block, blocks in row order.
6. Column (transposed) quantisation for the backward GEMMs: blocks are 16
   consecutive rows of one column, restarting at every segment (expert) start;
   segments are zero-padded to a multiple of 16 rows (padding quantises to
   scale 0, code 0).
7. BF16 dequantisation (the operands of the dequantized backward, *The 4-bitter
   Lesson*, section "Improving Gradient Stability": the backward takes the BF16
   value of DQ(Q(.)) of the very tensor the forward used).  The element value
   e2m1(q) * sf is exact in FP32 (at most 6 significant bits); it is multiplied
   by G in one correctly rounded FP32 operation and the product is rounded to
   BF16 (nearest, ties to even).  This is dequantisation in the quantiser's own
   precision followed by a cast to the BF16 storage format.

8. Stochastic rounding (optional, the pretraining recipe's gradient rounding):
   step 3's E2M1 rounding is replaced by ``formats.e2m1_encode_sr`` with one
   24-bit uniform per element from ``philox`` (counter = (position >> 3,
   output row, stream, 0), key = (seed, 0)); stream 0 for a row-direction output,
   1 for a column-direction (transposed) output.  Block scales stay
   round-to-nearest.

9. Weight scale groups.  The pages give weights one FP32 scale per tensor and
   count three projection matrices per expert (*The 4-bitter Lesson*, section
   "Why is the NVFP4 pretraining recipe not sufficient for RL?", "Baseline
   recipe" paragraph and footnote 5).  Each projection of each expert (gate,
   up, down) is therefore its own scale group.  Where gate and up are stored
   stacked in one matrix, they are two equal row segments with a scale each;
   in the transposed matrix (the data-gradient operand) they are the two halves
   of the new K dimension.

Each FP32 step above is one correctly rounded operation (``formats.f32_div`` and
``formats.f32_mul``), so the integer results (codes, scale bytes) are exactly
defined and the GPU path must reproduce them bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F
from . import philox

BLOCK = 16
SCALE_NUMERATOR = np.float32(6.0 * 448.0)   # largest E2M1 magnitude x largest E4M3 value


@dataclass
class NVFP4:
    """An NVFP4 tensor as the oracle holds it (codes unpacked, one per element)."""
    codes: np.ndarray        # uint8 [rows, K], values 0..15
    scales: np.ndarray       # uint8 [rows, K/16] E4M3 bytes
    G: np.ndarray            # float32 [ngroups] decode scales
    G_block: np.ndarray      # float32 [rows, K/16] decode scale that applies to each block
    amax: np.ndarray         # float32 [ngroups]

    def packed(self) -> np.ndarray:
        return pack_codes(self.codes)

    def dequant(self) -> np.ndarray:
        return dequantize(self.codes, self.scales, self.G_block)


def tensor_scales(amax) -> tuple[np.ndarray, np.ndarray]:
    """Reading 1: encode scale S and decode scale G from a group's amax."""
    A = np.atleast_1d(np.asarray(amax, dtype=np.float32))
    S = np.ones_like(A)
    pos = A > 0
    with np.errstate(over="ignore", divide="ignore"):
        q = F.f32_div(np.full_like(A, SCALE_NUMERATOR), np.where(pos, A, np.float32(1)))
    S = np.where(pos & np.isfinite(q), q, np.float32(1)).astype(np.float32)
    G = F.f32_div(np.ones_like(S), S)
    return S, G


def quantize_blocks(x: np.ndarray, S_block: np.ndarray, sr_seed: int | None = None,
                    sr_stream: int = 0, sr_rows=None, sr_pos0: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Readings 2 and 3 on x [rows, K] (FP32 values, K % 16 == 0) with the encode
    scale given per block (S_block [rows, K/16]); with sr_seed, reading 8 for the
    elements (x is in its output layout: element (i, j) is position sr_pos0 + j of
    output row sr_rows[i], by default row i).  Returns (codes, scale bytes)."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    if not np.isfinite(x).all():
        raise ValueError("non-finite input is outside the method's contract")
    xb = x.reshape(rows, K // BLOCK, BLOCK)
    a_b = np.abs(xb).max(axis=2)                                   # exact
    S_block = np.asarray(S_block, dtype=np.float32)
    t_b = F.f32_mul(F.f32_div(a_b, np.float32(6.0)), S_block)
    sf = F.e4m3_encode(t_b)
    sf_val = F.e4m3_decode(sf).astype(np.float32)                  # exact
    safe = np.where(sf > 0, sf_val, np.float32(1))
    inv = np.where(sf > 0, F.f32_div(S_block, safe), np.float32(0)).astype(np.float32)
    v = F.f32_mul(xb, inv[:, :, None])
    if sr_seed is None:
        codes = F.e2m1_encode(v).reshape(rows, K)
    else:
        ids = np.arange(rows) if sr_rows is None else np.asarray(sr_rows, np.int64)
        u = philox.uniform24(ids[:, None], sr_pos0 + np.arange(K)[None, :], sr_stream, sr_seed)
        codes = F.e2m1_encode_sr(v.reshape(rows, K), u)
    return codes, sf


def _group_amax(absx_rows_max: np.ndarray, group_of_row: np.ndarray, ngroups: int) -> np.ndarray:
    amax = np.zeros(ngroups, dtype=np.float32)
    np.maximum.at(amax, group_of_row, absx_rows_max)
    return amax


def row_groups(rows: int, scale_mode: str, seg_offsets=None, nseg: int | None = None) -> tuple[np.ndarray, int]:
    """Group index of every row.  ``tensor``: one group.  ``segment``: rows
    [seg_offsets[s], seg_offsets[s+1]) form group s (equal segments when
    seg_offsets is None and nseg is given).  ``row``: every row its own group
    (the per-token variant)."""
    if scale_mode == "tensor":
        return np.zeros(rows, dtype=np.int64), 1
    if scale_mode == "row":
        return np.arange(rows, dtype=np.int64), rows
    if scale_mode == "segment":
        if seg_offsets is None:
            if not nseg or rows % nseg:
                raise ValueError("equal segments need rows % nseg == 0")
            return np.arange(rows, dtype=np.int64) // (rows // nseg), nseg
        off = np.asarray(seg_offsets, dtype=np.int64)
        g = np.searchsorted(off, np.arange(rows), side="right") - 1
        return g.astype(np.int64), len(off) - 1
    raise ValueError(scale_mode)


def quantize_rows(x: np.ndarray, scale_mode: str = "tensor", seg_offsets=None, nseg=None,
                  amax=None, sr_seed: int | None = None, _sr_stream: int = 0, sr_rows=None) -> NVFP4:
    """NVFP4 along the contiguous dimension K of x [rows, K] (stochastic rounding of
    the elements with sr_seed; sr_rows: the rows' indices in the whole tensor when
    x is a selection of its rows)."""
    x = np.asarray(x, dtype=np.float32)
    rows, K = x.shape
    grp, ngroups = row_groups(rows, scale_mode, seg_offsets, nseg)
    if amax is None:
        row_max = np.abs(x).max(axis=1) if K else np.zeros(rows, np.float32)
        amax = _group_amax(row_max, grp, ngroups)
    amax = np.asarray(amax, dtype=np.float32).reshape(ngroups)
    S, G = tensor_scales(amax)
    S_block = np.repeat(S[grp][:, None], K // BLOCK, axis=1)
    codes, sf = quantize_blocks(x, S_block, sr_seed, _sr_stream, sr_rows)
    G_block = np.repeat(G[grp][:, None], K // BLOCK, axis=1)
    return NVFP4(codes, sf, G, G_block, amax)


def padded_offsets(seg_offsets) -> np.ndarray:
    """Segment starts after padding every segment to a multiple of 16 rows."""
    off = np.asarray(seg_offsets, dtype=np.int64)
    n = np.diff(off)
    return np.concatenate([[0], np.cumsum((n + BLOCK - 1) // BLOCK * BLOCK)]).astype(np.int64)


def quantize_cols(x: np.ndarray, seg_offsets, scale_mode: str = "tensor", amax=None,
                  sr_seed: int | None = None, sr_rows=None, sr_pos0: int = 0) -> tuple[NVFP4, np.ndarray]:
    """Reading 6, segmented-K form: x [R, C] -> NVFP4 of its transpose [C, Rpad],
    where the rows of segment s land in columns [po[s], po[s] + n_s) and the
    rest of the segment's padded range is zero.  The scale group is the whole
    tensor (``tensor``) or each segment (``segment``).  Returns the tensor and
    the padded offsets po.  For stochastic rounding of a selection of x's
    columns and rows, sr_rows are the output rows (x's column indices) and sr_pos0
    the position of the first row."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    off = np.asarray(seg_offsets, dtype=np.int64)
    po = padded_offsets(off)
    nseg = len(off) - 1
    xt = np.zeros((C, int(po[-1])), dtype=np.float32)
    seg_of_block = np.zeros(int(po[-1]) // BLOCK, dtype=np.int64)
    for s in range(nseg):
        xt[:, po[s]:po[s] + off[s + 1] - off[s]] = x[off[s]:off[s + 1]].T
        seg_of_block[po[s] // BLOCK:po[s + 1] // BLOCK] = s
    if scale_mode == "tensor":
        if amax is None:
            amax = np.abs(x).max() if x.size else np.float32(0)
        amax = np.asarray(amax, np.float32).reshape(1)
        S, G = tensor_scales(amax)
        S_block = np.full((C, xt.shape[1] // BLOCK), S[0], np.float32)
        G_block = np.full_like(S_block, G[0])
    elif scale_mode == "segment":
        if amax is None:
            amax = np.array([np.abs(x[off[s]:off[s + 1]]).max() if off[s + 1] > off[s] else 0
                             for s in range(nseg)], dtype=np.float32)
        amax = np.asarray(amax, np.float32).reshape(nseg)
        S, G = tensor_scales(amax)
        S_block = np.broadcast_to(S[seg_of_block][None, :], (C, len(seg_of_block))).astype(np.float32)
        G_block = np.broadcast_to(G[seg_of_block][None, :], (C, len(seg_of_block))).astype(np.float32)
    else:
        raise ValueError(scale_mode)
    codes, sf = quantize_blocks(xt, S_block, sr_seed, 1, sr_rows, sr_pos0)
    return NVFP4(codes, sf, G, G_block, amax), po


def quantize_cols_batched(x: np.ndarray, nbatch: int, scale_mode: str = "segment", amax=None,
                          sr_seed: int | None = None) -> NVFP4:
    """Reading 6, batched form (weights): x [nbatch*m, C] is nbatch matrices of
    m rows (m % 16 == 0); each is transposed to [C, m] and quantised along m.
    The result stacks the transposes: [nbatch*C, m].  Scale group: each matrix
    (``segment``), the whole tensor (``tensor``), or each half of each matrix's
    rows (``segment_halves``: reading 9, two projections stacked in one matrix,
    e.g. an expert's gate and up weights; the first half of the transposed
    matrix's new K then carries the first projection's scale and the second half
    the second's, so no block mixes them).  ``amax`` (optional) holds one value
    per group in that order."""
    x = np.asarray(x, dtype=np.float32)
    R, C = x.shape
    m = R // nbatch
    if R % nbatch or m % BLOCK:
        raise ValueError("batched column quantisation needs equal matrices of 16k rows")
    xt = x.reshape(nbatch, m, C).transpose(0, 2, 1).reshape(nbatch * C, m)
    if scale_mode == "segment":
        return quantize_rows(xt, "segment", nseg=nbatch, amax=amax, sr_seed=sr_seed, _sr_stream=1)
    if scale_mode == "tensor":
        return quantize_rows(xt, "tensor", amax=amax, sr_seed=sr_seed, _sr_stream=1)
    if scale_mode != "segment_halves":
        raise ValueError(scale_mode)
    half = m // 2
    if m % 2 or half % BLOCK:
        raise ValueError("halves of a matrix must be whole blocks of 16 rows")
    # group 2s + h: rows [s*m + h*half, s*m + (h+1)*half) of x
    if amax is None:
        amax = np.abs(x).reshape(2 * nbatch, half * C).max(axis=1) if x.size else np.zeros(2 * nbatch)
    amax = np.asarray(amax, np.float32).reshape(2 * nbatch)
    S, G = tensor_scales(amax)
    nblk = m // BLOCK
    grp = 2 * np.repeat(np.arange(nbatch), C)[:, None] + (np.arange(nblk)[None, :] >= nblk // 2)
    codes, sf = quantize_blocks(xt, S[grp], sr_seed, 1)
    return NVFP4(codes, sf, G, G[grp], amax)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Reading 5: two codes per byte, even element in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequantize_bf16(t: NVFP4) -> np.ndarray:
    """Reading 7: the BF16 value of every element of t, returned as float32 values
    (each exactly a BF16 number)."""
    vals = F.e2m1_decode(t.codes)
    rows, K = vals.shape
    sfv = F.e4m3_decode(t.scales).astype(np.float64)
    exact = (vals.reshape(rows, K // BLOCK, BLOCK) * sfv[:, :, None]).reshape(rows, K)   # e2m1 * sf, exact
    G = np.repeat(np.asarray(t.G_block, np.float32), BLOCK, axis=1)
    return F.bf16_bits_to_f32(F.f32_to_bf16_bits(F.f32_mul(exact.astype(np.float32), G)))


def dequantize(codes: np.ndarray, scales: np.ndarray, G_block: np.ndarray) -> np.ndarray:
    """Reading 4: e2m1(q) * sf * G per element, in FP64 (exact)."""
    vals = F.e2m1_decode(codes)
    rows, K = vals.shape
    sfv = F.e4m3_decode(scales).astype(np.float64) * np.asarray(G_block, np.float64)
    return (vals.reshape(rows, K // BLOCK, BLOCK) * sfv[:, :, None]).reshape(rows, K)
