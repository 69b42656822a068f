"""GPU NVFP4 quantiser vs the oracle: codes, scale bytes and tensor-scale bits must
match exactly; repeated calls must be bitwise identical."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import nvfp4 as Q
from oracle import pipeline as P
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, same_bits

pytestmark = pytest.mark.gpu


def _assert_exact(t, ref: Q.NVFP4, ng=None):
    codes = host(t.codes)
    assert codes.shape == (ref.codes.shape[0], ref.codes.shape[1] // 2)
    assert np.array_equal(codes, ref.packed()), "FP4 codes differ"
    assert np.array_equal(host(t.scales), ref.scales), "E4M3 scale bytes differ"
    G = host(t.tscale)[: (ng or len(ref.G))]
    assert np.array_equal(G.view(np.uint32), ref.G.astype(np.float32).view(np.uint32)), "tensor scales differ"


@pytest.mark.parametrize("T,H,outliers,seed", [(512, 256, True, 1), (37, 48, True, 2), (8192, 2048, False, 3),
                                               (16384, 2048, True, 4), (3, 16, False, 5)])
def test_rows_tensor_scale_bf16(gpu_lib, T, H, outliers, seed):
    x = synth.activations(T, H, seed, outliers=outliers)
    t = gpu_lib.nvfp4_quantize(dev_bf16(x))
    _assert_exact(t, Q.quantize_rows(x))
    t2 = gpu_lib.nvfp4_quantize(dev_bf16(x))
    assert same_bits(t.codes, t2.codes) and same_bits(t.scales, t2.scales) and same_bits(t.tscale, t2.tscale)


def test_rows_fp32_input_and_strided(gpu_lib):
    r = np.random.default_rng(7)
    x = (r.standard_normal((96, 160)) * 3).astype(np.float32)
    xd = torch.zeros((96, 192), dtype=torch.float32, device="cuda")
    xd[:, :160] = dev_f32(x)
    t = gpu_lib.nvfp4_quantize(xd[:, :160])
    _assert_exact(t, Q.quantize_rows(x))


def test_weights_per_expert_scale(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    W13, W2 = synth.expert_weights(cfg)
    t = gpu_lib.nvfp4_quantize(dev_bf16(W13.reshape(-1, cfg.H)), scale_mode=gpu_lib.NV4_SCALE_SEGMENT, nseg=cfg.E)
    _assert_exact(t, Q.quantize_rows(W13.reshape(-1, cfg.H), "segment", nseg=cfg.E))
    t = gpu_lib.nvfp4_quantize(dev_bf16(W2.reshape(-1, cfg.I)), scale_mode=gpu_lib.NV4_SCALE_SEGMENT, nseg=cfg.E)
    _assert_exact(t, Q.quantize_rows(W2.reshape(-1, cfg.I), "segment", nseg=cfg.E))


def test_weights_one_scale_per_projection(gpu_lib):
    """S2 and the weight transposes of S8 with one FP32 scale per expert and projection
    (gate, up, down), gate and up amax about 100x apart: W13 in 2E row segments, W13^T
    with a scale per K half (including a K half that is not a multiple of the 128-row
    tile, so a tile straddles the two scale groups), all bit-exact."""
    for E, I, H in ((8, 128, 256), (3, 80, 96)):
        W13 = synth.weights((E, 2 * I, H), 60 + I)
        W13[:, I:] *= 100.0
        W13 = synth.to_bf16_values(W13)
        W2 = synth.weights((E, H, I), 61 + I)
        ref13, ref2 = P.quantize_expert_weights(W13, W2)
        ref2t, ref13t = P.quantize_expert_weights_t(W13, W2)
        w = gpu_lib.quantize_expert_weights(dev_bf16(W13), dev_bf16(W2))
        wt = gpu_lib.quantize_expert_weights_t(dev_bf16(W13), dev_bf16(W2))
        _assert_exact(w.w13, ref13)
        _assert_exact(w.w2, ref2)
        _assert_exact(wt.w2t, ref2t)
        _assert_exact(wt.w13t, ref13t)
        assert w.w13.nseg == 2 * E and wt.w13t.scale_mode == gpu_lib.NV4_SCALE_SEGMENT_HALVES
        G = host(w.w13.tscale)
        assert (G[1::2] > 50 * G[0::2]).all()


def test_weights_full_size_sampled_experts(gpu_lib):
    """S2 at the Qwen3-30B-A3B expert shapes (128 experts, hidden 2048, intermediate
    768): all 384 tensor scales exact, and every byte of four experts' gate, up and
    down matrices and of their transposes exact."""
    cfg = synth.CONFIGS["learner_64k"]
    E, H, I = cfg.E, cfg.H, cfg.I
    W13, W2 = synth.expert_weights(cfg)
    w = gpu_lib.quantize_expert_weights(dev_bf16(W13), dev_bf16(W2))
    wt = gpu_lib.quantize_expert_weights_t(dev_bf16(W13), dev_bf16(W2))
    torch.cuda.synchronize()
    a13 = np.abs(W13.reshape(2 * E, I * H)).max(axis=1)
    a2 = np.abs(W2.reshape(E, H * I)).max(axis=1)
    G13 = Q.tensor_scales(a13)[1]
    G2 = Q.tensor_scales(a2)[1]
    assert np.array_equal(host(w.w13.tscale).view(np.uint32), G13.view(np.uint32))
    assert np.array_equal(host(w.w2.tscale).view(np.uint32), G2.view(np.uint32))
    assert np.array_equal(host(wt.w13t.tscale).view(np.uint32), G13.view(np.uint32))
    assert np.array_equal(host(wt.w2t.tscale).view(np.uint32), G2.view(np.uint32))
    for e in (0, 37, 90, 127):
        r13, r2 = P.quantize_expert_weights(W13[e:e + 1], W2[e:e + 1])
        r2t, r13t = P.quantize_expert_weights_t(W13[e:e + 1], W2[e:e + 1])
        sl = lambda t, a, b: (host(t.codes[a:b]), host(t.scales[a:b]))
        for t, ref, a, b in ((w.w13, r13, e * 2 * I, (e + 1) * 2 * I), (w.w2, r2, e * H, (e + 1) * H),
                             (wt.w13t, r13t, e * H, (e + 1) * H), (wt.w2t, r2t, e * I, (e + 1) * I)):
            c, sc = sl(t, a, b)
            assert np.array_equal(c, ref.packed()) and np.array_equal(sc, ref.scales)


def test_segment_offsets_with_empty_segments(gpu_lib):
    x = synth.activations(300, 128, 8)
    off = np.array([0, 0, 17, 17, 200, 300, 300])
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), scale_mode=gpu_lib.NV4_SCALE_SEGMENT, nseg=6, seg_offsets=dev_i32(off))
    ref = Q.quantize_rows(x, "segment", seg_offsets=off)
    _assert_exact(t, ref)
    assert host(t.tscale)[0] == 1.0 and host(t.tscale)[5] == 1.0


@pytest.mark.parametrize("T,H", [(512, 256), (1000, 2048), (7, 32)])
def test_rows_per_token_scale(gpu_lib, T, H):
    x = synth.activations(T, H, 9)
    amax = torch.empty(T, dtype=torch.float32, device="cuda")
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), scale_mode=gpu_lib.NV4_SCALE_ROW, amax_out=amax)
    ref = Q.quantize_rows(x, "row")
    _assert_exact(t, ref)
    assert np.array_equal(host(amax), np.abs(x).max(axis=1))


def test_amax_in_and_out(gpu_lib):
    x = synth.activations(256, 512, 10)
    A = np.float32(np.abs(x).max())
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    t1 = gpu_lib.nvfp4_quantize(dev_bf16(x), amax_out=amax)
    assert host(amax)[0] == A
    # a supplied amax (here twice the true one) replaces the amax pass
    a2 = torch.tensor([2 * A], dtype=torch.float32, device="cuda")
    t2 = gpu_lib.nvfp4_quantize(dev_bf16(x), amax_in=a2)
    _assert_exact(t2, Q.quantize_rows(x, amax=np.array([2 * A], np.float32)))
    _assert_exact(t1, Q.quantize_rows(x))


@pytest.mark.parametrize("case", ["zeros", "tiny", "subnormal_bf16", "huge", "outlier_rows"])
def test_edge_values(gpu_lib, case):
    r = np.random.default_rng(11)
    if case == "zeros":
        x = np.zeros((64, 64), np.float32)
        x[3, 5] = -0.0
    elif case == "tiny":           # 2688 / A overflows: S = 1
        x = (r.standard_normal((32, 64)) * 1e-37).astype(np.float32)
    elif case == "subnormal_bf16":
        x = synth.to_bf16_values((r.standard_normal((32, 64)) * 1e-39).astype(np.float32))
    elif case == "huge":
        x = synth.to_bf16_values((r.standard_normal((32, 64)) * 1e37).astype(np.float32))
    else:
        x = synth.activations(64, 256, 12)
        x[5] *= 1000
    x = synth.to_bf16_values(x)
    t = gpu_lib.nvfp4_quantize(dev_bf16(x))
    _assert_exact(t, Q.quantize_rows(x))


def test_nonfinite_sets_status(gpu_lib):
    x = np.ones((16, 64), np.float32)
    x[3, 7] = np.inf
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.nvfp4_quantize(dev_bf16(x), dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & gpu_lib.NV4_DS_NONFINITE


@pytest.mark.parametrize("layout", ["rows", "cols", "rows_and_cols", "per_row"])
@pytest.mark.parametrize("bad", [np.inf, -np.inf, np.nan])
def test_nonfinite_sets_status_without_amax_pass(gpu_lib, layout, bad):
    """With the amax given (no amax pass), each quantisation kernel itself flags a NaN
    or infinity, wherever it sits in the tile (here in a lane other than the first)."""
    R, K = 300, 256
    x = synth.to_bf16_values(synth.activations(R, K, 21))
    x[137, 203] = bad
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    amax = torch.tensor([4.0], dtype=torch.float32, device="cuda")
    xd = dev_bf16(x)
    if layout == "rows":
        gpu_lib.nvfp4_quantize(xd, amax_in=amax, dev_status=st)
    elif layout == "per_row":
        gpu_lib.nvfp4_quantize(xd, scale_mode=gpu_lib.NV4_SCALE_ROW, dev_status=st)
    else:
        off = torch.tensor([0, 120, R], dtype=torch.int32, device="cuda")
        pad = torch.tensor([0, 128, 128 + 192], dtype=torch.int32, device="cuda")
        kw = dict(nseg=2, seg_offsets=off, seg_padded_offsets=pad, amax_in=amax, dev_status=st)
        if layout == "cols":
            gpu_lib.nvfp4_quantize(xd, layout=gpu_lib.NV4_COLS, **kw)
        else:
            gpu_lib.nvfp4_quantize(xd, layout=gpu_lib.NV4_ROWS_AND_COLS, **kw)
    torch.cuda.synchronize()
    assert int(st.item()) & gpu_lib.NV4_DS_NONFINITE


def test_columns_segmented(gpu_lib):
    """Transposed quantisation by expert segment, as the weight-gradient GEMMs use."""
    cfg = synth.CONFIGS["tiny"]
    x = synth.activations(cfg.R, 96, 13)
    counts = np.bincount(synth.rng(14).integers(0, cfg.E, cfg.R), minlength=cfg.E)
    counts[2] = 0
    counts[3] += (cfg.R - counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)])
    po = Q.padded_offsets(off)
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), layout=gpu_lib.NV4_COLS, nseg=cfg.E, seg_offsets=dev_i32(off),
                               seg_padded_offsets=dev_i32(po))
    ref, po_ref = Q.quantize_cols(x, off)
    assert np.array_equal(po, po_ref)
    Kp = int(po[-1])
    codes = host(t.codes)[:, : Kp // 2]
    scales = host(t.scales)[:, : Kp // 16]
    assert np.array_equal(codes, ref.packed())
    assert np.array_equal(scales, ref.scales)
    assert host(t.tscale)[0] == ref.G[0]


def test_columns_batched_weights(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    _, W2 = synth.expert_weights(cfg)
    x = W2.reshape(cfg.E * cfg.H, cfg.I)
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), layout=gpu_lib.NV4_COLS_BATCHED, scale_mode=gpu_lib.NV4_SCALE_SEGMENT,
                               nseg=cfg.E)
    _assert_exact(t, Q.quantize_cols_batched(x, cfg.E))


@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_rows_and_columns_in_one_pass(gpu_lib, xdtype):
    """NV4_ROWS_AND_COLS: the column (token-direction, per segment) and the row
    quantisation of one tensor from a single read, one tensor scale: both equal the
    oracle's separate quantisations bit for bit (ragged segments, an empty one,
    columns not a multiple of the tile width)."""
    cfg = synth.CONFIGS["tiny"]
    C = 192
    x = synth.activations(cfg.R, C, 21)
    counts = np.bincount(synth.rng(22).integers(0, cfg.E, cfg.R), minlength=cfg.E)
    counts[5] = 0
    counts[0] += cfg.R - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)])
    po = Q.padded_offsets(off)
    xd = dev_bf16(x) if xdtype == "bf16" else dev_f32(x)
    t = gpu_lib.nvfp4_quantize(xd, layout=gpu_lib.NV4_ROWS_AND_COLS, nseg=cfg.E, seg_offsets=dev_i32(off),
                               seg_padded_offsets=dev_i32(po))
    ref_c, _ = Q.quantize_cols(x, off)
    Kp = int(po[-1])
    assert np.array_equal(host(t.codes)[:, : Kp // 2], ref_c.packed())
    assert np.array_equal(host(t.scales)[:, : Kp // 16], ref_c.scales)
    assert host(t.tscale)[0] == ref_c.G[0]
    _assert_exact(t.rows_out, Q.quantize_rows(x))


def test_rows_and_columns_with_row_gather(gpu_lib):
    """The fused gather (row_index) with the rows-and-columns layout: the row output
    is the quantisation of the gathered rows, the column output that of their
    transpose per segment."""
    T, C, R = 300, 128, 900
    x = synth.activations(T, C, 23)
    idx = synth.rng(24).integers(0, T, R).astype(np.int32)
    idx[:T] = np.arange(T)  # every row appears, so the gathered amax is the tensor's
    off = np.array([0, 400, 400, 900])
    po = Q.padded_offsets(off)
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), layout=gpu_lib.NV4_ROWS_AND_COLS, nseg=3, seg_offsets=dev_i32(off),
                               seg_padded_offsets=dev_i32(po), row_index=dev_i32(idx))
    xg = x[idx]
    ref_c, _ = Q.quantize_cols(xg, off)
    Kp = int(po[-1])
    assert np.array_equal(host(t.codes)[:, : Kp // 2], ref_c.packed())
    _assert_exact(t.rows_out, Q.quantize_rows(xg))


@pytest.mark.parametrize("C", [64, 320, 2048])
def test_columns_with_row_gather(gpu_lib, C):
    """NV4_COLS with the fused gather (X in expert order for the weight gradient): the
    column output is the per-segment transposed quantisation of the gathered rows,
    with several column tiles (taken column tile by column tile) and ragged, empty
    and padded segments; the tensor scale is X's (amax_in)."""
    T, R = 300, 900
    x = synth.activations(T, C, 25)
    idx = synth.rng(26).integers(0, T, R).astype(np.int32)
    off = np.array([0, 17, 17, 400, 899, 900])
    po = Q.padded_offsets(off)
    amax = torch.tensor([np.abs(x).max()], dtype=torch.float32, device="cuda")
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), layout=gpu_lib.NV4_COLS, nseg=len(off) - 1, seg_offsets=dev_i32(off),
                               seg_padded_offsets=dev_i32(po), row_index=dev_i32(idx), amax_in=amax)
    xg = x[idx]
    ref_c, _ = Q.quantize_cols(xg, off, amax=float(np.abs(x).max()))
    Kp = int(po[-1])
    assert np.array_equal(host(t.codes)[:, : Kp // 2], ref_c.packed())
    assert np.array_equal(host(t.scales)[:, : Kp // 16], ref_c.scales)


# ---------------------------------------------------------------- rounding edge cases
# The bytes are decided by two round-to-nearest-even steps ("The 4-bitter Lesson",
# section "Improving Gradient Stability", footnote 6: clip(round(w/s))): the E4M3
# block scale and the E2M1 element.  Random data almost never lands on a tie, so
# these inputs are built to: the GPU must give the oracle's bytes on every one.

def _tie_tensor() -> np.ndarray:
    """Rows of 16-element blocks under one tensor scale S = 1 (the amax is 2688 = 6 *
    448): every E4M3 midpoint as a block scale t_b (block max 6 m, exact in FP32 and
    BF16), blocks with power-of-two scales 2^j holding every E2M1 midpoint times 2^j
    (exact ties of v), values just above 6 (saturation), signed zeros and negative
    values that round to zero."""
    e4 = F.e4m3_finite_nonneg().astype(np.float64)                 # 127 values, 0 .. 448
    mids = (e4[:-1] + e4[1:]) / 2
    blocks = [[2688.0, 1344.0, -448.0, 0.0] + [0.0] * 12]
    r = np.random.default_rng(3)
    for m in mids:                                                 # t_b = m exactly: E4M3 ties
        a = 6 * m
        blocks.append([a, -a] + list(a * r.choice([0.5, 0.25, 0.75, 1 / 3, 0.9, 0.1, 1.0], 14)))
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for j in range(-9, 9):                                         # sf = 2^j exactly: E2M1 ties
        s = 2.0 ** j
        blocks.append(list(np.concatenate([[6.0], ties, [-6.0], -ties]) * s))
        blocks.append(list(np.array([6.25, 6.125, -6.25, 5.5, 4.5, 0.0, -0.0, 1e-3, -1e-3] + [0.5] * 7) * s))
    blocks.append([-0.0] * 8 + [0.0] * 8)                           # a zero block: sf 0, signs kept
    blocks.append([-0.0, 0.0] + [-1e-30] * 7 + [1e-30] * 7)        # sf 0 (t_b below half the smallest subnormal)
    x = np.array(blocks, np.float64).astype(np.float32)
    nb = len(blocks)
    per_row = 8
    pad = (-nb) % per_row
    x = np.vstack([x, np.zeros((pad, 16), np.float32)])
    # BF16 values throughout (the tie values have at most 7 significant bits and stay exact)
    xb = synth.to_bf16_values(x)
    assert np.array_equal(xb[1:127, 0], x[1:127, 0]) and np.array_equal(xb[127:163:2], x[127:163:2])
    return xb.reshape(-1, per_row * 16)


@pytest.mark.parametrize("xdtype", ["f32", "bf16"])
def test_rounding_ties_exact(gpu_lib, xdtype):
    x = _tie_tensor()
    ref = Q.quantize_rows(x)
    assert ref.G[0] == 1.0
    xd = dev_f32(x) if xdtype == "f32" else dev_bf16(x)
    t = gpu_lib.nvfp4_quantize(xd)
    _assert_exact(t, ref)
    # the cases are really there: every E4M3 tie went to the even code, E2M1 ties too
    sc = ref.scales.reshape(-1)
    assert (sc[1:127] % 2 == 0).all()
    assert ((ref.codes.reshape(-1, 16)[127] & 7)[1:8] == [0, 2, 2, 4, 4, 6, 6]).all()


def test_every_bf16_amax_per_row_exact(gpu_lib):
    """NV4_SCALE_ROW over every positive finite BF16 magnitude A as its row's amax
    (32639 rows): the GPU matches the oracle byte for byte, and where 2688/A is finite
    the block holding A has scale 448 (0x7E) and code 6 (0x7)."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    A = F.bf16_bits_to_f32(bits.astype(np.uint16))
    x = np.zeros((len(A), 32), np.float32)
    x[:, 0] = A
    x[:, 1] = -A
    x[:, 5] = F.bf16_bits_to_f32(F.f32_to_bf16_bits(F.f32(A / np.float32(3))))
    x[:, 20] = F.bf16_bits_to_f32(F.f32_to_bf16_bits(F.f32(A * np.float32(0.75))))
    ref = Q.quantize_rows(x, "row")
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), scale_mode=gpu_lib.NV4_SCALE_ROW)
    _assert_exact(t, ref)
    finite = np.float64(2688.0) / A.astype(np.float64) < np.finfo(np.float32).max
    sc = host(t.scales)
    assert (sc[finite, 0] == 0x7E).all() and ((host(t.codes)[finite, 0] & 0xF) == 7).all()


def test_columns_with_segment_scales_exact(gpu_lib):
    """NV4_COLS with one scale per segment (the per-block scale-group branch of the
    column kernel): ragged segments, one with an amax 40x the others, an empty one,
    a one-row one, columns not a multiple of the tile."""
    x = synth.activations(300, 96, 41)
    off = np.array([0, 70, 70, 71, 200, 300])
    x[71:200] *= 40.0
    x = synth.to_bf16_values(x)
    po = Q.padded_offsets(off)
    t = gpu_lib.nvfp4_quantize(dev_bf16(x), layout=gpu_lib.NV4_COLS, scale_mode=gpu_lib.NV4_SCALE_SEGMENT,
                               nseg=5, seg_offsets=dev_i32(off), seg_padded_offsets=dev_i32(po))
    ref, _ = Q.quantize_cols(x, off, "segment")
    Kp = int(po[-1])
    assert np.array_equal(host(t.codes)[:, : Kp // 2], ref.packed())
    assert np.array_equal(host(t.scales)[:, : Kp // 16], ref.scales)
    assert np.array_equal(host(t.tscale).view(np.uint32), ref.G.view(np.uint32))
    assert len(set(ref.G.tolist())) >= 3


@pytest.mark.parametrize("K,f32", [(4096, False), (4608, False), (784, True), (8192 + 16, True), (2048, False),
                                   (1040, True), (16, False)])
def test_rows_per_token_long_and_fp32_rows(gpu_lib, K, f32):
    """NV4_SCALE_ROW with rows held in registers (K <= 4096) and rows read twice
    (longer), BF16 and FP32 input: bit-exact, per-row amaxes exact."""
    x = synth.activations(37, K, 90 + K)
    amax = torch.empty(37, dtype=torch.float32, device="cuda")
    t = gpu_lib.nvfp4_quantize(dev_f32(x) if f32 else dev_bf16(x), scale_mode=gpu_lib.NV4_SCALE_ROW, amax_out=amax)
    _assert_exact(t, Q.quantize_rows(x, "row"))
    assert np.array_equal(host(amax), np.abs(x).max(axis=1))


def test_amax_of_recorded_row_amaxes(gpu_lib):
    """nv4_amax: the tensor amax from the per-row amaxes equals max |x| over the tensor,
    so the per-tensor column quantisation of a per-token-scaled tensor needs no extra
    pass; a NaN sets the status bit; n = 0 gives 0."""
    x = synth.activations(3001, 64, 95)
    rows = torch.empty(3001, dtype=torch.float32, device="cuda")
    gpu_lib.nvfp4_quantize(dev_bf16(x), scale_mode=gpu_lib.NV4_SCALE_ROW, amax_out=rows)
    A = gpu_lib.nv4_amax(rows)
    assert host(A)[0] == np.abs(x).max()
    z = gpu_lib.nv4_amax(torch.empty(0, dtype=torch.float32, device="cuda"))
    assert host(z)[0] == 0.0
    bad = torch.ones(100, dtype=torch.float32, device="cuda")
    bad[17] = float("nan")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.nv4_amax(bad, dev_status=st)
    assert int(st.item()) & gpu_lib.NV4_DS_NONFINITE
