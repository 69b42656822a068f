"""GPU NVFP4 quantiser vs the oracle: codes, scale bytes and tensor-scale bits must
match exactly; repeated calls must be bitwise identical."""

import numpy as np
import pytest
import torch

import synth
from oracle import nvfp4 as Q
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
