"""Stochastic rounding of NVFP4 elements on the GPU (nvfp4_quantize_sr) against the
oracle, bit for bit: codes and scale bytes of every layout (rows with each
tensor-scale grouping, segment columns with a gather, rows and columns from one
read, batched columns), the upstream-gradient quantisation of the backward with
its GEMMs, and the learner-sized gradients on sampled rows and one expert's
columns.  *The 4-bitter Lesson*, section "Why is the NVFP4 pretraining recipe not
sufficient for RL?" (stochastic rounding of gradients)."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from oracle import nvfp4 as Q
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, nvfp4_host, rel_frob

pytestmark = pytest.mark.gpu
SEED = 0x5EED1234ABCD


def _same(t, ref, ncols=None):
    c, sc = host(t.codes), host(t.scales)
    if ncols is not None:
        c, sc = c[:, : ncols // 2], sc[:, : ncols // 16]
    assert np.array_equal(sc, ref.scales)
    assert np.array_equal(c, ref.packed())


@pytest.mark.parametrize("mode,f32", [("tensor", False), ("segment", False), ("row", False), ("tensor", True)])
def test_rows_sr_exact(gpu_lib, mode, f32):
    x = synth.activations(333, 192, 8)
    m = {"tensor": gpu_lib.NV4_SCALE_TENSOR, "row": gpu_lib.NV4_SCALE_ROW, "segment": gpu_lib.NV4_SCALE_SEGMENT}[mode]
    xd = dev_f32(x) if f32 else dev_bf16(x)
    rows = 333 if mode != "segment" else 330
    xd = xd[:rows]
    q = gpu_lib.nvfp4_quantize(xd, scale_mode=m, nseg=3, sr_seed=SEED)
    _same(q, Q.quantize_rows(x[:rows], mode, nseg=3, sr_seed=SEED))
    # deterministic, seed-dependent, and one grid step from round-to-nearest at most
    again = gpu_lib.nvfp4_quantize(xd, scale_mode=m, nseg=3, sr_seed=SEED)
    other = gpu_lib.nvfp4_quantize(xd, scale_mode=m, nseg=3, sr_seed=SEED + 1)
    assert torch.equal(q.codes, again.codes) and not torch.equal(q.codes, other.codes)


def test_cols_sr_with_gather_exact(gpu_lib):
    R, C, E = 900, 128, 5
    r = synth.rng(2)
    counts = np.array([300, 0, 17, 1, 582])
    off = np.concatenate([[0], np.cumsum(counts)])
    po = Q.padded_offsets(off)
    src = synth.activations(400, C, 3)
    gidx = r.integers(0, 400, R).astype(np.int32)
    q = gpu_lib.nvfp4_quantize(dev_bf16(src), layout=gpu_lib.NV4_COLS, nseg=E, seg_offsets=dev_i32(off),
                               seg_padded_offsets=dev_i32(po), row_index=dev_i32(gidx), sr_seed=SEED)
    ref, _ = Q.quantize_cols(src[gidx], off, sr_seed=SEED)
    _same(q, ref, int(po[-1]))


@pytest.mark.parametrize("f32", [False, True])
def test_rows_and_cols_sr_exact(gpu_lib, f32):
    """One read, two outputs, two streams: the column output draws from stream 1
    and the row output from stream 0."""
    R, C, E = 700, 256, 4
    counts = np.array([123, 0, 400, 177])
    off = np.concatenate([[0], np.cumsum(counts)])
    po = Q.padded_offsets(off)
    x = synth.gradients((R, C), 77)
    xd = dev_f32(x) if f32 else dev_bf16(x)
    qc = gpu_lib.nvfp4_quantize(xd, layout=gpu_lib.NV4_ROWS_AND_COLS, nseg=E, seg_offsets=dev_i32(off),
                                seg_padded_offsets=dev_i32(po), sr_seed=SEED)
    refc, _ = Q.quantize_cols(x, off, sr_seed=SEED)
    _same(qc, refc, int(po[-1]))
    _same(qc.rows_out, Q.quantize_rows(x, sr_seed=SEED))


def test_batched_cols_sr_exact(gpu_lib):
    E, m, C = 3, 64, 96
    w = synth.weights((E * m, C), 12)
    q = gpu_lib.nvfp4_quantize(dev_bf16(w), layout=gpu_lib.NV4_COLS_BATCHED, scale_mode=gpu_lib.NV4_SCALE_SEGMENT,
                               nseg=E, sr_seed=SEED)
    _same(q, Q.quantize_cols_batched(w, E, sr_seed=SEED))


@pytest.mark.parametrize("dual", [True, False])
def test_backward_with_sr_gradients(gpu_lib, dual):
    """The NVFP4 backward with stochastically rounded upstream gradients: every
    quantised gradient operand bit for bit, the GEMMs within 1e-5 of the oracle's
    products of the GPU's operands."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    E, H, I = cfg.E, cfg.H, cfg.I
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    wt = gpu_lib.quantize_expert_weights_t(W13, W2)
    x = dev_bf16(d["X"])
    f = gpu_lib.moe_forward(x, dev_f32(d["logits"]), w, cfg.k)
    bufs = gpu_lib.alloc_backward(cfg.T, H, E, cfg.k, I, dgrad_dtype=torch.float32)
    b = gpu_lib.moe_backward(x, f, wt, dev_bf16(d["dY2"]), dev_bf16(d["dY13"]), bufs, dual=dual, sr_seed=SEED)
    torch.cuda.synchronize()
    off = host(f.routing.offsets).astype(np.int64)
    po = Q.padded_offsets(off)
    _same(b.dy2q, Q.quantize_rows(d["dY2"], sr_seed=SEED))
    _same(b.dy13q, Q.quantize_rows(d["dY13"], sr_seed=SEED + 1))
    dy2c, _ = Q.quantize_cols(d["dY2"], off, sr_seed=SEED)
    dy13c, _ = Q.quantize_cols(d["dY13"], off, sr_seed=SEED + 1)
    _same(b.dy2c, dy2c, int(po[-1]))
    _same(b.dy13c, dy13c, int(po[-1]))
    dh = moe.grouped_gemm_m(nvfp4_host(b.dy2q).dequant(), nvfp4_host(wt.w2t).dequant(), off, E, I)
    assert rel_frob(host(b.dhact), dh) <= 1e-5
    Kp = int(po[-1])
    dq = lambda t: nvfp4_host(t).dequant()[:, :Kp]
    assert rel_frob(host(b.dw2), moe.grouped_gemm_k(dq(b.dy2c), dq(b.hc), po, E)) <= 1e-5
    assert rel_frob(host(b.dw13), moe.grouped_gemm_k(dq(b.dy13c), dq(b.xc), po, E)) <= 1e-5


def test_learner_sr_gradients_sampled(gpu_lib):
    """The learner batch's upstream gradient dY2 ([524288, 2048]) quantised with
    stochastic rounding for both backward operands in one pass, as the backward
    launches it: sampled rows of the row output and the columns of one ordinary
    expert's segment (sampled output rows), bit for bit."""
    cfg = synth.CONFIGS["learner_64k"]
    R, H = cfg.R, cfg.H
    dY2 = synth.gradients((R, H), cfg.seed + synth.SEED_DY2)
    rt = gpu_lib.moe_permute(dev_f32(synth.router_logits(cfg)), cfg.E, cfg.k)
    off = host(rt.offsets).astype(np.int64)
    po = host(rt.padded_offsets).astype(np.int64)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    qc = gpu_lib.nvfp4_quantize(dev_bf16(dY2), layout=gpu_lib.NV4_ROWS_AND_COLS, nseg=cfg.E, seg_offsets=rt.offsets,
                                seg_padded_offsets=rt.padded_offsets, out_K=gpu_lib.cols_capacity(R, cfg.E),
                                amax_out=amax, sr_seed=SEED)
    torch.cuda.synchronize()
    a = float(np.abs(dY2).max())
    assert host(amax)[0] == a
    r = synth.rng(31)
    rows = np.sort(r.choice(R, 200, replace=False))
    idx = torch.as_tensor(rows, device="cuda")
    ref = Q.quantize_rows(dY2[rows], amax=a, sr_seed=SEED, sr_rows=rows)
    assert np.array_equal(host(qc.rows_out.codes.index_select(0, idx)), ref.packed())
    assert np.array_equal(host(qc.rows_out.scales.index_select(0, idx)), ref.scales)
    counts = np.diff(off)
    e = int(np.flatnonzero((counts > 0) & (counts < counts.max()))[0])
    cols = np.sort(r.choice(H, 24, replace=False))
    seg = np.arange(off[e], off[e + 1])
    refc, _ = Q.quantize_cols(dY2[seg][:, cols], np.array([0, len(seg)]), amax=a, sr_seed=SEED, sr_rows=cols,
                              sr_pos0=int(po[e]))
    cidx = torch.as_tensor(cols, device="cuda")
    got = host(qc.codes.index_select(0, cidx))[:, po[e] // 2: po[e + 1] // 2]
    assert np.array_equal(got, refc.packed())
    assert np.array_equal(host(qc.scales.index_select(0, cidx))[:, po[e] // 16: po[e + 1] // 16], refc.scales)


def test_sr_empty_and_degenerate(gpu_lib):
    """No rows; an all-zero tensor (scale 0, codes 0 whatever the uniforms);
    values on the E2M1 grid times a power-of-two scale round exactly."""
    for seed in (None, SEED):                  # an empty input reads nothing and writes G = 1
        q = gpu_lib.nvfp4_quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), sr_seed=seed)
        assert q.codes.shape == (0, 32) and host(q.tscale)[0] == 1.0
    q = gpu_lib.nvfp4_quantize(torch.zeros((40, 64), dtype=torch.bfloat16, device="cuda"), sr_seed=SEED)
    torch.cuda.synchronize()
    assert not host(q.codes).any() and not host(q.scales).any()
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 6], np.float32)
    x = np.tile(grid, (32, 4)) * np.float32(2.0 ** -3)
    q = gpu_lib.nvfp4_quantize(dev_bf16(x), sr_seed=SEED)
    ref = Q.quantize_rows(x)
    _same(q, ref)                              # on-grid values: stochastic = nearest
