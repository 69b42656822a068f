"""Decoded FP16 weights: nvfp4_decode_f16 against the oracle's dequantisation with the
decode scale left out (every value exact), and the grouped GEMM that reads its B
operand from them (GROUP_M: the down projection, gate/up with SwiGLU and per-projection
scales, the data gradients with per-K-half scales) against the oracle's FP64 product
of the same dequantised operands, within 1e-5 relative Frobenius error.  The BF16
output is the round-to-nearest-even of the FP32 output, calls repeat bitwise, and the
layer built on FP16 weights matches the oracle stage by stage.

Method: "The 4-bitter Lesson", section "Improving Gradient Stability" (a GEMM consumes
DQ(Q(.)) of its operands); e2m1 x e4m3 has at most 6 significant bits, so FP16 holds
the decoded weight exactly and only the FP32 tensor scale is left for the epilogue."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from oracle import nvfp4 as Q
from tests.gpu_util import bf16_rne_of, dev_bf16, dev_f32, dev_i32, host, nvfp4_host, rel_frob

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _undecoded(t) -> np.ndarray:
    """Oracle values e2m1 * e4m3 of a GPU NVFP4 tensor (decode scale 1)."""
    h = nvfp4_host(t)
    return Q.dequantize(h.codes, h.scales, np.ones_like(h.G_block))


@pytest.mark.parametrize("rows,K", [(1, 16), (37, 48), (512, 256), (3072, 2048)])
def test_decode_f16_is_exact(gpu_lib, rows, K):
    w = synth.weights((rows, K), 61 + K)
    w[0, :16] = 0.0                     # a block of zeros (scale 0)
    q = gpu_lib.nvfp4_quantize(dev_bf16(w))
    f = gpu_lib.nvfp4_decode_f16(q)
    ref = _undecoded(q)
    assert np.array_equal(host(f).astype(np.float64), ref)
    # into a wider buffer: the padding is left alone
    out = torch.full((rows, K + 8), 7.0, dtype=torch.float16, device="cuda")
    gpu_lib.nvfp4_decode_f16(q, out=out[:, :K])
    assert np.array_equal(host(out[:, :K]).astype(np.float64), ref) and bool((out[:, K:] == 7.0).all())


def _ragged(gpu_lib, E, counts, K, nb, seg):
    R = int(np.sum(counts))
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = synth.activations(R, K, 71 + K)
    b = synth.weights((E * nb, K), 72 + K)
    aq = gpu_lib.nvfp4_quantize(dev_bf16(a))
    bq = gpu_lib.nvfp4_quantize(dev_bf16(b), scale_mode=gpu_lib.NV4_SCALE_SEGMENT, nseg=seg)
    return R, off, aq, bq


@pytest.mark.parametrize("N,epi,K", [(200, 0, 192), (40, 1, 64), (64, 1, 128), (1024, 0, 256), (300, 1, 2048)])
def test_gemm_f16_weights_ragged(gpu_lib, N, epi, K):
    """Ragged experts (empty, 1 row, just under / at / over a tile), partial column
    tiles, K from one 64-wide stage up; SwiGLU with one decode scale per projection."""
    E = 7
    counts = np.array([0, 1, 255, 256, 257, 300, 0])
    nb = 2 * N if epi else N
    R, off, aq, bq = _ragged(gpu_lib, E, counts, K, nb, 2 * E if epi else E)
    gpu_lib.with_f16(bq)
    C = torch.full((R, N), 12345.0, dtype=torch.float32, device="cuda")
    gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(off), E, N, M_cap=R, epilogue=epi, C=C)
    h = nvfp4_host(bq) if not epi else nvfp4_host(bq, np.arange(E * nb) // N)
    raw = moe.grouped_gemm_m(nvfp4_host(aq).dequant(), h.dequant(), off, E, nb)
    ref = moe.swiglu(raw) if epi else raw
    assert rel_frob(host(C), ref) <= TOL
    for e in range(E):
        if counts[e]:
            sl = slice(off[e], off[e + 1])
            assert rel_frob(host(C)[sl], ref[sl]) <= 1e-4
    C16 = gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(off), E, N, M_cap=R, epilogue=epi, out_dtype=torch.bfloat16)
    assert np.array_equal(host(C16), bf16_rne_of(host(C)))
    C2 = gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(off), E, N, M_cap=R, epilogue=epi)
    assert torch.equal(C.view(torch.int32), C2.view(torch.int32))


def test_gemm_f16_weights_per_half_scales(gpu_lib):
    """The data gradient through W13^T: B's K halves carry the gate and the up scale
    of the expert (gate and up amax 100x apart)."""
    E, H, I = 4, 256, 128
    counts = np.array([100, 0, 300, 37])
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    W13 = synth.weights((E, 2 * I, H), 81)
    W13[:, I:, :] *= 100.0                       # up rows 100x the gate rows
    dy = synth.gradients((R, 2 * I), 82)
    dyq = gpu_lib.nvfp4_quantize(dev_bf16(dy))
    wt = gpu_lib.quantize_expert_weights_t(dev_bf16(W13), dev_bf16(synth.weights((E, H, I), 83)), f16=True)
    C = gpu_lib.nvfp4_grouped_gemm(dyq, wt.w13t, dev_i32(off), E, H, M_cap=R)
    ref = moe.grouped_gemm_m(nvfp4_host(dyq).dequant(), nvfp4_host(wt.w13t).dequant(), off, E, H)
    assert rel_frob(host(C), ref) <= TOL
    assert wt.w13t.f16 is not None and wt.w2t.f16 is not None


def test_layer_on_f16_weights_matches_oracle(gpu_lib):
    """Forward and backward on FP16 weights: each GEMM within 1e-5 of the oracle's
    product of the GPU's own dequantised operands."""
    cfg = synth.CONFIGS["tiny"]
    E, H, I = cfg.E, cfg.H, cfg.I
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2, f16=True)
    wt = gpu_lib.quantize_expert_weights_t(W13, W2, f16=True)
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    fb = gpu_lib.alloc_forward(cfg.T, H, E, cfg.k, I, out_dtype=torch.float32, hact_dtype=torch.float32)
    f = gpu_lib.moe_forward(x, lg, w, cfg.k, fb)
    torch.cuda.synchronize()
    rt = f.routing
    off = host(rt.offsets)
    xh = nvfp4_host(f.xq)
    w13h = nvfp4_host(w.w13, np.arange(E * 2 * I) // I)
    ref_h = moe.swiglu(moe.grouped_gemm_m(xh.dequant()[host(rt.row_token)], w13h.dequant(), off, E, 2 * I))
    assert rel_frob(host(f.hact), ref_h) <= TOL
    ref_y = moe.grouped_gemm_m(nvfp4_host(f.hq).dequant(), nvfp4_host(w.w2).dequant(), off, E, H)
    assert rel_frob(host(f.y), ref_y) <= TOL
    bufs = gpu_lib.alloc_backward(cfg.T, H, E, cfg.k, I, dgrad_dtype=torch.float32)
    b = gpu_lib.moe_backward(x, f, wt, dev_bf16(d["dY2"]), dev_bf16(d["dY13"]), bufs)
    torch.cuda.synchronize()
    ref = moe.grouped_gemm_m(nvfp4_host(b.dy2q).dequant(), nvfp4_host(wt.w2t).dequant(), off, E, I)
    assert rel_frob(host(b.dhact), ref) <= TOL
    ref = moe.grouped_gemm_m(nvfp4_host(b.dy13q).dequant(), nvfp4_host(wt.w13t).dequant(), off, E, H)
    assert rel_frob(host(b.dxperm), ref) <= TOL


def test_learner_gemm1_on_f16_weights_sampled(gpu_lib):
    """Learner-sized gate/up GEMM with SwiGLU on FP16 weights, in the launch
    configuration the benchmark times: 256 sampled rows against the oracle."""
    cfg = synth.CONFIGS["learner_64k"]
    d = synth.layer_inputs(cfg)
    xq = gpu_lib.nvfp4_quantize(dev_bf16(d["X"]))
    w = gpu_lib.quantize_expert_weights(dev_bf16(d["W13"]), dev_bf16(d["W2"]), f16=True)
    rt = gpu_lib.moe_permute(dev_f32(d["logits"]), cfg.E, cfg.k)
    C = gpu_lib.nvfp4_grouped_gemm(xq, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=cfg.R, a_rows=rt.row_token,
                                   epilogue=gpu_lib.NV4_EPI_SWIGLU)
    off, rtok = host(rt.offsets), host(rt.row_token)
    rows = np.sort(synth.rng(98).choice(cfg.R, 256, replace=False))
    e_of = np.searchsorted(off, rows, side="right") - 1
    A = nvfp4_host(xq).dequant()[rtok[rows]]
    G = host(w.w13.tscale)
    n2 = 2 * cfg.I
    idx = torch.as_tensor(rows, device=C.device)
    got = host(C.index_select(0, idx))
    ref = np.zeros_like(got, dtype=np.float64)
    for e in np.unique(e_of):
        m = e_of == e
        sl = torch.arange(e * n2, (e + 1) * n2, device=C.device)
        codes = Q.unpack_codes(host(w.w13.codes.index_select(0, sl)))
        sc = host(w.w13.scales.index_select(0, sl))
        Gb = np.repeat(np.repeat(G[2 * e:2 * e + 2], cfg.I)[:, None], sc.shape[1], axis=1)
        ref[m] = moe.swiglu(A[m] @ Q.dequantize(codes, sc, Gb).T)
    assert rel_frob(got, ref) <= TOL
