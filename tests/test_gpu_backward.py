"""The expert layer's backward on the GPU (re-quantised transposes, two data-gradient
and two weight-gradient grouped GEMMs), checked stage by stage against the oracle:
every quantisation bit-exact, every GEMM within 1e-5 relative Frobenius error of
the oracle's FP64 product of the GPU's own (dequantised) operands, BF16 outputs
equal to the RNE of the FP32 outputs, and bitwise repeatability."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from oracle import nvfp4 as Q
from oracle import pipeline as P
from tests.gpu_util import bf16_rne_of, dev_bf16, dev_f32, host, nvfp4_host, rel_frob

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _layer(gpu_lib, cfg, dgrad_dtype=torch.float32, dual=True):
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    wt = gpu_lib.quantize_expert_weights_t(W13, W2)
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    f = gpu_lib.moe_forward(x, lg, w, cfg.k)
    dY2, dY13 = dev_bf16(d["dY2"]), dev_bf16(d["dY13"])
    bufs = gpu_lib.alloc_backward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, dgrad_dtype=dgrad_dtype)
    b = gpu_lib.moe_backward(x, f, wt, dY2, dY13, bufs, dual=dual)
    torch.cuda.synchronize()
    return d, (x, dY2, dY13), f, wt, b


def _exact_rows(t, ref):
    assert np.array_equal(host(t.codes), ref.packed())
    assert np.array_equal(host(t.scales), ref.scales)
    assert np.array_equal(host(t.tscale)[: len(ref.G)], ref.G)


def _exact_cols(t, ref):
    Kp = ref.codes.shape[1]
    assert np.array_equal(host(t.codes)[:, : Kp // 2], ref.packed())
    assert np.array_equal(host(t.scales)[:, : Kp // 16], ref.scales)
    assert host(t.tscale)[0] == ref.G[0]


@pytest.mark.parametrize("dual", [True, False])
def test_tiny_backward_stagewise(gpu_lib, dual):
    cfg = synth.CONFIGS["tiny"]
    E, H, I = cfg.E, cfg.H, cfg.I
    d, _, f, wt, b = _layer(gpu_lib, cfg, dual=dual)
    rt = f.routing
    off = host(rt.offsets)
    # S8: upstream gradients quantised along their rows (the dgrad contraction)
    _exact_rows(b.dy2q, Q.quantize_rows(d["dY2"]))
    _exact_rows(b.dy13q, Q.quantize_rows(d["dY13"]))
    assert host(b.dy2_amax)[0] == np.abs(d["dY2"]).max()
    # S8: expert weights transposed and quantised along the new K, one scale per expert
    # (W13^T carries the gate scale on K [0, I) and the up scale on [I, 2I))
    w2t_ref, w13t_ref = P.quantize_expert_weights_t(d["W13"], d["W2"])
    _exact_rows(wt.w2t, w2t_ref)
    _exact_rows(wt.w13t, w13t_ref)
    assert wt.w13t.scale_mode == gpu_lib.NV4_SCALE_SEGMENT_HALVES and len(w13t_ref.G) == 2 * E
    # S9: data gradients on the GPU's own operands
    dh_ref = moe.grouped_gemm_m(nvfp4_host(b.dy2q).dequant(), nvfp4_host(wt.w2t).dequant(), off, E, I)
    assert rel_frob(host(b.dhact), dh_ref) <= TOL
    dx_ref = moe.grouped_gemm_m(nvfp4_host(b.dy13q).dequant(), nvfp4_host(wt.w13t).dequant(), off, E, H)
    assert rel_frob(host(b.dxperm), dx_ref) <= TOL
    # S8: column (token-direction) quantisation per expert segment, zero-padded to 16
    dy2c, po = Q.quantize_cols(d["dY2"], off)
    assert np.array_equal(host(rt.padded_offsets), po)
    _exact_cols(b.dy2c, dy2c)
    hc, _ = Q.quantize_cols(host(f.hact), off)
    _exact_cols(b.hc, hc)
    dy13c, _ = Q.quantize_cols(d["dY13"], off)
    _exact_cols(b.dy13c, dy13c)
    xc, _ = Q.quantize_cols(d["X"][host(rt.row_token)], off)   # X rows in expert order
    _exact_cols(b.xc, xc)
    # S10: weight gradients, contraction over each expert's own tokens
    Kp = int(po[-1])
    dq = lambda t: nvfp4_host(t).dequant()[:, :Kp]
    dw2_ref = moe.grouped_gemm_k(dq(b.dy2c), dq(b.hc), po, E)
    assert rel_frob(host(b.dw2), dw2_ref) <= TOL
    dw13_ref = moe.grouped_gemm_k(dq(b.dy13c), dq(b.xc), po, E)
    assert rel_frob(host(b.dw13), dw13_ref) <= TOL


@pytest.mark.parametrize("cfg_name", ["tiny", "qwen3_bwd"])
def test_forward_makes_the_swiglu_columns(gpu_lib, cfg_name):
    """A forward that also produces the SwiGLU output's column form (one read of
    Hact for its row and its column quantisation): the rows are the separate pass's
    bytes, the columns are the oracle's segment-column quantisation of the GPU's own
    Hact with the tensor scale of its amax (all of them at tiny size, sampled output
    rows at 16384 tokens), and the backward that takes them gives the same weight
    gradient as one that quantises Hact itself."""
    cfg = synth.CONFIGS[cfg_name]
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    wt = gpu_lib.quantize_expert_weights_t(W13, W2)
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    f1 = gpu_lib.moe_forward(x, lg, w, cfg.k)
    fb = gpu_lib.alloc_forward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, hact_cols=True)
    f2 = gpu_lib.moe_forward(x, lg, w, cfg.k, fb)
    torch.cuda.synchronize()
    for a, b in ((f1.hq.codes, f2.hq.codes), (f1.hq.scales, f2.hq.scales), (f1.hq.tscale, f2.hq.tscale),
                 (f1.out, f2.out)):
        assert torch.equal(a, b)
    off = host(f2.routing.offsets).astype(np.int64)
    po = host(f2.routing.padded_offsets).astype(np.int64)
    A = float(host(f2.hamax)[0])
    if cfg_name == "tiny":
        ref, _ = Q.quantize_cols(host(f2.hact), off, amax=A)
        _exact_cols(f2.hc, ref)
    else:
        r = synth.rng(11)
        cols = np.sort(r.choice(cfg.I, 24, replace=False))
        hcols = host(f2.hact[:, torch.as_tensor(cols, device=f2.hact.device)])
        ref, _ = Q.quantize_cols(hcols, off, amax=A)
        c, sc = _codes(f2.hc, cols, 0, int(po[-1]))
        assert np.array_equal(c, ref.packed()) and np.array_equal(sc, ref.scales)
        assert host(f2.hc.tscale)[0] == ref.G[0]
    dY2, dY13 = dev_bf16(d["dY2"]), dev_bf16(d["dY13"])
    b1 = gpu_lib.moe_backward(x, f1, wt, dY2, dY13)
    b2 = gpu_lib.moe_backward(x, f2, wt, dY2, dY13)
    torch.cuda.synchronize()
    assert torch.equal(b1.dw2, b2.dw2) and torch.equal(b1.dw13, b2.dw13)


def test_backward_bf16_dgrad_is_rne_of_f32(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    _, _, _, _, b32 = _layer(gpu_lib, cfg, torch.float32)
    _, _, _, _, b16 = _layer(gpu_lib, cfg, torch.bfloat16)
    assert np.array_equal(host(b16.dhact), bf16_rne_of(host(b32.dhact)))
    assert np.array_equal(host(b16.dxperm), bf16_rne_of(host(b32.dxperm)))
    assert torch.equal(b16.dw2, b32.dw2) and torch.equal(b16.dw13, b32.dw13)


def test_backward_is_bitwise_repeatable(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    _, (x, dY2, dY13), f, wt, b = _layer(gpu_lib, cfg, torch.bfloat16)
    first = [t.clone() for t in (b.dhact, b.dxperm, b.dw2, b.dw13)]
    gpu_lib.moe_backward(x, f, wt, dY2, dY13, b)
    torch.cuda.synchronize()
    for a, c in zip(first, (b.dhact, b.dxperm, b.dw2, b.dw13)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32))


def _deq(t, rows, c0, c1, G):
    """Dequantised block [rows][c0:c1] of a GPU NVFP4 tensor with one decode scale G,
    or with G = (G_lo, G_hi) the scales of the columns before and after (c0 + c1) / 2
    (sliced on the device, decoded by the oracle)."""
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=t.codes.device)
    codes = Q.unpack_codes(host(t.codes.index_select(0, idx)[:, c0 // 2:c1 // 2].contiguous()))
    sc = host(t.scales.index_select(0, idx)[:, c0 // 16:c1 // 16].contiguous())
    Gb = np.empty(sc.shape, np.float32)
    if np.ndim(G) == 0:
        Gb[:] = G
    else:
        Gb[:, : sc.shape[1] // 2], Gb[:, sc.shape[1] // 2:] = G[0], G[1]
    return Q.dequantize(codes, sc, Gb).astype(np.float64)


def _codes(t, rows, c0, c1):
    idx = torch.as_tensor(np.asarray(rows, np.int64), device=t.codes.device)
    return (host(t.codes.index_select(0, idx)[:, c0 // 2:c1 // 2].contiguous()),
            host(t.scales.index_select(0, idx)[:, c0 // 16:c1 // 16].contiguous()))


def test_learner_shaped_backward_sampled(gpu_lib):
    """Long-sequence learner batch (65536 tokens, 128 experts with 13 empty and 4 hot
    ones holding a quarter of the assignments, top-8), in the launch configuration
    the benchmark times.  Quantised operands are compared bit-exactly on sampled
    rows (row quantisation) and sampled output rows of the transposes (column
    quantisation); GEMM outputs on sampled rows (dgrad) and, for a hot, an ordinary
    and an empty expert, on sampled output rows (wgrad), each against the oracle's
    FP64 product of the GPU's own operands."""
    cfg = synth.CONFIGS["learner_64k"]
    E, H, I, R = cfg.E, cfg.H, cfg.I, cfg.R
    d, _, f, wt, b = _layer(gpu_lib, cfg, torch.float32)
    rt = f.routing
    off = host(rt.offsets).astype(np.int64)
    po = host(rt.padded_offsets).astype(np.int64)
    counts = np.diff(off)
    assert (counts == 0).sum() == 13 and np.sort(counts)[-4:].sum() == R // 4
    r = synth.rng(7)
    a_dy2, a_dy13, a_x = (np.abs(d[n]).max() for n in ("dY2", "dY13", "X"))
    G = lambda t: float(host(t.tscale)[0])
    # S8 row quantisation of the upstream gradients, sampled rows
    rows = np.sort(r.choice(R, 256, replace=False))
    e_of = np.searchsorted(off, rows, side="right") - 1
    for t, src, am in ((b.dy2q, d["dY2"], a_dy2), (b.dy13q, d["dY13"], a_dy13)):
        ref = Q.quantize_rows(src[rows], amax=am)
        c, sc = _codes(t, rows, 0, src.shape[1])
        assert np.array_equal(c, ref.packed()) and np.array_equal(sc, ref.scales)
    # S9 dgrad rows (operands decoded once per expert)
    w2tG, w13tG = host(wt.w2t.tscale), host(wt.w13t.tscale)
    dy2 = _deq(b.dy2q, rows, 0, H, G(b.dy2q))
    dy13 = _deq(b.dy13q, rows, 0, 2 * I, G(b.dy13q))
    ref2 = np.zeros((len(rows), I))
    ref13 = np.zeros((len(rows), H))
    for e in np.unique(e_of):
        m = e_of == e
        ref2[m] = dy2[m] @ _deq(wt.w2t, np.arange(e * I, (e + 1) * I), 0, H, w2tG[e]).T
        ref13[m] = dy13[m] @ _deq(wt.w13t, np.arange(e * H, (e + 1) * H), 0, 2 * I, w13tG[2 * e:2 * e + 2]).T
    idx = torch.as_tensor(rows, device=b.dhact.device)
    assert rel_frob(host(b.dhact.index_select(0, idx)), ref2) <= TOL
    assert rel_frob(host(b.dxperm.index_select(0, idx)), ref13) <= TOL
    # S8 column quantisation and S10 wgrad for a hot, an ordinary and an empty expert
    rtok = host(rt.row_token).astype(np.int64)
    hot = int(np.argmax(counts))
    plain = int(np.flatnonzero((counts > 0) & (counts < counts.max()))[0])
    empty = int(np.flatnonzero(counts == 0)[0])
    for e in (hot, plain, empty):
        a, z = int(po[e]), int(po[e + 1])
        seg = np.arange(off[e], off[e + 1])
        o2 = np.sort(r.choice(H, 32, replace=False))
        o13 = np.sort(r.choice(2 * I, 32, replace=False))
        if len(seg):
            one = np.array([0, len(seg)])
            # (the SwiGLU output's columns are pinned by the tiny stagewise test)
            for t, src, cols, am in ((b.dy2c, d["dY2"][seg], o2, a_dy2), (b.dy13c, d["dY13"][seg], o13, a_dy13),
                                     (b.xc, d["X"][rtok[seg]], o2, a_x)):
                ref, _ = Q.quantize_cols(src[:, cols], one, amax=am)
                c, sc = _codes(t, cols, a, z)
                assert np.array_equal(c, ref.packed()) and np.array_equal(sc, ref.scales)
        got2 = host(b.dw2[e])[o2]
        got13 = host(b.dw13[e])[o13]
        if e == empty:
            assert a == z and not got2.any() and not got13.any()
            continue
        ref = _deq(b.dy2c, o2, a, z, G(b.dy2c)) @ _deq(b.hc, np.arange(I), a, z, G(b.hc)).T
        assert rel_frob(got2, ref) <= TOL
        ref = _deq(b.dy13c, o13, a, z, G(b.dy13c)) @ _deq(b.xc, np.arange(H), a, z, G(b.xc)).T
        assert rel_frob(got13, ref) <= TOL
