"""BF16 operands and the BF16 grouped GEMM on the GPU: the unquantised layer and
the BF16 / dequantized backward (*The 4-bitter Lesson*, sections "Why is the
NVFP4 pretraining recipe not sufficient for RL?" and "Improving Gradient
Stability").

Bars: the BF16 operands (dequantised NVFP4 values, gathers, transposes, zero
padding) bit for bit against the oracle; every GEMM within 1e-5 relative
Frobenius error of the oracle's FP64 product of the same BF16 operands; BF16
outputs equal to the round-to-nearest-even of the FP32 outputs; bitwise
repeatability."""

import numpy as np
import pytest
import torch

import nvfp4_w4a4_moe_amd as nv4
import synth
from oracle import moe
from oracle import nvfp4 as Q
from oracle import pipeline
from tests.gpu_util import bf16_rne_of, dev_bf16, dev_f32, dev_i32, host, nvfp4_host, rel_frob

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _ragged_offsets(R, E, seed, empty=(1,)):
    """Ragged expert segments summing to R, with the listed experts empty."""
    r = synth.rng(seed)
    w = r.uniform(0.2, 2.0, E)
    w[list(empty)] = 0
    n = np.floor(w / w.sum() * R).astype(np.int64)
    n[np.argmax(w)] += R - n.sum()
    return np.concatenate([[0], np.cumsum(n)]).astype(np.int64)


def _bf16_vals(shape, seed, std=1.0):
    return synth.to_bf16_values(synth.rng(seed).standard_normal(shape).astype(np.float32) * std)


# ----------------------------------------------------------------------------- operands

@pytest.mark.parametrize("mode", ["tensor", "row", "segment"])
def test_dequantize_rows_exact(gpu_lib, mode):
    """nv4_to_bf16 of an NVFP4 tensor (rows) equals the oracle's BF16 dequantisation
    of the same bytes, for each tensor-scale grouping; K = 80 is not a multiple of 64."""
    x = synth.activations(300, 80, 5)
    m = {"tensor": gpu_lib.NV4_SCALE_TENSOR, "row": gpu_lib.NV4_SCALE_ROW, "segment": gpu_lib.NV4_SCALE_SEGMENT}[mode]
    q = gpu_lib.nvfp4_quantize(dev_bf16(x), scale_mode=m, nseg=3)
    ref = Q.dequantize_bf16(nvfp4_host(q))
    got = gpu_lib.nv4_to_bf16(q)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), ref)
    # and the quantiser's own bytes are the oracle's
    qr = Q.quantize_rows(x, mode, nseg=3)
    assert np.array_equal(host(q.codes), qr.packed())


def test_columns_of_bf16_and_nvfp4_with_gather_exact(gpu_lib):
    """Segment transposes (zero-padded to 16 per segment) of a BF16 tensor and of
    the dequantised NVFP4 tensor, directly and through a row gather; an empty and
    a 1-row segment included."""
    R, C, E = 1000, 96, 7
    off = _ragged_offsets(R, E, 3, empty=(2,))
    off[4] = off[3] + 1                        # a one-row segment
    off[5:] = np.maximum(off[5:], off[4])
    po = moe.transpose_segments(np.zeros((R, 1)), off)[1]
    x = _bf16_vals((R, C), 4)
    src = synth.to_bf16_values(synth.rng(5).standard_normal((333, C)).astype(np.float32))
    gidx = synth.rng(6).integers(0, 333, R).astype(np.int32)
    d_off, d_po = dev_i32(off), dev_i32(po)
    seg = dict(layout=gpu_lib.NV4_COLS, nseg=E, seg_offsets=d_off, seg_padded_offsets=d_po)
    cap = gpu_lib.cols_capacity_bf16(R, E)
    got = gpu_lib.nv4_to_bf16(dev_bf16(x), **seg)
    ref, _ = moe.transpose_segments(x, off)
    assert got.shape == (C, cap)
    assert np.array_equal(host(got)[:, :po[-1]], ref)
    got = gpu_lib.nv4_to_bf16(dev_bf16(src), row_index=dev_i32(gidx), **seg)
    assert np.array_equal(host(got)[:, :po[-1]], moe.transpose_segments(src[gidx], off)[0])
    q = gpu_lib.nvfp4_quantize(dev_bf16(src), scale_mode=gpu_lib.NV4_SCALE_ROW)
    got = gpu_lib.nv4_to_bf16(q, row_index=dev_i32(gidx), **seg)
    deq = Q.dequantize_bf16(nvfp4_host(q))
    assert np.array_equal(host(got)[:, :po[-1]], moe.transpose_segments(deq[gidx], off)[0])


def test_batched_weight_transposes_exact(gpu_lib):
    """Per-expert transposes of BF16 weights and of the dequantised NVFP4 weights
    (one scale per expert)."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg)
    E, H, I = cfg.E, cfg.H, cfg.I
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    bt = gpu_lib.bf16_expert_weights_t(W13, W2)
    assert np.array_equal(host(bt.w2t), moe.transpose_batched(d["W2"].reshape(E * H, I), E))
    assert np.array_equal(host(bt.w13t), moe.transpose_batched(d["W13"].reshape(E * 2 * I, H), E))
    w = gpu_lib.quantize_expert_weights(W13, W2)
    dt = gpu_lib.dequantize_expert_weights_t(w)
    torch.cuda.synchronize()
    assert np.array_equal(host(dt.w2t), moe.transpose_batched(Q.dequantize_bf16(nvfp4_host(w.w2)), E))
    assert np.array_equal(host(dt.w13t), moe.transpose_batched(Q.dequantize_bf16(nvfp4_host(w.w13)), E))


# ----------------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("R,K,N,E", [(1000, 256, 384, 5), (4099, 768, 2048, 9), (40, 64, 96, 3)])
def test_bf16_gemm_group_m(gpu_lib, R, K, N, E):
    """Ragged experts (one empty), several tiles and a ragged tail; FP32 and BF16 out."""
    off = _ragged_offsets(R, E, R + K)
    A = _bf16_vals((R, K), 1)
    B = _bf16_vals((E * N, K), 2, 0.05)
    dA, dB, doff = dev_bf16(A), dev_bf16(B), dev_i32(off)
    C32 = gpu_lib.bf16_grouped_gemm(dA, dB, doff, E, N)
    assert rel_frob(host(C32), moe.grouped_gemm_m(A, B, off, E, N)) <= TOL
    C16 = gpu_lib.bf16_grouped_gemm(dA, dB, doff, E, N, out_dtype=torch.bfloat16)
    assert np.array_equal(host(C16), bf16_rne_of(host(C32)))
    again = gpu_lib.bf16_grouped_gemm(dA, dB, doff, E, N)
    assert torch.equal(C32.view(torch.int32), again.view(torch.int32))


def test_bf16_gemm_swiglu_gather(gpu_lib):
    """Gate/up GEMM with the row gather and the SwiGLU epilogue (FP32 and BF16 out,
    the BF16 amax of the stored values)."""
    T, H, I, E, k = 700, 256, 192, 6, 2
    R = T * k
    off = _ragged_offsets(R, E, 9)
    X = _bf16_vals((T, H), 3)
    rtok = synth.rng(4).integers(0, T, R).astype(np.int32)
    W13 = _bf16_vals((E * 2 * I, H), 5, 0.05)
    dX, dW, doff, drt = dev_bf16(X), dev_bf16(W13), dev_i32(off), dev_i32(rtok)
    h32 = gpu_lib.bf16_grouped_gemm(dX, dW, doff, E, I, M_cap=R, a_rows=drt, epilogue=gpu_lib.NV4_EPI_SWIGLU)
    ref = moe.swiglu(moe.grouped_gemm_m(X[rtok], W13, off, E, 2 * I))
    assert rel_frob(host(h32), ref) <= TOL
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    h16 = gpu_lib.bf16_grouped_gemm(dX, dW, doff, E, I, M_cap=R, a_rows=drt, epilogue=gpu_lib.NV4_EPI_SWIGLU,
                                    out_dtype=torch.bfloat16, amax_out=amax)
    assert np.array_equal(host(h16), bf16_rne_of(host(h32)))
    assert host(amax)[0] == np.abs(host(h16)).max()


@pytest.mark.parametrize("R,N,M,E", [(1000, 256, 128, 5), (5000, 384, 768, 9)])
def test_bf16_gemm_group_k(gpu_lib, R, N, M, E):
    """Weight-gradient form: per-expert contraction over the expert's own rows of
    column operands built by nv4_to_bf16; an empty expert gives zeros."""
    off = _ragged_offsets(R, E, R + N, empty=(0, 3))
    A = _bf16_vals((R, N), 7)
    B = _bf16_vals((R, M), 8)
    po = moe.transpose_segments(np.zeros((R, 1)), off)[1]
    d_off, d_po = dev_i32(off), dev_i32(po)
    seg = dict(layout=gpu_lib.NV4_COLS, nseg=E, seg_offsets=d_off, seg_padded_offsets=d_po)
    Ac = gpu_lib.nv4_to_bf16(dev_bf16(A), **seg)
    Bc = gpu_lib.nv4_to_bf16(dev_bf16(B), **seg)
    C = gpu_lib.bf16_grouped_gemm(Ac, Bc, d_po, E, N, group_mode=gpu_lib.NV4_GROUP_K)
    ref = moe.grouped_gemm_k(moe.transpose_segments(A, off)[0], moe.transpose_segments(B, off)[0], po, E)
    assert rel_frob(host(C), ref) <= TOL
    assert not host(C[0]).any() and not host(C[3]).any()


# ----------------------------------------------------------------------------- layer

def test_bf16_layer_forward_tiny(gpu_lib):
    """The unquantised layer: routing and permutation exact, GEMM1 + SwiGLU and
    GEMM2 within 1e-5 of the oracle on the GPU's own stage inputs, combine."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg)
    E, H, I, R = cfg.E, cfg.H, cfg.I, cfg.R
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    b = gpu_lib.moe_forward_bf16(dev_bf16(d["X"]), dev_f32(d["logits"]), W13, W2, cfg.k)
    torch.cuda.synchronize()
    rt = b.routing
    ref = pipeline.moe_forward_bf16(d["X"], d["logits"], d["W13"], d["W2"], cfg.k)
    assert np.array_equal(host(rt.row_token), ref["perm"]["row_token"])
    off = host(rt.offsets)
    h32 = gpu_lib.bf16_grouped_gemm(dev_bf16(d["X"]), W13.reshape(E * 2 * I, H), rt.offsets, E, I, M_cap=R,
                                    a_rows=rt.row_token, epilogue=gpu_lib.NV4_EPI_SWIGLU)
    assert rel_frob(host(h32), ref["Hact"]) <= TOL
    assert np.array_equal(host(b.hact), bf16_rne_of(host(h32)))
    y_ref = moe.grouped_gemm_m(host(b.hact), d["W2"].reshape(E * H, I), off, E, H)
    assert rel_frob(host(b.y), y_ref) <= TOL
    o32 = gpu_lib.moe_combine(b.y, rt.token_row, rt.topk_w)
    assert rel_frob(host(o32), moe.combine(host(b.y), host(rt.token_row), host(rt.topk_w))) <= TOL
    assert np.array_equal(host(b.out), bf16_rne_of(host(o32)))
    # end to end against the oracle's BF16 layer (same roundings; agreement up to
    # FP32-vs-FP64 accumulation moving a BF16 rounding of the SwiGLU output)
    assert rel_frob(host(b.out), ref["out"]) <= 1e-2


@pytest.mark.parametrize("recipe", ["dequantized", "bf16"])
def test_tiny_bf16_backward_stagewise(gpu_lib, recipe):
    """Backward on BF16 operands after the NVFP4 forward: the forward's NVFP4
    tensors dequantised (dequantized backward) or the BF16 tensors (baseline).
    Operands exact, the four GEMMs within 1e-5 of the oracle's gradients."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    E, H, I = cfg.E, cfg.H, cfg.I
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    x = dev_bf16(d["X"])
    f = gpu_lib.moe_forward(x, dev_f32(d["logits"]), w, cfg.k)
    if recipe == "dequantized":
        wt = gpu_lib.dequantize_expert_weights_t(w)
        x_op, h_op = f.xq, f.hq
    else:
        wt = gpu_lib.bf16_expert_weights_t(W13, W2)
        x_op, h_op = x, f.hact
    bufs = gpu_lib.alloc_backward_bf16(cfg.T, H, E, cfg.k, I, dgrad_dtype=torch.float32)
    b = gpu_lib.moe_backward_bf16(x_op, h_op, wt, dev_bf16(d["dY2"]), dev_bf16(d["dY13"]), f.routing, bufs)
    torch.cuda.synchronize()
    # the oracle's gradients from the forward's own tensors (the GPU forward is
    # bit-exact with the oracle up to the SwiGLU output, which is taken from the GPU)
    if recipe == "dequantized":
        fwd = dict(Xq=nvfp4_host(f.xq), Hq=nvfp4_host(f.hq), W13q=nvfp4_host(w.w13), W2q=nvfp4_host(w.w2))
        ops = pipeline.backward_operands_bf16(d["X"], None, d["W13"], d["W2"], fwd)
    else:
        ops = pipeline.backward_operands_bf16(d["X"], host(f.hact), d["W13"], d["W2"])
    perm = dict(offsets=host(f.routing.offsets).astype(np.int64), row_token=host(f.routing.row_token))
    g = pipeline.moe_backward_bf16(ops, d["dY2"], d["dY13"], perm)
    Kp = int(g["padded_offsets"][-1])
    assert np.array_equal(host(wt.w2t), g["W2t"]) and np.array_equal(host(wt.w13t), g["W13t"])
    for name in ("dy2c", "hc", "dy13c", "xc"):
        ref = {"dy2c": g["dY2c"], "hc": g["Hc"], "dy13c": g["dY13c"], "xc": g["Xc"]}[name]
        assert np.array_equal(host(getattr(b, name))[:, :Kp], ref), name
    for name, key in (("dhact", "dHact"), ("dxperm", "dXperm"), ("dw2", "dW2"), ("dw13", "dW13")):
        assert rel_frob(host(getattr(b, name)), g[key]) <= TOL, name


def test_bf16_backward_repeatable_and_bf16_dgrad_is_rne(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    f = gpu_lib.moe_forward(dev_bf16(d["X"]), dev_f32(d["logits"]), w, cfg.k)
    wt = gpu_lib.dequantize_expert_weights_t(w)
    dY2, dY13 = dev_bf16(d["dY2"]), dev_bf16(d["dY13"])
    b32 = gpu_lib.alloc_backward_bf16(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, dgrad_dtype=torch.float32)
    gpu_lib.moe_backward_bf16(f.xq, f.hq, wt, dY2, dY13, f.routing, b32)
    b16 = gpu_lib.moe_backward_bf16(f.xq, f.hq, wt, dY2, dY13, f.routing)
    first = [t.clone() for t in (b16.dhact, b16.dxperm, b16.dw2, b16.dw13)]
    gpu_lib.moe_backward_bf16(f.xq, f.hq, wt, dY2, dY13, f.routing, b16)
    torch.cuda.synchronize()
    assert np.array_equal(host(b16.dhact), bf16_rne_of(host(b32.dhact)))
    assert np.array_equal(host(b16.dxperm), bf16_rne_of(host(b32.dxperm)))
    for a, c in zip(first, (b16.dhact, b16.dxperm, b16.dw2, b16.dw13)):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32))


@pytest.mark.parametrize("recipe", ["bf16", "dequantized"])
def test_captured_graph_replays_match_eager_bf16(gpu_lib, recipe):
    """The BF16 layer and the dequantized-backward step captured into a HIP graph
    (as the benchmark times them): every replay, with eager work in between,
    equals the eager result bit for bit."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    dY2, dY13 = dev_bf16(d["dY2"]), dev_bf16(d["dY13"])
    bb = gpu_lib.alloc_backward_bf16(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
    if recipe == "bf16":
        fb = gpu_lib.alloc_forward_bf16(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
        wt = gpu_lib.bf16_expert_weights_t(W13, W2)

        def step():
            gpu_lib.moe_forward_bf16(x, lg, W13, W2, cfg.k, fb)
            gpu_lib.moe_backward_bf16(x, fb.hact, wt, dY2, dY13, fb.routing, bb)
    else:
        fb = gpu_lib.alloc_forward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
        w = gpu_lib.quantize_expert_weights(W13, W2)
        wt = gpu_lib.dequantize_expert_weights_t(w)

        def step():
            gpu_lib.moe_forward(x, lg, w, cfg.k, fb)
            gpu_lib.moe_backward_bf16(fb.xq, fb.hq, wt, dY2, dY13, fb.routing, bb)

    step()
    torch.cuda.synchronize()
    Kp = int(fb.routing.padded_offsets[-1])   # column operands: only the segments' range is written
    outs = lambda: [t.clone() for t in (fb.out, bb.dhact, bb.dxperm, bb.dw2, bb.dw13, bb.xc[:, :Kp], bb.hc[:, :Kp])]
    ref = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (fb.out, bb.dw2, bb.dxperm, bb.xc):
            t.fill_(7)           # eager work between replays that the replay must overwrite
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs()):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"



def _dq_rows(t, rows) -> np.ndarray:
    """The oracle's BF16 dequantisation of rows `rows` of a GPU NVFP4 tensor (bytes
    gathered on the device), with each row's own tensor scale."""
    rows = np.asarray(rows, np.int64)
    idx = torch.as_tensor(rows, device=t.codes.device)
    codes = Q.unpack_codes(host(t.codes.index_select(0, idx)))
    sc = host(t.scales.index_select(0, idx))
    G = host(t.tscale).astype(np.float32)
    if t.scale_mode == nv4.NV4_SCALE_TENSOR:
        g = np.full(len(rows), G[0], np.float32)
    elif t.scale_mode == nv4.NV4_SCALE_SEGMENT:
        g = G[rows // (t.rows // t.nseg)]
    else:
        g = G[rows]
    Gb = np.repeat(g[:, None], sc.shape[1], axis=1)
    return Q.dequantize_bf16(Q.NVFP4(codes, sc, G, Gb, np.zeros(1, np.float32)))


def test_learner_dequantized_backward_sampled(gpu_lib):
    """The long-sequence learner batch (65536 tokens, 128 experts with 13 empty and 4
    hot ones, top-8) through the NVFP4 forward and the dequantized backward, in the
    launch configuration the benchmark times.  Sampled rows of the BF16 operands
    bit for bit (transposed weights; column operands of a hot and an ordinary
    expert); sampled rows of both data gradients and sampled output rows of both
    weight gradients (a hot, an ordinary and an empty expert) against the oracle's
    FP64 products of those operands."""
    cfg = synth.CONFIGS["learner_64k"]
    E, H, I, R = cfg.E, cfg.H, cfg.I, cfg.R
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    wt = gpu_lib.dequantize_expert_weights_t(w)
    f = gpu_lib.moe_forward(dev_bf16(d["X"]), dev_f32(d["logits"]), w, cfg.k)
    bufs = gpu_lib.alloc_backward_bf16(cfg.T, H, E, cfg.k, I, dgrad_dtype=torch.float32)
    b = gpu_lib.moe_backward_bf16(f.xq, f.hq, wt, dev_bf16(d["dY2"]), dev_bf16(d["dY13"]), f.routing, bufs)
    torch.cuda.synchronize()
    rt = f.routing
    off = host(rt.offsets).astype(np.int64)
    po = host(rt.padded_offsets).astype(np.int64)
    counts = np.diff(off)
    assert (counts == 0).sum() == 13
    r = synth.rng(17)
    sel = lambda t, rows: host(t.index_select(0, torch.as_tensor(np.asarray(rows, np.int64), device=t.device)))
    hot = int(np.argmax(counts))
    plain = int(np.flatnonzero((counts > 0) & (counts < counts.max()))[0])
    empty = int(np.flatnonzero(counts == 0)[0])
    # transposed dequantised weights of sampled experts
    for e in (hot, plain):
        assert np.array_equal(sel(wt.w2t, np.arange(e * I, (e + 1) * I)), _dq_rows(w.w2, np.arange(e * H, (e + 1) * H)).T)
        assert np.array_equal(sel(wt.w13t, np.arange(e * H, (e + 1) * H)),
                              _dq_rows(w.w13, np.arange(e * 2 * I, (e + 1) * 2 * I)).T)
    # data gradients on sampled rows
    rows = np.sort(r.choice(R, 192, replace=False))
    e_of = np.searchsorted(off, rows, side="right") - 1
    dy2, dy13 = d["dY2"][rows].astype(np.float64), d["dY13"][rows].astype(np.float64)
    ref2, ref13 = np.zeros((len(rows), I)), np.zeros((len(rows), H))
    for e in np.unique(e_of):
        m = e_of == e
        ref2[m] = dy2[m] @ sel(wt.w2t, np.arange(e * I, (e + 1) * I)).astype(np.float64).T
        ref13[m] = dy13[m] @ sel(wt.w13t, np.arange(e * H, (e + 1) * H)).astype(np.float64).T
    assert rel_frob(sel(b.dhact, rows), ref2) <= TOL
    assert rel_frob(sel(b.dxperm, rows), ref13) <= TOL
    # weight gradients (and their column operands) for a hot, an ordinary and an empty expert
    rtok = host(rt.row_token).astype(np.int64)
    for e in (hot, plain, empty):
        a, z = int(po[e]), int(po[e + 1])
        seg = np.arange(off[e], off[e + 1])
        n = len(seg)
        o2 = np.sort(r.choice(H, 24, replace=False))
        o13 = np.sort(r.choice(2 * I, 24, replace=False))
        got2, got13 = host(b.dw2[e])[o2], host(b.dw13[e])[o13]
        if e == empty:
            assert a == z and not got2.any() and not got13.any()
            continue
        hc = _dq_rows(f.hq, seg)            # [n, I]: the forward's NVFP4 SwiGLU output, dequantised
        xc = _dq_rows(f.xq, rtok[seg])      # [n, H]: the forward's NVFP4 X rows in expert order
        assert np.array_equal(host(b.hc[:, a:a + n]), hc.T) and not host(b.hc[:, a + n:z]).any()
        assert np.array_equal(host(b.xc[:, a:a + n]), xc.T)
        assert np.array_equal(host(b.dy2c[:, a:a + n]), d["dY2"][seg].T)
        ref = d["dY2"][seg][:, o2].astype(np.float64).T @ hc.astype(np.float64)
        assert rel_frob(got2, ref) <= TOL
        ref = d["dY13"][seg][:, o13].astype(np.float64).T @ xc.astype(np.float64)
        assert rel_frob(got13, ref) <= TOL


def test_bf16_edge_cases_empty_inputs(gpu_lib):
    """Empty inputs: no rows to convert, every expert empty (GROUP_M writes nothing,
    GROUP_K writes zeros), and the dense single-expert case (E = 1)."""
    K, N, E = 64, 96, 4
    z = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    assert gpu_lib.nv4_to_bf16(z).shape == (0, K)
    off = dev_i32(np.zeros(E + 1, np.int64))
    cols = gpu_lib.nv4_to_bf16(z, layout=gpu_lib.NV4_COLS, nseg=E, seg_offsets=off, seg_padded_offsets=off)
    assert cols.shape[0] == K
    B = dev_bf16(_bf16_vals((E * N, K), 3))
    C = torch.full((8, N), 7.0, device="cuda")
    gpu_lib.bf16_grouped_gemm(dev_bf16(_bf16_vals((8, K), 4)), B, off, E, N, M_cap=8, C=C)
    torch.cuda.synchronize()
    assert torch.all(C == 7.0)                 # rows past offsets[E] are not written
    Ac = torch.zeros((N, 64), dtype=torch.bfloat16, device="cuda")
    Bc = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    Cw = torch.full((E, N, 32), 7.0, device="cuda")
    gpu_lib.bf16_grouped_gemm(Ac, Bc, off, E, N, group_mode=gpu_lib.NV4_GROUP_K, C=Cw)
    torch.cuda.synchronize()
    assert not Cw.any()                        # empty contraction ranges give zeros
    # one expert: a dense GEMM
    A = _bf16_vals((300, 256), 5)
    Bd = _bf16_vals((160, 256), 6, 0.05)
    Cd = gpu_lib.bf16_grouped_gemm(dev_bf16(A), dev_bf16(Bd), dev_i32(np.array([0, 300])), 1, 160)
    assert rel_frob(host(Cd), A.astype(np.float64) @ Bd.astype(np.float64).T) <= TOL


def test_learner_bf16_layer_sampled(gpu_lib):
    """The unquantised BF16 layer, forward and backward, on the learner batch in the
    launch configuration the benchmark times: sampled rows of the SwiGLU output,
    the expert outputs, the combined tokens and both data gradients, and sampled
    output rows of both weight gradients of a hot and an ordinary expert, each
    against the oracle's FP64 products of the GPU's own BF16 stage inputs."""
    cfg = synth.CONFIGS["learner_64k"]
    E, H, I, R, T, k = cfg.E, cfg.H, cfg.I, cfg.R, cfg.T, cfg.k
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2, X = d["W13"], d["W2"], d["X"]
    dW13, dW2 = dev_bf16(W13), dev_bf16(W2)
    f = gpu_lib.moe_forward_bf16(dev_bf16(X), dev_f32(d["logits"]), dW13, dW2, k)
    wt = gpu_lib.bf16_expert_weights_t(dW13, dW2)
    bufs = gpu_lib.alloc_backward_bf16(T, H, E, k, I, dgrad_dtype=torch.float32)
    b = gpu_lib.moe_backward_bf16(dev_bf16(X), f.hact, wt, dev_bf16(d["dY2"]), dev_bf16(d["dY13"]), f.routing, bufs)
    torch.cuda.synchronize()
    rt = f.routing
    off = host(rt.offsets).astype(np.int64)
    po = host(rt.padded_offsets).astype(np.int64)
    rtok = host(rt.row_token).astype(np.int64)
    counts = np.diff(off)
    r = synth.rng(41)
    sel = lambda t, rows: host(t.index_select(0, torch.as_tensor(np.asarray(rows, np.int64), device=t.device)))
    rows = np.sort(r.choice(R, 160, replace=False))
    e_of = np.searchsorted(off, rows, side="right") - 1
    h_ref = np.zeros((len(rows), I))
    y_ref = np.zeros((len(rows), H))
    dh_ref = np.zeros((len(rows), I))
    dx_ref = np.zeros((len(rows), H))
    hact_rows = sel(f.hact, rows).astype(np.float64)
    for e in np.unique(e_of):
        m = e_of == e
        c1 = X[rtok[rows[m]]].astype(np.float64) @ W13[e].astype(np.float64).T
        h_ref[m] = moe.swiglu(c1)
        y_ref[m] = hact_rows[m] @ W2[e].astype(np.float64).T
        dh_ref[m] = d["dY2"][rows[m]].astype(np.float64) @ W2[e].astype(np.float64)
        dx_ref[m] = d["dY13"][rows[m]].astype(np.float64) @ W13[e].astype(np.float64)
    assert rel_frob(hact_rows, h_ref) <= 4e-3          # BF16 storage of the SwiGLU output (2^-9 relative)
    assert rel_frob(sel(f.y, rows), y_ref) <= TOL
    assert rel_frob(sel(b.dhact, rows), dh_ref) <= TOL
    assert rel_frob(sel(b.dxperm, rows), dx_ref) <= TOL
    toks = np.sort(r.choice(T, 64, replace=False))
    tr = host(rt.token_row)[toks].astype(np.int64)
    y_tok = np.stack([sel(f.y, tr[:, j]) for j in range(k)], axis=1)           # [t, k, H]
    o_ref = np.einsum("tk,tkh->th", host(rt.topk_w)[toks].astype(np.float64), y_tok.astype(np.float64))
    assert rel_frob(sel(f.out, toks), o_ref) <= 4e-3                           # BF16 output
    hot = int(np.argmax(counts))
    plain = int(np.flatnonzero((counts > 0) & (counts < counts.max()))[0])
    for e in (hot, plain):
        seg = np.arange(off[e], off[e + 1])
        o2 = np.sort(r.choice(H, 16, replace=False))
        o13 = np.sort(r.choice(2 * I, 16, replace=False))
        he = sel(f.hact, seg).astype(np.float64)
        ref = d["dY2"][seg][:, o2].astype(np.float64).T @ he
        assert rel_frob(host(b.dw2[e])[o2], ref) <= TOL
        ref = d["dY13"][seg][:, o13].astype(np.float64).T @ X[rtok[seg]].astype(np.float64)
        assert rel_frob(host(b.dw13[e])[o13], ref) <= TOL
        assert np.array_equal(host(b.hc[:, po[e]:po[e] + len(seg)]), he.T.astype(np.float32))
