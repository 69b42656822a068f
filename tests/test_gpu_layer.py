"""The whole expert-layer forward on the GPU, checked stage by stage against the
oracle (each oracle stage fed the GPU's own stage inputs), plus bitwise
repeatability of the whole forward.  Against the oracle's own pipeline (each side
feeding itself), the SwiGLU output before re-quantisation agrees to one BF16 spacing
per element (plus a small absolute allowance for cancelling sums), and the layer
output only loosely: re-quantising the SwiGLU output can
flip FP4 rounding decisions after FP32-vs-FP64 differences."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe, pipeline
from oracle import nvfp4 as Q
from tests.gpu_util import bf16_rne_of, dev_bf16, dev_f32, host, nvfp4_host, rel_frob

pytestmark = pytest.mark.gpu
TOL = 1e-5


def bf16_ulp(x) -> np.ndarray:
    """The BF16 spacing at |x| (8 significant bits): 2^(floor(log2|x|) - 7), 0 at 0."""
    m, e = np.frexp(np.abs(np.asarray(x, np.float64)))  # |x| = m 2^e, m in [0.5, 1)
    return np.where(m > 0, np.ldexp(1.0, e - 8), 0.0)


@pytest.mark.parametrize("fuse_gather", [True, False])
def test_tiny_forward_stagewise(gpu_lib, fuse_gather):
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg)
    w = gpu_lib.quantize_expert_weights(dev_bf16(d["W13"]), dev_bf16(d["W2"]))
    x = dev_bf16(d["X"])
    lg = dev_f32(d["logits"])
    b = gpu_lib.moe_forward(x, lg, w, cfg.k, fuse_gather=fuse_gather)
    torch.cuda.synchronize()
    rt = b.routing
    # S1 quantise X: exact
    xq_ref = Q.quantize_rows(d["X"])
    assert np.array_equal(host(b.xq.codes), xq_ref.packed()) and np.array_equal(host(b.xq.scales), xq_ref.scales)
    # S0/S3 routing and permutation: exact
    ids, wts = moe.route_topk(d["logits"], cfg.k)
    p = moe.permute(ids, cfg.E)
    assert np.array_equal(host(rt.topk_ids), ids) and np.array_equal(host(rt.row_token), p["row_token"])
    assert rel_frob(host(rt.topk_w), wts) <= TOL
    # S2 weights: exact
    w13_ref, w2_ref = pipeline.quantize_expert_weights(d["W13"], d["W2"])   # one scale per projection
    assert np.array_equal(host(w.w13.codes), w13_ref.packed()) and np.array_equal(host(w.w13.tscale), w13_ref.G)
    assert np.array_equal(host(w.w2.codes), w2_ref.packed()) and np.array_equal(host(w.w2.tscale), w2_ref.G)
    assert len(w13_ref.G) == 2 * cfg.E
    # S4 GEMM1 + SwiGLU: FP32 variant vs oracle, stored BF16 == RNE(FP32 variant)
    h32 = gpu_lib.nvfp4_grouped_gemm(b.xq, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=cfg.R, a_rows=rt.row_token,
                                     epilogue=gpu_lib.NV4_EPI_SWIGLU)
    A = nvfp4_host(b.xq).dequant()[host(rt.row_token)]
    h_ref = moe.swiglu(moe.grouped_gemm_m(A, nvfp4_host(w.w13).dequant(), host(rt.offsets), cfg.E, 2 * cfg.I))
    assert rel_frob(host(h32), h_ref) <= TOL
    assert np.array_equal(host(b.hact), bf16_rne_of(host(h32)))
    assert host(b.hamax)[0] == np.abs(host(b.hact)).max()
    # S5 quantise Hact with the epilogue's amax: exact
    hq_ref = Q.quantize_rows(host(b.hact))
    assert np.array_equal(host(b.hq.codes), hq_ref.packed()) and np.array_equal(host(b.hq.scales), hq_ref.scales)
    # S6 GEMM2
    y_ref = moe.grouped_gemm_m(nvfp4_host(b.hq).dequant(), nvfp4_host(w.w2).dequant(), host(rt.offsets), cfg.E, cfg.H)
    assert rel_frob(host(b.y), y_ref) <= TOL
    # S7 combine (BF16 output == RNE of the FP32 combine of the same Y)
    o32 = gpu_lib.moe_combine(b.y, rt.token_row, rt.topk_w)
    assert rel_frob(host(o32), moe.combine(host(b.y), host(rt.token_row), host(rt.topk_w))) <= TOL
    assert np.array_equal(host(b.out), bf16_rne_of(host(o32)))
    # end to end vs the oracle pipeline (each side feeding itself)
    ref = pipeline.moe_forward(d["X"], d["logits"], d["W13"], d["W2"], cfg.k, out_bf16=True)
    # the SwiGLU output, before any re-quantisation (same NVFP4 operands on both sides):
    # the GPU's BF16 value is within one BF16 spacing of the oracle's FP64 value, plus
    # an absolute FP32-accumulation allowance of 1e-6 of the largest value (results
    # near zero come from cancelling sums)
    h64 = ref["Hact"]
    assert np.all(np.abs(host(b.hact) - h64) <= bf16_ulp(h64) + 1e-6 * np.abs(h64).max())
    e2e = rel_frob(host(b.out), ref["out"])
    print(f"tiny forward end-to-end rel Frobenius vs oracle pipeline: {e2e:.3e}")
    assert e2e < 5e-2


def test_forward_is_bitwise_repeatable(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg)
    w = gpu_lib.quantize_expert_weights(dev_bf16(d["W13"]), dev_bf16(d["W2"]))
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    o1 = gpu_lib.moe_forward(x, lg, w, cfg.k).out.clone()
    o2 = gpu_lib.moe_forward(x, lg, w, cfg.k).out.clone()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_single_expert_top1_is_dense_mlp(gpu_lib):
    """E = 1, k = 1: routing weight 1, identity permutation; the layer is a dense
    W4A4 SwiGLU MLP (oracle pins this reduction; here the GPU follows it)."""
    T, H, I = 300, 256, 128
    X = synth.activations(T, H, 50)
    W13 = synth.weights((1, 2 * I, H), 51)
    W2 = synth.weights((1, H, I), 52)
    w = gpu_lib.quantize_expert_weights(dev_bf16(W13), dev_bf16(W2))
    b = gpu_lib.moe_forward(dev_bf16(X), dev_f32(np.zeros((T, 1), np.float32)), w, 1)
    torch.cuda.synchronize()
    assert (host(b.routing.topk_w) == 1.0).all()
    assert np.array_equal(host(b.routing.row_token), np.arange(T))
    y_ref = moe.grouped_gemm_m(nvfp4_host(b.hq).dequant(), nvfp4_host(w.w2).dequant(), [0, T], 1, H)
    assert rel_frob(host(b.y), y_ref) <= TOL


def test_tiny_forward_per_token_scales(gpu_lib):
    """The per-token recipe (one FP32 scale per row of X and of the SwiGLU output):
    codes and scales bit-exact, GEMMs within 1e-5 of the oracle on the GPU's
    operands, and the backward still runs (tensor amax of X taken there)."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    bufs = gpu_lib.alloc_forward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, out_dtype=torch.float32, token_scale=True)
    b = gpu_lib.moe_forward(x, lg, w, cfg.k, bufs)
    torch.cuda.synchronize()
    rt = b.routing
    xq_ref = Q.quantize_rows(d["X"], "row")
    assert np.array_equal(host(b.xq.codes), xq_ref.packed()) and np.array_equal(host(b.xq.scales), xq_ref.scales)
    assert np.array_equal(host(b.xq.tscale), xq_ref.G)
    A = nvfp4_host(b.xq).dequant()[host(rt.row_token)]
    h_ref = moe.swiglu(moe.grouped_gemm_m(A, nvfp4_host(w.w13).dequant(), host(rt.offsets), cfg.E, 2 * cfg.I))
    h = host(b.hact)
    assert rel_frob(h, bf16_rne_of(h_ref)) <= 1e-2   # BF16 storage of the FP32 SwiGLU output
    hq_ref = Q.quantize_rows(h, "row")
    assert np.array_equal(host(b.hq.codes), hq_ref.packed()) and np.array_equal(host(b.hq.tscale), hq_ref.G)
    y_ref = moe.grouped_gemm_m(nvfp4_host(b.hq).dequant(), nvfp4_host(w.w2).dequant(), host(rt.offsets), cfg.E, cfg.H)
    assert rel_frob(host(b.y), y_ref) <= TOL
    assert rel_frob(host(b.out), moe.combine(host(b.y), host(rt.token_row), host(rt.topk_w))) <= TOL
    wt = gpu_lib.quantize_expert_weights_t(W13, W2)
    g = gpu_lib.moe_backward(x, b, wt, dev_bf16(d["dY2"]), dev_bf16(d["dY13"]))
    torch.cuda.synchronize()
    xc_ref, _ = Q.quantize_cols(d["X"][host(rt.row_token)], host(rt.offsets))
    Kp = xc_ref.codes.shape[1]
    assert np.array_equal(host(g.xc.codes)[:, : Kp // 2], xc_ref.packed())


def test_captured_graph_replays_match_eager(gpu_lib):
    """The whole forward + backward captured into a HIP graph (as the benchmark
    times it): every replay, with eager work and synchronisations in between,
    equals the eager result bit for bit."""
    cfg = synth.CONFIGS["tiny"]
    d = synth.layer_inputs(cfg, with_grads=True)
    W13, W2 = dev_bf16(d["W13"]), dev_bf16(d["W2"])
    w = gpu_lib.quantize_expert_weights(W13, W2)
    wt = gpu_lib.quantize_expert_weights_t(W13, W2)
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    dY2, dY13 = dev_bf16(d["dY2"]), dev_bf16(d["dY13"])
    fb = gpu_lib.alloc_forward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)
    bb = gpu_lib.alloc_backward(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I)

    def step():
        gpu_lib.moe_forward(x, lg, w, cfg.k, fb)
        gpu_lib.moe_backward(x, fb, wt, dY2, dY13, bb)

    step()
    torch.cuda.synchronize()
    outs = lambda: [t.clone() for t in (fb.out, fb.hq.codes, bb.dhact, bb.dxperm, bb.dw2, bb.dw13, bb.xc.codes)]
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
        for t in (fb.out, bb.dw2, bb.dxperm):
            t.fill_(7)           # eager work between replays that the replay must overwrite
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs()):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"


def test_learner_forward_sampled(gpu_lib):
    """The long-sequence learner batch's forward (65536 tokens, 128 experts, top-8,
    skewed routing) in the launch configuration the benchmark times, stage by stage
    on sampled rows, each oracle stage fed the GPU's own stage input: routing and
    permutation exact; SwiGLU rows within 1e-5 (FP32 variant of the same call); the
    quantised SwiGLU output bit-exact on sampled rows (amax of the whole stored
    tensor); down-projection rows within 1e-5; combined tokens within 1e-5 and their
    BF16 storage equal to the RNE of the FP32 combine."""
    cfg = synth.CONFIGS["learner_64k"]
    E, H, I, R, T = cfg.E, cfg.H, cfg.I, cfg.R, cfg.T
    d = synth.layer_inputs(cfg)
    w = gpu_lib.quantize_expert_weights(dev_bf16(d["W13"]), dev_bf16(d["W2"]))
    x, lg = dev_bf16(d["X"]), dev_f32(d["logits"])
    b = gpu_lib.moe_forward(x, lg, w, cfg.k)
    torch.cuda.synchronize()
    rt = b.routing
    ids, _ = moe.route_topk(d["logits"], cfg.k)
    p = moe.permute(ids, E)
    assert np.array_equal(host(rt.topk_ids), ids) and np.array_equal(host(rt.offsets), p["offsets"])
    assert np.array_equal(host(rt.row_token), p["row_token"])
    off = p["offsets"].astype(np.int64)
    r = synth.rng(17)
    rows = np.sort(r.choice(R, 192, replace=False))
    e_of = np.searchsorted(off, rows, side="right") - 1
    idx = torch.as_tensor(rows, device="cuda")
    # S1 on the sampled tokens' rows (the whole tensor is pinned at this size elsewhere)
    xq = nvfp4_host(b.xq)
    # S4: FP32 variant of GEMM1 + SwiGLU, sampled rows; the stored BF16 is its RNE
    h32 = gpu_lib.nvfp4_grouped_gemm(b.xq, w.w13, rt.offsets, E, I, M_cap=R, a_rows=rt.row_token,
                                     epilogue=gpu_lib.NV4_EPI_SWIGLU)
    w13 = nvfp4_host(w.w13)
    w2 = nvfp4_host(w.w2)
    tk = p["row_token"][rows]
    A = Q.dequantize(xq.codes[tk], xq.scales[tk], xq.G_block[tk])
    ref_h = np.zeros((len(rows), I))
    for e in np.unique(e_of):
        m = e_of == e
        sl = slice(e * 2 * I, (e + 1) * 2 * I)
        ref_h[m] = moe.swiglu(A[m] @ Q.dequantize(w13.codes[sl], w13.scales[sl], w13.G_block[sl]).T)
    got_h32 = host(h32.index_select(0, idx))
    assert rel_frob(got_h32, ref_h) <= TOL
    assert np.array_equal(host(b.hact.index_select(0, idx)), bf16_rne_of(got_h32))
    # S5: the epilogue's amax is the amax of the whole stored tensor; sampled rows exact
    hact = host(b.hact)
    assert host(b.hamax)[0] == np.abs(hact).max()
    hq_ref = Q.quantize_rows(hact[rows], amax=np.abs(hact).max())
    assert np.array_equal(host(b.hq.codes.index_select(0, idx)), hq_ref.packed())
    assert np.array_equal(host(b.hq.scales.index_select(0, idx)), hq_ref.scales)
    assert host(b.hq.tscale)[0] == hq_ref.G[0]
    del hact
    # S6: down projection on the GPU's quantised SwiGLU rows
    Hd = Q.dequantize(hq_ref.codes, hq_ref.scales, hq_ref.G_block)
    ref_y = np.zeros((len(rows), H))
    for e in np.unique(e_of):
        m = e_of == e
        sl = slice(e * H, (e + 1) * H)
        ref_y[m] = Hd[m] @ Q.dequantize(w2.codes[sl], w2.scales[sl], w2.G_block[sl]).T
    assert rel_frob(host(b.y.index_select(0, idx)), ref_y) <= TOL
    # S7: sampled tokens, from the GPU's expert rows
    toks = np.sort(r.choice(T, 96, replace=False))
    tr = host(rt.token_row)[toks]
    ysel = host(b.y.index_select(0, torch.as_tensor(tr.reshape(-1).astype(np.int64), device="cuda")))
    ref_o = moe.combine(ysel, np.arange(tr.size).reshape(tr.shape), host(rt.topk_w)[toks])
    o32 = gpu_lib.moe_combine(b.y, rt.token_row, rt.topk_w)
    got = host(o32)[toks]
    assert rel_frob(got, ref_o) <= TOL
    assert np.array_equal(host(b.out)[toks], bf16_rne_of(got))
