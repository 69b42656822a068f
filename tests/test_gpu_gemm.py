"""GPU grouped NVFP4 GEMM vs the oracle on the same dequantised operands (the GPU's
own codes, scale bytes and tensor scales): FP32 outputs within 1e-5 relative
Frobenius error of the FP64 oracle; the BF16 output equals the round-to-nearest-
even of the FP32 output bit for bit; every call repeats bitwise."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from oracle import nvfp4 as Q
from tests.gpu_util import bf16_rne_of, dev_bf16, dev_f32, dev_i32, host, nvfp4_host, rel_frob

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _layer(gpu_lib, cfg, seed_shift=0):
    d = synth.layer_inputs(cfg)
    xq = gpu_lib.nvfp4_quantize(dev_bf16(d["X"]))
    w = gpu_lib.quantize_expert_weights(dev_bf16(d["W13"]), dev_bf16(d["W2"]))
    rt = gpu_lib.moe_permute(dev_f32(d["logits"]), cfg.E, cfg.k)
    return d, xq, w, rt


def _swiglu_oracle(xq_h, w13_h, rtok, off, E, I):
    A = xq_h.dequant()[rtok]
    B = w13_h.dequant()
    return moe.swiglu(moe.grouped_gemm_m(A, B, off, E, 2 * I))


@pytest.mark.parametrize("fused", [True, False])
def test_gemm1_swiglu_tiny(gpu_lib, fused):
    cfg = synth.CONFIGS["tiny"]
    d, xq, w, rt = _layer(gpu_lib, cfg)
    R = cfg.R
    amax32 = torch.zeros(1, dtype=torch.float32, device="cuda")
    if fused:
        A, a_rows = xq, rt.row_token
    else:
        A = gpu_lib.NVFP4.empty(R, cfg.H)
        gpu_lib.moe_permute(dev_f32(d["logits"]), cfg.E, cfg.k, gather_src=xq, gather_dst=A)
        A.tscale = xq.tscale
        a_rows = None
    C32 = gpu_lib.nvfp4_grouped_gemm(A, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=R, a_rows=a_rows,
                                     epilogue=gpu_lib.NV4_EPI_SWIGLU, amax_out=amax32)
    ref = _swiglu_oracle(nvfp4_host(xq), nvfp4_host(w.w13), host(rt.row_token), host(rt.offsets), cfg.E, cfg.I)
    assert rel_frob(host(C32), ref) <= TOL
    amax16 = torch.zeros(1, dtype=torch.float32, device="cuda")
    C16 = gpu_lib.nvfp4_grouped_gemm(A, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=R, a_rows=a_rows,
                                     epilogue=gpu_lib.NV4_EPI_SWIGLU, out_dtype=torch.bfloat16, amax_out=amax16)
    assert np.array_equal(host(C16), bf16_rne_of(host(C32)))
    assert host(amax16)[0] == np.abs(host(C16)).max()
    assert host(amax32)[0] == np.abs(host(C32)).max()
    C32b = gpu_lib.nvfp4_grouped_gemm(A, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=R, a_rows=a_rows,
                                      epilogue=gpu_lib.NV4_EPI_SWIGLU)
    assert torch.equal(C32.view(torch.int32), C32b.view(torch.int32))


def test_fused_gather_is_bitwise_materialized_gather(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    d, xq, w, rt = _layer(gpu_lib, cfg)
    A = gpu_lib.NVFP4.empty(cfg.R, cfg.H)
    gpu_lib.moe_permute(dev_f32(d["logits"]), cfg.E, cfg.k, gather_src=xq, gather_dst=A)
    A.tscale = xq.tscale
    c1 = gpu_lib.nvfp4_grouped_gemm(xq, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=cfg.R, a_rows=rt.row_token,
                                    epilogue=gpu_lib.NV4_EPI_SWIGLU)
    c2 = gpu_lib.nvfp4_grouped_gemm(A, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=cfg.R,
                                    epilogue=gpu_lib.NV4_EPI_SWIGLU)
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))


def test_gemm2_down_tiny(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    d, xq, w, rt = _layer(gpu_lib, cfg)
    hact = synth.activations(cfg.R, cfg.I, 77)
    hq = gpu_lib.nvfp4_quantize(dev_bf16(hact))
    Y = gpu_lib.nvfp4_grouped_gemm(hq, w.w2, rt.offsets, cfg.E, cfg.H, M_cap=cfg.R)
    ref = moe.grouped_gemm_m(nvfp4_host(hq).dequant(), nvfp4_host(w.w2).dequant(), host(rt.offsets), cfg.E, cfg.H)
    assert rel_frob(host(Y), ref) <= TOL
    Y16 = gpu_lib.nvfp4_grouped_gemm(hq, w.w2, rt.offsets, cfg.E, cfg.H, M_cap=cfg.R, out_dtype=torch.bfloat16)
    assert np.array_equal(host(Y16), bf16_rne_of(host(Y)))


def test_dense_gemm_8192x2048x768(gpu_lib):
    cfg = synth.CONFIGS["dense_gemm"]
    A, B = synth.dense_gemm_inputs(cfg)
    aq = gpu_lib.nvfp4_quantize(dev_bf16(A))
    bq = gpu_lib.nvfp4_quantize(dev_bf16(B))
    off = dev_i32(np.array([0, cfg.T]))
    C = gpu_lib.nvfp4_grouped_gemm(aq, bq, off, 1, cfg.I, M_cap=cfg.T)
    ref = nvfp4_host(aq).dequant() @ nvfp4_host(bq).dequant().T
    err = rel_frob(host(C), ref)
    print(f"dense 8192x2048x768 rel Frobenius error {err:.3e}")
    assert err <= TOL
    C2 = gpu_lib.nvfp4_grouped_gemm(aq, bq, off, 1, cfg.I, M_cap=cfg.T)
    assert torch.equal(C.view(torch.int32), C2.view(torch.int32))


@pytest.mark.parametrize("N,epi", [(200, 0), (40, 1), (64, 1), (1024, 0)])
def test_ragged_experts_and_columns(gpu_lib, N, epi):
    E, K = 7, 192
    counts = np.array([0, 1, 127, 128, 129, 300, 0])
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = synth.activations(R, K, 21)
    nb = (2 * N if epi else N)
    b = synth.weights((E * nb, K), 22)
    aq = gpu_lib.nvfp4_quantize(dev_bf16(a))
    bq = gpu_lib.nvfp4_quantize(dev_bf16(b), scale_mode=gpu_lib.NV4_SCALE_SEGMENT, nseg=E)
    C = torch.full((R, N), 12345.0, dtype=torch.float32, device="cuda")
    gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(off), E, N, M_cap=R, epilogue=epi, C=C)
    raw = moe.grouped_gemm_m(nvfp4_host(aq).dequant(), nvfp4_host(bq).dequant(), off, E, nb)
    ref = moe.swiglu(raw) if epi else raw
    assert rel_frob(host(C), ref) <= TOL
    # per-expert errors
    for e in range(E):
        if counts[e]:
            sl = slice(off[e], off[e + 1])
            assert rel_frob(host(C)[sl], ref[sl]) <= 1e-4


def test_per_token_activation_scale(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    d, _, w, rt = _layer(gpu_lib, cfg)
    xq = gpu_lib.nvfp4_quantize(dev_bf16(d["X"]), scale_mode=gpu_lib.NV4_SCALE_ROW)
    C = gpu_lib.nvfp4_grouped_gemm(xq, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=cfg.R, a_rows=rt.row_token,
                                   epilogue=gpu_lib.NV4_EPI_SWIGLU)
    ref = _swiglu_oracle(nvfp4_host(xq), nvfp4_host(w.w13), host(rt.row_token), host(rt.offsets), cfg.E, cfg.I)
    assert rel_frob(host(C), ref) <= TOL


def test_group_k_weight_gradient_tiny(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    d, _, _, rt = _layer(gpu_lib, cfg)
    off = host(rt.offsets)
    dy = synth.gradients((cfg.R, cfg.H), 31)
    hact = synth.activations(cfg.R, cfg.I, 32)
    po = rt.padded_offsets
    dyc = gpu_lib.nvfp4_quantize(dev_bf16(dy), layout=gpu_lib.NV4_COLS, nseg=cfg.E, seg_offsets=rt.offsets,
                                 seg_padded_offsets=po)
    hc = gpu_lib.nvfp4_quantize(dev_bf16(hact), layout=gpu_lib.NV4_COLS, nseg=cfg.E, seg_offsets=rt.offsets,
                                seg_padded_offsets=po, out_K=dyc.K)
    dW = gpu_lib.nvfp4_grouped_gemm(dyc, hc, po, cfg.E, 0, group_mode=gpu_lib.NV4_GROUP_K)
    ref_a, po_ref = Q.quantize_cols(dy, off)
    ref_b, _ = Q.quantize_cols(hact, off)
    ref = moe.grouped_gemm_k(ref_a.dequant(), ref_b.dequant(), po_ref, cfg.E)
    # the oracle quantised the same inputs itself; its codes equal the GPU's (checked by the quantiser tests)
    assert rel_frob(host(dW), ref) <= TOL


def test_qwen_shaped_gemm1_sampled_rows(gpu_lib):
    """Full Qwen3-30B-A3B-shaped GEMM1 (16384 tokens, 128 experts, top-8, I = 768)
    in the launch configuration the benchmark times; 384 sampled rows checked."""
    cfg = synth.CONFIGS["qwen3_fwd"]
    d, xq, w, rt = _layer(gpu_lib, cfg)
    C = gpu_lib.nvfp4_grouped_gemm(xq, w.w13, rt.offsets, cfg.E, cfg.I, M_cap=cfg.R, a_rows=rt.row_token,
                                   epilogue=gpu_lib.NV4_EPI_SWIGLU)
    off = host(rt.offsets)
    rtok = host(rt.row_token)
    rows = np.sort(synth.rng(99).choice(cfg.R, 384, replace=False))
    xh = nvfp4_host(xq)
    w13 = nvfp4_host(w.w13)
    e_of = np.searchsorted(off, rows, side="right") - 1
    A = xh.dequant()[rtok[rows]]
    got = host(C)[rows]
    ref = np.zeros_like(got, dtype=np.float64)
    for i, (r, e) in enumerate(zip(rows, e_of)):
        Be = Q.dequantize(w13.codes[e * 1536:(e + 1) * 1536], w13.scales[e * 1536:(e + 1) * 1536],
                          w13.G_block[e * 1536:(e + 1) * 1536])
        ref[i] = moe.swiglu((A[i:i + 1] @ Be.T))[0]
    err = rel_frob(got, ref)
    print(f"qwen GEMM1 sampled rows rel Frobenius error {err:.3e}")
    assert err <= TOL


def test_combine_tiny(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    lg = synth.router_logits(cfg)
    rt = gpu_lib.moe_permute(dev_f32(lg), cfg.E, cfg.k)
    Y = synth.activations(cfg.R, cfg.H, 41)
    out32 = gpu_lib.moe_combine(dev_f32(Y), rt.token_row, rt.topk_w)
    ref = moe.combine(Y, host(rt.token_row), host(rt.topk_w))
    assert rel_frob(host(out32), ref) <= TOL
    out16 = gpu_lib.moe_combine(dev_f32(Y), rt.token_row, rt.topk_w, out_dtype=torch.bfloat16)
    assert np.array_equal(host(out16), bf16_rne_of(host(out32)))
    # BF16 expert rows
    out_b = gpu_lib.moe_combine(dev_bf16(Y), rt.token_row, rt.topk_w)
    assert rel_frob(host(out_b), ref) <= TOL


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_combine_other_k(gpu_lib, k):
    """The combine for k other than 8 (k = 3 and 5 take the kernel's run-time k loop),
    H not a multiple of the workgroup's 1024 columns, FP32 and BF16 expert rows."""
    T, E, H = 200, 12, 1344
    lg = synth.rng(44 + k).standard_normal((T, E)).astype(np.float32)
    rt = gpu_lib.moe_permute(dev_f32(lg), E, k)
    Y = synth.activations(T * k, H, 45)
    ref = moe.combine(Y, host(rt.token_row), host(rt.topk_w))
    assert rel_frob(host(gpu_lib.moe_combine(dev_f32(Y), rt.token_row, rt.topk_w)), ref) <= TOL
    assert rel_frob(host(gpu_lib.moe_combine(dev_bf16(Y), rt.token_row, rt.topk_w)), ref) <= TOL


def test_combine_unpermute_exact(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    lg = synth.router_logits(cfg)
    rt = gpu_lib.moe_permute(dev_f32(lg), cfg.E, 1)
    X = synth.activations(cfg.T, cfg.H, 42)
    Y = X[host(rt.row_token)]
    ones = torch.ones((cfg.T, 1), dtype=torch.float32, device="cuda")
    out = gpu_lib.moe_combine(dev_f32(Y), rt.token_row, ones)
    assert np.array_equal(host(out), X)


def test_combine_qwen_sampled(gpu_lib):
    cfg = synth.CONFIGS["qwen3_fwd"]
    lg = synth.router_logits(cfg)
    rt = gpu_lib.moe_permute(dev_f32(lg), cfg.E, cfg.k)
    Y = synth.activations(cfg.R, cfg.H, 43)
    out = gpu_lib.moe_combine(dev_f32(Y), rt.token_row, rt.topk_w)
    toks = synth.rng(6).choice(cfg.T, 64, replace=False)
    tr = host(rt.token_row)[toks]
    w = host(rt.topk_w)[toks]
    ref = moe.combine(Y, tr, w)
    assert rel_frob(host(out)[toks], ref) <= TOL


def test_gate_and_up_scales_per_projection(gpu_lib):
    """One FP32 scale per expert projection ("The 4-bitter Lesson", "Why is the NVFP4
    pretraining recipe not sufficient for RL?": one scale per weight tensor; footnote
    5: three projections per expert), with up weights ~100x the gate weights so that
    a swapped or shared scale is off by far more than the tolerance: the SwiGLU
    epilogue applies G_gate to the gate and G_up to the up accumulators, and the data
    gradient through the transposed W13 applies G_gate to K [0, I) and G_up to
    [I, 2I) (one rescale at K = I)."""
    cfg = synth.CONFIGS["tiny"]
    E, H, I, R = cfg.E, cfg.H, cfg.I, cfg.R
    d = synth.layer_inputs(cfg)
    W13 = d["W13"].copy()
    W13[:, I:] *= 100.0
    W13 = synth.to_bf16_values(W13)
    w = gpu_lib.quantize_expert_weights(dev_bf16(W13), dev_bf16(d["W2"]))
    wt = gpu_lib.quantize_expert_weights_t(dev_bf16(W13), dev_bf16(d["W2"]))
    xq = gpu_lib.nvfp4_quantize(dev_bf16(d["X"]))
    rt = gpu_lib.moe_permute(dev_f32(d["logits"]), E, cfg.k)
    G = host(w.w13.tscale)
    assert (G[1::2] > 50 * G[0::2]).all()
    C = gpu_lib.nvfp4_grouped_gemm(xq, w.w13, rt.offsets, E, I, M_cap=R, a_rows=rt.row_token,
                                   epilogue=gpu_lib.NV4_EPI_SWIGLU)
    ref = _swiglu_oracle(nvfp4_host(xq), nvfp4_host(w.w13), host(rt.row_token), host(rt.offsets), E, I)
    assert rel_frob(host(C), ref) <= TOL
    dy13 = synth.gradients((R, 2 * I), 55)
    dyq = gpu_lib.nvfp4_quantize(dev_bf16(dy13))
    dX = gpu_lib.nvfp4_grouped_gemm(dyq, wt.w13t, rt.offsets, E, H, M_cap=R)
    ref = moe.grouped_gemm_m(nvfp4_host(dyq).dequant(), nvfp4_host(wt.w13t).dequant(), host(rt.offsets), E, H)
    err = rel_frob(host(dX), ref)
    print(f"dgrad through W13^T with per-half scales: rel Frobenius error {err:.3e}")
    assert err <= TOL
    # with one shared scale the error would be O(1): the test can see a swap
    h = nvfp4_host(wt.w13t)
    Gw = h.G_block.copy()
    Gw[:, : I // 16] = Gw[:, I // 16:]                  # the up scale on both halves
    wrong = moe.grouped_gemm_m(nvfp4_host(dyq).dequant(), Q.dequantize(h.codes, h.scales, Gw), host(rt.offsets), E, H)
    assert rel_frob(wrong, ref) > 1e-2
    dX16 = gpu_lib.nvfp4_grouped_gemm(dyq, wt.w13t, rt.offsets, E, H, M_cap=R, out_dtype=torch.bfloat16)
    assert np.array_equal(host(dX16), bf16_rne_of(host(dX)))
    dX2 = gpu_lib.nvfp4_grouped_gemm(dyq, wt.w13t, rt.offsets, E, H, M_cap=R)
    assert torch.equal(dX.view(torch.int32), dX2.view(torch.int32))


def test_per_half_scales_need_whole_stages(gpu_lib):
    """A B operand with a scale per K half is accepted only where K/2 is a whole number
    of 128-wide stages; otherwise the call fails on the host and launches nothing."""
    E, I, H = 2, 80, 128
    W13 = synth.weights((E, 2 * I, H), 57)
    wt = gpu_lib.quantize_expert_weights_t(dev_bf16(W13), dev_bf16(synth.weights((E, H, I), 58)))
    dyq = gpu_lib.nvfp4_quantize(dev_bf16(synth.gradients((64, 2 * I), 59)))
    off = dev_i32(np.array([0, 30, 64]))
    with pytest.raises(gpu_lib.NV4Error) as ei:
        gpu_lib.nvfp4_grouped_gemm(dyq, wt.w13t, off, E, H, M_cap=64)
    assert "NV4_EUNSUPPORTED" in str(ei.value) or "NV4_EALIGN" in str(ei.value)


@pytest.mark.parametrize("K", [16, 48, 80, 208])
def test_k_multiple_of_16(gpu_lib, K):
    """The format's only constraint on K is whole 16-element blocks ("The 4-bitter
    Lesson", "Baseline": blocks of 16).  K % 64 != 0 runs through the workspace copy
    zero-padded to 64: GROUP_M (with a ragged and an empty expert, the SwiGLU epilogue
    and the fused gather) and GROUP_K (ragged 16-aligned contraction ranges), each
    within 1e-5 of the oracle, bitwise repeatable."""
    E = 4
    counts = np.array([37, 0, 130, 9])
    R = int(counts.sum())
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    for epi, N in ((0, 96), (1, 64)):
        nb = 2 * N if epi else N
        a = synth.activations(R, K, 70 + K)
        b = synth.weights((E * nb, K), 71 + K)
        aq = gpu_lib.nvfp4_quantize(dev_bf16(a))
        bq = gpu_lib.nvfp4_quantize(dev_bf16(b), scale_mode=gpu_lib.NV4_SCALE_SEGMENT, nseg=E)
        perm = synth.rng(K).permutation(R).astype(np.int32)
        C = gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(off), E, N, M_cap=R, a_rows=dev_i32(perm), epilogue=epi)
        A_h = nvfp4_host(aq).dequant()[perm]
        raw = moe.grouped_gemm_m(A_h, nvfp4_host(bq).dequant(), off, E, nb)
        ref = moe.swiglu(raw) if epi else raw
        assert rel_frob(host(C), ref) <= TOL
        C2 = gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(off), E, N, M_cap=R, a_rows=dev_i32(perm), epilogue=epi)
        assert torch.equal(C.view(torch.int32), C2.view(torch.int32))
    # GROUP_K: A [N][Kcap], B [M][Kcap] with 16-aligned expert ranges inside Kcap = K
    Kc = K
    ko = np.array([0, min(16, Kc), min(16, Kc), Kc, Kc]).astype(np.int32)
    a = synth.activations(72, Kc, 80 + K)
    b = synth.activations(40, Kc, 81 + K)
    aq, bq = gpu_lib.nvfp4_quantize(dev_bf16(a)), gpu_lib.nvfp4_quantize(dev_bf16(b))
    Cg = gpu_lib.nvfp4_grouped_gemm(aq, bq, dev_i32(ko), E, 72, group_mode=gpu_lib.NV4_GROUP_K)
    ref = moe.grouped_gemm_k(nvfp4_host(aq).dequant(), nvfp4_host(bq).dequant(), ko, E)
    assert rel_frob(host(Cg), ref) <= TOL
    assert not host(Cg)[1].any() and not host(Cg)[3].any()     # empty ranges give zeros
