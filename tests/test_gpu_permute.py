"""GPU routing and permutation vs the oracle: top-k ids, expert offsets, padded
offsets and both maps must match exactly; the routing weights within 1e-5
relative Frobenius error of the FP64 softmax; gathered FP4 rows exactly."""

import numpy as np
import pytest
import torch

import synth
from oracle import moe
from oracle import nvfp4 as Q
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, rel_frob

pytestmark = pytest.mark.gpu


def _check(rt, ids_ref, w_ref, E):
    p = moe.permute(ids_ref, E)
    assert np.array_equal(host(rt.topk_ids), ids_ref)
    if w_ref is not None:
        assert rel_frob(host(rt.topk_w), w_ref) <= 1e-5
    assert np.array_equal(host(rt.offsets), p["offsets"])
    assert np.array_equal(host(rt.padded_offsets), p["padded_offsets"])
    assert np.array_equal(host(rt.row_token), p["row_token"])
    assert np.array_equal(host(rt.token_row), p["token_row"])
    return p


@pytest.mark.parametrize("cfg_name", ["tiny", "qwen3_fwd", "learner_64k"])
def test_route_and_permute_configs(gpu_lib, cfg_name):
    cfg = synth.CONFIGS[cfg_name]
    lg = synth.router_logits(cfg)
    rt = gpu_lib.moe_permute(dev_f32(lg), cfg.E, cfg.k)
    ids, w = moe.route_topk(lg, cfg.k)
    _check(rt, ids, w, cfg.E)
    rt2 = gpu_lib.moe_permute(dev_f32(lg), cfg.E, cfg.k)
    for a, b in zip((rt.topk_ids, rt.topk_w, rt.offsets, rt.row_token, rt.token_row),
                    (rt2.topk_ids, rt2.topk_w, rt2.offsets, rt2.row_token, rt2.token_row)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (100, 1, 1), (33, 8, 8), (257, 300, 5), (64, 1024, 32), (5000, 64, 3),
                                   (77, 128, 32), (31, 65, 4), (3, 128, 8)])
def test_route_shapes(gpu_lib, T, E, k):
    lg = synth.rng(T + E + k).standard_normal((T, E)).astype(np.float32)
    lg[0, :] = 0.25  # full tie in one row: lowest ids
    rt = gpu_lib.moe_permute(dev_f32(lg), E, k)
    ids, w = moe.route_topk(lg, k)
    _check(rt, ids, w, E)
    if k == E:
        assert np.allclose(host(rt.topk_w).sum(axis=1), 1.0, rtol=1e-5)


def test_renorm_flag(gpu_lib):
    lg = synth.logits_softmax(300, 16, 3)
    rt = gpu_lib.moe_permute(dev_f32(lg), 16, 4, flags=gpu_lib.NV4_RENORM)
    ids, w = moe.route_topk(lg, 4, renorm=True)
    _check(rt, ids, w, 16)


def test_given_ids_and_empty_experts(gpu_lib):
    T, E, k = 700, 20, 3
    r = synth.rng(5)
    ids = np.stack([r.choice(E - 5, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    rt = gpu_lib.moe_permute(None, E, k, topk_ids=dev_i32(ids))
    p = _check(rt, ids, None, E)
    assert (np.diff(p["offsets"])[E - 5:] == 0).all()


def test_bad_expert_id_sets_status(gpu_lib):
    ids = np.array([[0, 1], [2, 9]], np.int32)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.moe_permute(None, 4, 2, topk_ids=dev_i32(ids), dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & gpu_lib.NV4_DS_BAD_EXPERT


def test_nan_logit_sets_status(gpu_lib):
    """A NaN router logit is out of contract: the status word says so, the token's
    selection skips the NaN (top-k of its finite logits, ties to the lower id), and
    every other token is routed exactly as without it."""
    T, E, k = 64, 16, 4
    lg = synth.rng(11).standard_normal((T, E)).astype(np.float32)
    bad = lg.copy()
    bad[5, [2, 7]] = np.nan
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    rt = gpu_lib.moe_permute(dev_f32(bad), E, k, dev_status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & gpu_lib.NV4_DS_NAN_LOGIT
    ids_ref, _ = moe.route_topk(lg, k)
    got = host(rt.topk_ids)
    keep = np.arange(T) != 5
    assert np.array_equal(got[keep], ids_ref[keep])
    finite = np.where(np.isnan(bad[5]), -np.inf, bad[5])
    assert list(got[5]) == list(np.argsort(-finite, kind="stable")[:k])


def test_gather_rows_exact(gpu_lib):
    cfg = synth.CONFIGS["tiny"]
    x = synth.activations(cfg.T, cfg.H, cfg.seed)
    xq = gpu_lib.nvfp4_quantize(dev_bf16(x))
    dst = gpu_lib.NVFP4.empty(cfg.R, cfg.H)
    lg = synth.router_logits(cfg)
    rt = gpu_lib.moe_permute(dev_f32(lg), cfg.E, cfg.k, gather_src=xq, gather_dst=dst)
    rtok = host(rt.row_token)
    assert np.array_equal(host(dst.codes), host(xq.codes)[rtok])
    assert np.array_equal(host(dst.scales), host(xq.scales)[rtok])
    # gather-then-quantise equals quantise-then-gather for the per-tensor scale
    ref = Q.quantize_rows(x[rtok])
    assert np.array_equal(host(dst.codes), ref.packed())
