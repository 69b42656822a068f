"""moe_permute_noalloc (the routing and permutation for callers that cannot
allocate) against moe_permute with a caller workspace: the same top-k ids and
weights, offsets, padded offsets, row maps and gathered rows, bit for bit, on two
calls in a row, the second with a smaller input (the static workspace keeps the
first call's contents, which the second must not read)."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev_bf16, dev_f32

pytestmark = pytest.mark.gpu


def _routing_buffers(nv4, T, E, k):
    z = lambda *shape, dt=torch.int32: torch.full(shape, -7, dtype=dt, device="cuda")
    return nv4.Routing(z(T, k), z(T, k, dt=torch.float32), z(E + 1), z(E + 1), z(T * k), z(T, k))


def _same(a, b):
    for x, y in zip((a.topk_ids, a.topk_w, a.offsets, a.padded_offsets, a.row_token, a.token_row),
                    (b.topk_ids, b.topk_w, b.offsets, b.padded_offsets, b.row_token, b.token_row)):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


@pytest.mark.parametrize("cfgs", [("qwen3_fwd", "tiny"), ("learner_64k", "tiny")])
def test_noalloc_permute_matches_permute_twice(gpu_lib, cfgs):
    nv4 = gpu_lib
    for name in cfgs:                         # the second call is the smaller one
        cfg = synth.CONFIGS[name]
        lg = dev_f32(synth.router_logits(cfg))
        ref = nv4.moe_permute(lg, cfg.E, cfg.k)
        out = _routing_buffers(nv4, cfg.T, cfg.E, cfg.k)
        torch.cuda.synchronize()
        n_alloc = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        got = nv4.moe_permute_noalloc(lg, cfg.E, cfg.k, out)
        # the binding makes no torch allocation either (cumulative allocation count)
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == n_alloc
        torch.cuda.synchronize()
        _same(got, ref)
        counts = np.diff(got.offsets.cpu().numpy())
        assert counts.sum() == cfg.R


def test_noalloc_permute_given_ids_and_gather(gpu_lib):
    """Given top-k ids (no router) and the materialised row gather of an NVFP4
    tensor, large then small."""
    nv4 = gpu_lib
    for T, E, k, H, seed in ((4096, 64, 6, 256, 1), (300, 8, 2, 64, 2)):
        r = synth.rng(seed)
        ids = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        ids_d = torch.from_numpy(ids).cuda()
        xq = nv4.nvfp4_quantize(dev_bf16(synth.activations(T, H, seed + 10)))
        g_ref = nv4.NVFP4.empty(T * k, H)
        ref = nv4.moe_permute(None, E, k, topk_ids=ids_d, gather_src=xq, gather_dst=g_ref)
        g_got = nv4.NVFP4.empty(T * k, H)
        out = _routing_buffers(nv4, T, E, k)
        got = nv4.moe_permute_noalloc(None, E, k, out, topk_ids=ids_d, gather_src=xq, gather_dst=g_got)
        torch.cuda.synchronize()
        for x, y in ((got.offsets, ref.offsets), (got.padded_offsets, ref.padded_offsets),
                     (got.row_token, ref.row_token), (got.token_row, ref.token_row)):
            assert torch.equal(x, y)
        assert torch.equal(g_got.codes, g_ref.codes) and torch.equal(g_got.scales, g_ref.scales)
