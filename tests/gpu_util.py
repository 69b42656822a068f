"""Helpers of the GPU parity tests: moving seeded inputs to the device and turning
the GPU's NVFP4 bytes into the oracle's representation (so each oracle stage is
fed the GPU's own stage inputs)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import nvfp4 as Q


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def nvfp4_host(t, group_of_row=None) -> Q.NVFP4:
    """GPU NVFP4 tensor -> oracle NVFP4 (codes unpacked, G per block)."""
    codes = Q.unpack_codes(host(t.codes))
    scales = host(t.scales)
    G = host(t.tscale).astype(np.float32)
    rows = codes.shape[0]
    if t.scale_mode == 3 and group_of_row is None:
        # one scale per segment and K half: block b of row r takes 2 * segment + (b >= nblk / 2)
        nblk = scales.shape[1]
        seg = np.arange(rows) // (rows // t.nseg)
        grp = 2 * seg[:, None] + (np.arange(nblk)[None, :] >= nblk // 2)
        return Q.NVFP4(codes, scales, G[: 2 * t.nseg], G[grp], np.zeros(1, np.float32))
    if group_of_row is None:
        if t.scale_mode == 0:
            group_of_row = np.zeros(rows, np.int64)
        elif t.scale_mode == 2:
            group_of_row = np.arange(rows)
        else:
            group_of_row = np.arange(rows) // (rows // t.nseg)
    G_block = np.repeat(G[group_of_row][:, None], scales.shape[1], axis=1)
    return Q.NVFP4(codes, scales, G[: t.nseg] if t.scale_mode != 2 else G, G_block, np.zeros(1, np.float32))


def rel_frob(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def bf16_rne_of(x: np.ndarray) -> np.ndarray:
    """FP32 -> BF16 values by torch's CPU cast (an independent RNE)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return bool(torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                            b.view(torch.uint8) if b.dtype != torch.uint8 else b))
