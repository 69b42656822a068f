"""Seeded synthetic inputs for the NVFP4 W4A4 expert path.

This module only draws random numbers; it contains none of the method's
arithmetic and is shared by the oracle-side and the GPU-side of every test and
of the benchmark.  Values that must be BF16 are drawn in FP32 and rounded to
BF16 by torch's CPU cast (round to nearest even); they are returned as FP32
arrays holding BF16-representable values.

Workload shapes follow the pages' setting (*The 4-bitter Lesson*, section
"Baseline: A starting recipe with stable training dynamics": Qwen3-30B-A3B at 8k
sequence length): hidden 2048, 128 experts, top-8, expert intermediate 768.
The model weights and the RL dataset the pages train on are not used; these
seeded draws stand in for them.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# Large draws are split into chunks of this many elements, chunk i drawn from the
# stream PCG64([seed, i]) (chunks fill in parallel threads; the values do not
# depend on the thread count).  Draws of at most one chunk use PCG64(seed).
CHUNK = 1 << 22


def _draw(shape, seed: int, kind: str) -> np.ndarray:
    n = int(np.prod(shape))
    if n <= CHUNK:
        g = rng(seed)
        return g.standard_normal(shape, dtype=np.float32) if kind == "normal" else g.random(shape, dtype=np.float32)
    out = np.empty(n, dtype=np.float32)

    def fill(i):
        g = np.random.Generator(np.random.PCG64([seed, i]))
        a, b = i * CHUNK, min(n, (i + 1) * CHUNK)
        if kind == "normal":
            g.standard_normal(b - a, dtype=np.float32, out=out[a:b])
        else:
            g.random(b - a, dtype=np.float32, out=out[a:b])

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range((n + CHUNK - 1) // CHUNK)))
    return out.reshape(shape)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round FP32 draws to BF16 (torch CPU cast) and return them as FP32."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int              # tokens
    H: int              # hidden size
    E: int              # experts
    k: int              # experts per token
    I: int              # expert intermediate size
    routing: str        # "softmax" | "zipf" | "exact_counts" | "dense"
    seed: int
    outliers: bool = True
    notes: str = field(default="", compare=False)

    @property
    def R(self) -> int:
        return self.T * self.k


CONFIGS = {
    "tiny": LayerConfig("tiny", T=512, H=256, E=8, k=2, I=128, routing="softmax", seed=1000,
                        notes="tiny layer: 512 tokens, hidden 256, 8 experts, top-2, intermediate 128"),
    "dense_gemm": LayerConfig("dense_gemm", T=8192, H=2048, E=1, k=1, I=768, routing="dense", seed=2000,
                              outliers=False,
                              notes="single NVFP4 GEMM M=8192 K=2048 N=768"),
    "qwen3_fwd": LayerConfig("qwen3_fwd", T=16384, H=2048, E=128, k=8, I=768, routing="zipf", seed=3000,
                             notes="Qwen3-30B-A3B-shaped layer: 16384 tokens, Zipf(1.1) expert load"),
    "qwen3_bwd": LayerConfig("qwen3_bwd", T=16384, H=2048, E=128, k=8, I=768, routing="zipf", seed=3000,
                             notes="same layer, dgrad and wgrad grouped GEMMs"),
    "learner_64k": LayerConfig("learner_64k", T=65536, H=2048, E=128, k=8, I=768, routing="exact_counts",
                               seed=5000,
                               notes="8 sequences x 8192 tokens; 10% of experts empty, top-4 take 25%"),
}

# Per-tensor seed offsets from a config's base seed.
SEED_X, SEED_OUTLIER, SEED_WGATE, SEED_WUP, SEED_WDOWN, SEED_LOGITS, SEED_DY2, SEED_DY13, \
    SEED_RANKPERM, SEED_SHUFFLE = range(1, 11)


def activations(T: int, H: int, seed: int, outlier_frac: float = 1e-3, outlier_scale: float = 20.0,
                outliers: bool = True) -> np.ndarray:
    """N(0, 1) activations; a Bernoulli(outlier_frac) mask multiplies by outlier_scale."""
    x = _draw((T, H), seed + SEED_X, "normal")
    if outliers:
        m = _draw((T, H), seed + SEED_OUTLIER, "uniform") < outlier_frac
        x[m] *= np.float32(outlier_scale)
    return to_bf16_values(x)


def weights(shape, seed: int, std: float = 0.02) -> np.ndarray:
    w = _draw(shape, seed, "normal")
    w *= np.float32(std)
    return to_bf16_values(w)


def expert_weights(cfg: LayerConfig) -> tuple[np.ndarray, np.ndarray]:
    """W13 [E, 2I, H] (rows: gate then up) and W2 [E, H, I], N(0, 0.02^2), BF16."""
    wg = weights((cfg.E, cfg.I, cfg.H), cfg.seed + SEED_WGATE)
    wu = weights((cfg.E, cfg.I, cfg.H), cfg.seed + SEED_WUP)
    w2 = weights((cfg.E, cfg.H, cfg.I), cfg.seed + SEED_WDOWN)
    return np.concatenate([wg, wu], axis=1), w2


def gradients(shape, seed: int, std: float = 1e-3) -> np.ndarray:
    return weights(shape, seed, std)


def logits_softmax(T: int, E: int, seed: int) -> np.ndarray:
    """Plain N(0, 1) router logits (FP32)."""
    return rng(seed + SEED_LOGITS).standard_normal((T, E), dtype=np.float32)


def logits_zipf(T: int, E: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Zipf-skewed routing: l[t, e] = -s * ln(rank_e) + Gumbel(0, 1), rank a seeded
    permutation of 1..E.  Top-k of these logits is an exact draw without
    replacement with probabilities proportional to rank^-s (Gumbel top-k)."""
    rank = rng(seed + SEED_RANKPERM).permutation(E).astype(np.float64) + 1.0
    g = rng(seed + SEED_LOGITS).gumbel(size=(T, E))
    return (-s * np.log(rank)[None, :] + g).astype(np.float32)


def logits_exact_counts(T: int, E: int, k: int, seed: int, empty_frac: float = 0.1,
                        hot: int = 4, hot_share: float = 0.25) -> np.ndarray:
    """Logits whose top-k reproduces a fixed expert load: round(empty_frac*E)
    experts get no tokens, `hot` experts share `hot_share` of the T*k
    assignments equally, the rest share the remainder as evenly as possible."""
    R = T * k
    n_empty = int(round(empty_frac * E))
    n_rest = E - n_empty - hot
    hot_each = int(round(hot_share * R / hot))
    rest_total = R - hot * hot_each
    counts = np.zeros(E, dtype=np.int64)
    counts[:hot] = hot_each
    counts[hot:hot + n_rest] = rest_total // n_rest
    counts[hot:hot + (rest_total % n_rest)] += 1
    if counts.max() > T:
        raise ValueError("an expert cannot receive more than T assignments")
    # slots sorted by expert; token t takes slots t + i*T, i = 0..k-1 (no duplicates since every run <= T)
    slot_expert = np.repeat(np.arange(E), counts)
    assign = slot_expert.reshape(k, T).T                      # [T, k]
    r = rng(seed + SEED_SHUFFLE)
    assign = assign[r.permutation(T)]
    eperm = rng(seed + SEED_RANKPERM).permutation(E)
    assign = eperm[assign]
    z = rng(seed + SEED_LOGITS).standard_normal((T, E))
    lg = np.minimum(z, 2.5)
    rows = np.arange(T)[:, None]
    lg[rows, assign] = 3.0 + np.abs(z[rows, assign])
    return lg.astype(np.float32)


def router_logits(cfg: LayerConfig) -> np.ndarray:
    if cfg.routing == "softmax":
        return logits_softmax(cfg.T, cfg.E, cfg.seed)
    if cfg.routing == "zipf":
        return logits_zipf(cfg.T, cfg.E, cfg.seed)
    if cfg.routing == "exact_counts":
        return logits_exact_counts(cfg.T, cfg.E, cfg.k, cfg.seed)
    if cfg.routing == "dense":
        return np.zeros((cfg.T, 1), dtype=np.float32)
    raise ValueError(cfg.routing)


def layer_inputs(cfg: LayerConfig, with_grads: bool = False) -> dict:
    """Every input of one expert layer for a config."""
    X = activations(cfg.T, cfg.H, cfg.seed, outliers=cfg.outliers)
    W13, W2 = expert_weights(cfg)
    d = dict(X=X, logits=router_logits(cfg), W13=W13, W2=W2)
    if with_grads:
        d["dY2"] = gradients((cfg.R, cfg.H), cfg.seed + SEED_DY2)
        d["dY13"] = gradients((cfg.R, 2 * cfg.I), cfg.seed + SEED_DY13)
    return d


def dense_gemm_inputs(cfg: LayerConfig = CONFIGS["dense_gemm"]) -> tuple[np.ndarray, np.ndarray]:
    """A [M, K] N(0, 1) and B [N, K] N(0, 0.02^2), both BF16."""
    A = activations(cfg.T, cfg.H, cfg.seed, outliers=False)
    B = weights((cfg.I, cfg.H), cfg.seed + SEED_WGATE)
    return A, B
