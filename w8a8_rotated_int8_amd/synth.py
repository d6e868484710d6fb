"""Seeded synthetic inputs for the expert-choice MoE layer (shared by the tests, the smoke check and the
benchmark; holds none of the method's arithmetic).

The shapes and distributions stand in for the activations of the Nucleus-Image MoE DiT: T = 8192 tokens is a
1024x1024 image with batched CFG, T = 2048 is 512x512 (Nucleus-Image INT8 Convrot model card, "Model size
and VRAM"); d = 2048, 64 routed experts with a fused gate/up [2I, d] and a down [d, I], I = 1536 ("MLX
Nucleus-Image" overview).  No dataset or trained weight is involved.

Recipe
  * numpy ``Generator(PCG64(seed))`` draws ``standard_normal`` in fp32, scaled in fp32, then rounded to bf16
    (nearest-even, via torch); bf16 tensors are returned as raw ``uint16`` bits on the host.
  * seed = 1000 * config + role; roles: x = 1, W (or W_gu) = 2, W_dn = 3, router logits = 4, outlier channel
    choice = 5, bias = 6.  The dense linears at large M (attention and FFN projections of the same T = 8192
    tokens) use seed base 5000.
  * Activations ~ N(0, 1) with floor(1% of d) outlier feature columns (the same for every token, chosen by the
    role-5 generator without replacement) multiplied by 20 before the bf16 rounding; the single-linear case
    uses 4 outlier columns of 512.
  * Weights ~ N(0, 0.02); router logits fp32 ~ N(0, 1); biases ~ N(0, 0.02).
  * The 29-layer stack draws on the GPU with torch's generator, seed = 4000 + 10 * layer + role, because 17.5 G
    host draws would dominate the run; each layer reuses the same x.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROLE_X, ROLE_W, ROLE_WDN, ROLE_LOGITS, ROLE_OUTLIER, ROLE_BIAS = 1, 2, 3, 4, 5, 6
DENSE_SEED_BASE = 5000
# Dense W8A8 ConvRot linears over the T = 8192 tokens of d = 2048: fused qkv [6144, 2048], FFN-down-like
# [2048, 8192] and the attention output projection [2048, 2048] (M, K, N, group).
DENSE_SHAPES = {"qkv": (8192, 2048, 6144, 256), "ffn_down": (8192, 8192, 2048, 256), "out": (8192, 2048, 2048, 64)}
OUTLIER_GAIN = 20.0
W_STD = 0.02


@dataclass(frozen=True)
class MoEShape:
    """Sizes of one routed-expert layer."""
    T: int
    d: int
    E: int
    I: int
    C: int
    g_gu: int = 256
    g_dn: int = 64


# The five benchmark configurations (index = config number).
LINEAR_CFG = dict(M=64, K=512, N=256, g=64, n_outlier=4)          # config 0: one W8A8 ConvRot linear
CONFIGS = {
    1: MoEShape(T=1024, d=2048, E=1, I=1536, C=1024),             # one SwiGLU expert, no routing
    2: MoEShape(T=2048, d=2048, E=64, I=1536, C=64),              # 512x512 batched CFG
    3: MoEShape(T=8192, d=2048, E=64, I=1536, C=256),             # 1024x1024 batched CFG
    4: MoEShape(T=8192, d=2048, E=64, I=1536, C=256),             # config 3 x 29 layers (+ W4A8 variant)
}
N_LAYERS_STACK = 29


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bits (uint16), nearest-even, through torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_columns(seed_base: int, d: int, n: int | None = None) -> np.ndarray:
    n = int(0.01 * d) if n is None else n
    return np.sort(_rng(seed_base + ROLE_OUTLIER).choice(d, size=n, replace=False))


def activations(seed_base: int, rows: int, d: int, n_outlier: int | None = None) -> np.ndarray:
    """x [rows, d] bf16 bits: N(0, 1) with outlier columns x20."""
    x = _rng(seed_base + ROLE_X).standard_normal((rows, d), dtype=np.float32)
    cols = outlier_columns(seed_base, d, n_outlier)
    x[:, cols] *= np.float32(OUTLIER_GAIN)
    return to_bf16_bits(x)


def weights(seed: int, shape) -> np.ndarray:
    """W ~ N(0, 0.02) as bf16 bits."""
    w = _rng(seed).standard_normal(shape, dtype=np.float32)
    w *= np.float32(W_STD)
    return to_bf16_bits(w)


def logits(seed_base: int, T: int, E: int) -> np.ndarray:
    return _rng(seed_base + ROLE_LOGITS).standard_normal((T, E), dtype=np.float32)


def large_gap_logits(T: int, E: int, seed: int) -> np.ndarray:
    """Router logits [T, E] whose gaps to each token's maximum are 86 to 100 nats, on a grid of 0.25 nats
    (probabilities 4.5e-38 down to 3.7e-44, mostly subnormal in fp32; distinct gaps stay tens of subnormal
    units apart, equal gaps tie exactly).  Expert 0 holds every token's maximum, 0."""
    lg = -(86.0 + 0.25 * _rng(seed).integers(0, 57, size=(T, E))).astype(np.float32)
    lg[:, 0] = 0.0
    return lg


def linear_inputs(cfg: int = 0, M=None, K=None, N=None, n_outlier=None):
    """x [M, K] and W [N, K] (bf16 bits) for the single-linear case."""
    c = dict(LINEAR_CFG)
    M = c["M"] if M is None else M
    K = c["K"] if K is None else K
    N = c["N"] if N is None else N
    n_outlier = c["n_outlier"] if n_outlier is None else n_outlier
    base = 1000 * cfg
    return activations(base, M, K, n_outlier), weights(base + ROLE_W, (N, K))


def dense_linear_inputs(M: int, K: int, N: int, with_bias: bool = False):
    """x [M, K], W [N, K] and optionally a bias [N] (bf16 bits) for a dense linear at large M."""
    base = DENSE_SEED_BASE
    x = activations(base, M, K, max(1, K // 100))
    w = weights(base + ROLE_W, (N, K))
    b = weights(base + ROLE_BIAS, (N,)) if with_bias else None
    return x, w, b


def moe_inputs(cfg: int, shape: MoEShape | None = None, seed_base: int | None = None):
    """x [T, d], logits [T, E], W_gu [E, 2I, d], W_dn [E, d, I] on the host (bf16 bits / fp32)."""
    s = CONFIGS[cfg] if shape is None else shape
    base = 1000 * cfg if seed_base is None else seed_base
    x = activations(base, s.T, s.d)
    lg = logits(base, s.T, s.E) if s.E > 1 else np.zeros((s.T, 1), np.float32)
    w_gu = weights(base + ROLE_W, (s.E, 2 * s.I, s.d))
    w_dn = weights(base + ROLE_WDN, (s.E, s.d, s.I))
    return x, lg, w_gu, w_dn


def stack_x(shape: MoEShape) -> np.ndarray:
    """The tokens every layer of the 29-layer stack takes (host bf16 bits [T, d]; seed base 4000)."""
    return activations(4000, shape.T, shape.d)


def stack_layer_device(layer: int, shape: MoEShape, device):
    """One layer of the 29-layer stack drawn on the GPU: (logits fp32, W_gu bf16, W_dn bf16) torch tensors."""
    import torch
    base = 4000 + 10 * layer
    out = []
    for role, shp, std in ((ROLE_LOGITS, (shape.T, shape.E), 1.0),
                           (ROLE_W, (shape.E, 2 * shape.I, shape.d), W_STD),
                           (ROLE_WDN, (shape.E, shape.d, shape.I), W_STD)):
        g = torch.Generator(device=device)
        g.manual_seed(base + role)
        t = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
            t = t.to(torch.bfloat16)
        out.append(t)
    return tuple(out)
