"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays out shapes; it holds none of the optimizer's
arithmetic. Layer shapes follow the LLaMA-style linear layers the Q-GaLore pages train
(pre-training of LLaMA-60M ... 7B; AIMech curated page on Q-GaLore, application claim,
paper Section 4.1): per transformer block the q, k, v, o projections (d x d) and the MLP's
gate, up (f x d) and down (d x f), as out x in row-major weights.

Every draw comes from numpy.random.default_rng([DATA_SEED, config, layer, step, tag]) (host)
or from a torch CUDA generator seeded from the same tuple (device, for the large layer sets).
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

DATA_SEED = 0
SR_SEED = 1234

TAG_G, TAG_W, TAG_P, TAG_PNEW, TAG_M, TAG_V = 1, 2, 3, 4, 5, 6
TAG_DRIFT_A, TAG_DRIFT_B, TAG_NOISE, TAG_SKETCH = 7, 8, 9, 10

BLOCK_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


@dataclasses.dataclass(frozen=True)
class LayerShape:
    layer_id: int
    name: str
    m: int
    n: int


@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    index: int
    layers: tuple
    r: int
    sigma: float          # standard deviation of the synthetic gradient
    w_scale: float = 1e-3
    steps: int = 1
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    alpha: float = 0.25

    @property
    def weight_elems(self) -> int:
        return sum(l.m * l.n for l in self.layers)


def llama_layers(blocks: int, d: int, f: int) -> tuple:
    out = []
    for b in range(blocks):
        for idx, name in enumerate(BLOCK_NAMES):
            m, n = (f, d) if name in ("gate", "up") else (d, f) if name == "down" else (d, d)
            out.append(LayerShape(7 * b + idx, f"{name}{b}", m, n))
    return tuple(out)


CONFIGS = {
    # one 256 x 256 layer, rank 32, ten steps (exercises the INT8 moment path from t = 2)
    "single256": Config("single256", 0, (LayerShape(0, "single", 256, 256),), r=32,
                        sigma=1e-3, steps=10),
    "llama60m": Config("llama60m", 1, llama_layers(8, 512, 1376), r=128, sigma=1e-3),
    "llama1b": Config("llama1b", 2, llama_layers(24, 2048, 5461), r=512, sigma=1e-3),
    "llama7b_r1024": Config("llama7b_r1024", 3, llama_layers(32, 4096, 11008), r=1024,
                            sigma=1e-4),
    "llama7b_r128": Config("llama7b_r128", 3, llama_layers(32, 4096, 11008), r=128,
                           sigma=1e-4),
    # adaptive refresh schedule: 7B shapes, rank 128, 200 steps of drifting low-rank gradients
    "schedule7b": Config("schedule7b", 4, llama_layers(32, 4096, 11008), r=128, sigma=1e-4,
                         steps=200),
}

# Drifting-subspace workload of the schedule configuration: layer k (0 .. 223) turns its
# column space at rate rho_k = DRIFT_MAX * k / 223 radians per step.
DRIFT_MAX = 0.05
SCHEDULE_DELTA0 = 25          # initial refresh interval: 200 steps / 8
SCHEDULE_GAMMA = 0.4


def rng(cfg: Config, layer: int, step: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([DATA_SEED, cfg.index, layer, step, tag])


def torch_seed(cfg: Config, layer: int, step: int, tag: int) -> int:
    return zlib.crc32(np.array([DATA_SEED, cfg.index, layer, step, tag], np.int64).tobytes())


# ------------------------------- host (numpy) draws ------------------------------------

def gradient_f32(cfg: Config, L: LayerShape, step: int) -> np.ndarray:
    g = rng(cfg, L.layer_id, step, TAG_G).standard_normal((L.m, L.n), dtype=np.float32)
    return g * np.float32(cfg.sigma)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 with torch's CPU conversion; returns uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gradient_bf16(cfg: Config, L: LayerShape, step: int) -> np.ndarray:
    return to_bf16_bits(gradient_f32(cfg, L, step))


def weights_int8(cfg: Config, L: LayerShape) -> np.ndarray:
    return rng(cfg, L.layer_id, 0, TAG_W).integers(-127, 128, size=(L.m, L.n), dtype=np.int8)


def weight_scales(cfg: Config, L: LayerShape) -> np.ndarray:
    return np.full(-(-(L.m * L.n) // 256), cfg.w_scale, dtype=np.float32)


def orthonormal_f32(cfg: Config, L: LayerShape, r: int, tag: int = TAG_P, step: int = 0):
    a = rng(cfg, L.layer_id, step, tag).standard_normal((L.m, r))
    q, _ = np.linalg.qr(a)
    return np.ascontiguousarray(q, dtype=np.float32)


def zero_moments(r: int, n: int):
    ng = -(-(r * n) // 256)
    return (np.zeros((r, n), np.int8), np.zeros(ng, np.float32),
            np.zeros((r, n), np.int8), np.zeros(ng, np.float32))


def random_moments(cfg: Config, L: LayerShape, r: int):
    """Non-zero INT8 moments (M signed, V non-negative) with positive scales."""
    g = rng(cfg, L.layer_id, 0, TAG_M)
    ng = -(-(r * L.n) // 256)
    Mq = g.integers(-127, 128, size=(r, L.n), dtype=np.int8)
    Ms = (g.random(ng, dtype=np.float32) * np.float32(1e-4)).astype(np.float32)
    Vq = g.integers(0, 128, size=(r, L.n), dtype=np.int8)
    Vs = (g.random(ng, dtype=np.float32) * np.float32(1e-8)).astype(np.float32)
    return Mq, Ms, Vq, Vs


# ------------------------------- device (torch) draws ----------------------------------

def gradient_bf16_device(cfg: Config, L: LayerShape, step: int, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, step, TAG_G))
    g = torch.randn((L.m, L.n), generator=gen, device=device, dtype=torch.float32)
    return (g * cfg.sigma).to(torch.bfloat16)


def weights_int8_device(cfg: Config, L: LayerShape, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, 0, TAG_W))
    return torch.randint(-127, 128, (L.m, L.n), generator=gen, device=device,
                         dtype=torch.int32).to(torch.int8)


def orthonormal_device(cfg: Config, L: LayerShape, r: int, tag: int = TAG_P, step: int = 0,
                       device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, step, tag))
    a = torch.randn((L.m, r), generator=gen, device=device, dtype=torch.float32)
    q, _ = torch.linalg.qr(a)
    return q.contiguous()


# ------------------------------ drifting low-rank gradients ---------------------------
# G_t = A_t S B^T + 0.1 sigma Z_t with A_t = A0 cos(rho t) + A1 sin(rho t): [A0 A1] is the Q of
# a seeded Gaussian m x 2k, B the Q of a Gaussian n x k, S = diag(sigma sqrt(m n / k) *
# linspace(1.5, 0.5, k)), Z_t standard normal. The top-k left singular subspace of the
# noise-free G_t is span(A_t), so the subspace similarity of steps t and s is |cos(rho (t-s))|.

def drift_rate(cfg: Config, index: int) -> float:
    return DRIFT_MAX * index / max(1, len(cfg.layers) - 1)


def drift_basis_device(cfg: Config, L: LayerShape, device="cuda"):
    """(A0, A1, B scaled by S): A0, A1 m x k, BS = B S  n x k (fp32), with k = cfg.r."""
    import torch
    k = cfg.r
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, 0, TAG_DRIFT_A))
    a, _ = torch.linalg.qr(torch.randn((L.m, 2 * k), generator=gen, device=device))
    gen.manual_seed(torch_seed(cfg, L.layer_id, 0, TAG_DRIFT_B))
    b, _ = torch.linalg.qr(torch.randn((L.n, k), generator=gen, device=device))
    sv = cfg.sigma * (L.m * L.n / k) ** 0.5 * torch.linspace(1.5, 0.5, k, device=device)
    return a[:, :k].contiguous(), a[:, k:].contiguous(), (b * sv[None, :]).contiguous()


def drift_gradient_device(cfg: Config, L: LayerShape, basis, rho: float, step: int, out=None):
    """G_t (bf16, m x n) of the drifting workload; written into `out` when given."""
    import math
    import torch
    A0, A1, BS = basis
    At = A0 * math.cos(rho * step) + A1 * math.sin(rho * step)
    gen = torch.Generator(device=A0.device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, step, TAG_NOISE))
    G = torch.randn((L.m, L.n), generator=gen, device=A0.device) * (0.1 * cfg.sigma)
    G.addmm_(At, BS.t())
    if out is None:
        return G.to(torch.bfloat16)
    out.copy_(G)
    return out


def sketch_device(cfg: Config, L: LayerShape, width: int, step: int, device="cuda"):
    """Gaussian sketch (bf16 n x width) of the randomized refresh of layer L at `step`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, step, TAG_SKETCH))
    return torch.randn((L.n, width), generator=gen, device=device).to(torch.bfloat16)


def top_subspace_device(cfg: Config, L: LayerShape, G, k: int, step: int, oversample: int = 8,
                        power_iters: int = 2):
    """Orthonormal basis (m x k, fp32) of the top-k left singular subspace of G, by a
    randomized range finder with power iterations (Halko, Martinsson and Tropp, 2011): a
    Gaussian sketch of k + oversample columns, power iterations re-orthonormalized by QR, then
    the leading eigenvectors of the small Gram matrix of the sketch's projection."""
    import torch
    Gf = G.float()
    gen = torch.Generator(device=G.device)
    gen.manual_seed(torch_seed(cfg, L.layer_id, step, TAG_SKETCH))
    Om = torch.randn((L.n, k + oversample), generator=gen, device=G.device)
    Q, _ = torch.linalg.qr(Gf @ Om)
    for _ in range(power_iters):
        Z, _ = torch.linalg.qr(Gf.t() @ Q)
        Q, _ = torch.linalg.qr(Gf @ Z)
    Bm = Q.t() @ Gf                        # (k + p) x n
    evals, evecs = torch.linalg.eigh(Bm @ Bm.t())
    top = evecs[:, torch.argsort(evals, descending=True)[:k]]
    return (Q @ top).contiguous()
