"""Seeded synthetic INT8 tensors shaped like the workloads the Shannonic codec targets.

This module draws random numbers and nothing else: it holds none of the codec's
arithmetic, so both the HIP path and the CPU oracle can be fed from it.

Every generator uses numpy's PCG64 with a fixed seed, rounds half-to-even
(``np.rint``), clips to [-128, 127] and casts to int8.  The real tensors the
Shannonic talk notes evaluate on (8-bit quantised vision/NLP/LLM weights and
activations, section "Evaluation: compression ratio", paper section 5) are not
available, so these distributions stand in for them:

* ``tiny``         65,536 values, N(0, 20).
* ``weight``       4096 x 1024, Laplace(0, b=12) with probability 0.98, else N(0, 60).
* ``kv_cache``     [2, 8, 32768, 128]; per (K/V, head) slab a Gaussian with
                   sigma_h = exp(N(2.5, 0.5)); 4 channels per head drawn at 5 sigma_h.
* ``activations``  [16, 2048, 4096], Student-t (nu=3) rescaled to sigma = 25.
* ``model_tensors`` 224 weight tensors of an 8B-style layout (32 layers x
                   q, k, v, o, gate, up, down), each Laplace(0, b ~ U(6, 20)),
                   with an all-zero and a uniform-over-256 edge tensor in layer 0.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "quantize",
    "tiny",
    "weight",
    "kv_cache",
    "activations",
    "model_layout",
    "model_tensor",
    "model_tensor_torch",
    "uniform_exact",
    "CONFIGS",
]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def quantize(a: np.ndarray) -> np.ndarray:
    """Round half-to-even, clip to the INT8 range and cast."""
    return np.clip(np.rint(a), -128, 127).astype(np.int8)


def tiny(seed: int = 1, n: int = 65536) -> np.ndarray:
    return quantize(_rng(seed).normal(0.0, 20.0, size=n))


def weight(seed: int = 2, rows: int = 4096, cols: int = 1024, b: float = 12.0) -> np.ndarray:
    g = _rng(seed)
    n = rows * cols
    lap = g.laplace(0.0, b, size=n)
    wide = g.normal(0.0, 60.0, size=n)
    pick = g.random(size=n) < 0.02
    return quantize(np.where(pick, wide, lap)).reshape(rows, cols)


def kv_cache(seed: int = 3, kv: int = 2, heads: int = 8, tokens: int = 32768,
             head_dim: int = 128, outliers: int = 4) -> np.ndarray:
    g = _rng(seed)
    out = np.empty((kv, heads, tokens, head_dim), dtype=np.int8)
    for a in range(kv):
        for h in range(heads):
            sigma = float(np.exp(g.normal(2.5, 0.5)))
            scale = np.full(head_dim, sigma)
            scale[g.choice(head_dim, size=outliers, replace=False)] = 5.0 * sigma
            out[a, h] = quantize(g.standard_normal((tokens, head_dim)) * scale)
    return out


def activations(seed: int = 4, batch: int = 16, seq: int = 2048, hidden: int = 4096,
                nu: float = 3.0, sigma: float = 25.0) -> np.ndarray:
    g = _rng(seed)
    out = np.empty((batch, seq, hidden), dtype=np.int8)
    # the variance of Student-t(nu) is nu / (nu - 2)
    s = sigma / np.sqrt(nu / (nu - 2.0))
    for b in range(batch):
        out[b] = quantize(g.standard_t(nu, size=(seq, hidden)) * s)
    return out


def model_layout(layers: int = 32, hidden: int = 4096, kv_dim: int = 1024,
                 ffn: int = 14336):
    """(name, shape) of every weight tensor, in layer order."""
    per_layer = [
        ("q_proj", (hidden, hidden)),
        ("k_proj", (kv_dim, hidden)),
        ("v_proj", (kv_dim, hidden)),
        ("o_proj", (hidden, hidden)),
        ("gate_proj", (ffn, hidden)),
        ("up_proj", (ffn, hidden)),
        ("down_proj", (hidden, ffn)),
    ]
    return [(f"layers.{i}.{nm}", shp) for i in range(layers) for nm, shp in per_layer]


def model_tensor(idx: int, seed: int = 5, **layout) -> np.ndarray:
    """Tensor ``idx`` of ``model_layout``: Laplace(0, b ~ U(6, 20)), seed + idx.

    Layer 0's q_proj is all zero and its o_proj is uniform over the 256 codes.
    """
    name, shape = model_layout(**layout)[idx]
    g = _rng(seed + idx)
    if name == "layers.0.q_proj":
        return np.zeros(shape, dtype=np.int8)
    if name == "layers.0.o_proj":
        return g.integers(-128, 128, size=shape, dtype=np.int16).astype(np.int8)
    b = g.uniform(6.0, 20.0)
    return quantize(g.laplace(0.0, b, size=shape))


def uniform_exact(count: int = 1000, seed: int = 0) -> np.ndarray:
    """Every INT8 value exactly ``count`` times, in a seeded random order."""
    x = np.repeat(np.arange(-128, 128, dtype=np.int16), count).astype(np.int8)
    _rng(seed).shuffle(x)
    return x


# Codec parameters of each workload: (ranges K, log2 of tANS states, chunk symbols, streams).
CONFIGS = {
    "tiny": dict(K=16, log2_L=7, chunk=4096, streams=32),
    "weight": dict(K=16, log2_L=7, chunk=4096, streams=32),
    "kv_cache": dict(K=16, log2_L=7, chunk=8192, streams=32),
    # the activation workload fixes no stream count: 64 streams a chunk give its 8,192 chunks
    # twice the independent streams of 32, at about 0.13% of H more framing (measured on
    # MI355X: decode 98.8 -> 81.6 us with four streams a lane, encode 168 -> 152 us)
    "activations": dict(K=16, log2_L=7, chunk=16384, streams=64),
    # the model-scale workload fixes neither: 16,384 values (as for the activations) keep the
    # per-chunk framing (lane initial states, index entry, padding) near 0.4% of H on these
    # weights, where 4,096 cost about 1.2%; 64 streams (four a lane, one LDS write of the
    # lane's four bytes a step) decoded a 48-tensor launch in 625 us against 676 us for 32,
    # for 0.12% of H more framing
    "model": dict(K=16, log2_L=7, chunk=16384, streams=64),
}


def model_tensor_torch(idx: int, device, seed: int = 5, **layout):
    """Tensor ``idx`` of ``model_layout`` drawn on ``device`` with torch's seeded generator,
    the same recipe as ``model_tensor`` (Laplace(0, b), b ~ U(6, 20) from the same numpy
    seed; layer 0's q_proj all zero, o_proj uniform) but other draws: a model's 7e9 values
    are generated on the GPU in about a second instead of minutes on the host.  Laplace by
    inversion: x = -b sign(v) log(1 - 2|v|), v uniform on [-1/2, 1/2)."""
    import torch
    name, shape = model_layout(**layout)[idx]
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + idx)
    if name == "layers.0.q_proj":
        return torch.zeros(shape, dtype=torch.int8, device=device)
    if name == "layers.0.o_proj":
        return torch.randint(-128, 128, shape, generator=g, device=device,
                             dtype=torch.int16).to(torch.int8)
    b = float(_rng(seed + idx).uniform(6.0, 20.0))
    v = torch.rand(shape, generator=g, device=device, dtype=torch.float32) - 0.5
    x = -b * torch.sign(v) * torch.log1p(-2.0 * v.abs())
    return torch.clamp(torch.round(x), -128, 127).to(torch.int8)
