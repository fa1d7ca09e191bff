"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers: it holds none of the method's
arithmetic (no rotation, no quantisation, no product).  The random sign
vector the method uses is drawn here and passed as an input to both the
kernels and the oracle.

Recipes (each reproducible from ``(config_id, seed)`` through
``numpy.random.default_rng([config_id, seed])``; draws happen in the order
listed):

* outlier channels follow the activation-outlier description in the llms.blog
  page "Rotational Quantization: How Orthogonal Transforms and Hadamard
  Incoherence Enable Outlier-Free Low-Bit Inference", section "The Activation
  Outlier Bottleneck in Low-Bit Serving": a small fixed set of channels (about
  0.1%, at least one) is scaled up, and the same channels are scaled in every
  token.  The set is drawn without replacement once per seed.
* Rademacher signs: integers(0, 2, n) * 2 - 1 as int8.
* Gaussian values are drawn in float32, outlier channels are multiplied after
  the draw, and the result is cast to the stated storage dtype (fp16 rounds
  to nearest even).
* Weights are i.i.d. N(0, 0.02^2), so W^T [k][d] (the stored layout) is drawn
  directly.
"""

from __future__ import annotations

import numpy as np

CONFIG_TINY = 0
CONFIG_FWHT = 1
CONFIG_DECODE = 2
CONFIG_PREFILL = 3
CONFIG_KV = 4


def rng_for(config_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(seed)])


def rademacher(rng: np.random.Generator, n: int) -> np.ndarray:
    return (rng.integers(0, 2, n) * 2 - 1).astype(np.int8)


def outlier_channels(rng: np.random.Generator, d: int, frac: float = 0.001) -> np.ndarray:
    count = max(1, int(round(frac * d)))
    return np.sort(rng.choice(d, size=count, replace=False))


def gaussian(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def activations(rng, m: int, d: int, channels: np.ndarray, factor: float,
                dtype=np.float16) -> np.ndarray:
    x = gaussian(rng, (m, d))
    x[:, channels] *= np.float32(factor)
    return x.astype(dtype)


def tiny_linear(seed: int = 0) -> dict:
    """8 x 256 fp32 activations with channels 3 and 77 scaled x50, weights
    256 -> 512 ~ N(0, 0.02^2), rotation n = 256 with Rademacher signs."""
    rng = rng_for(CONFIG_TINY, seed)
    d, m, k = 256, 8, 512
    signs = rademacher(rng, d)
    channels = np.array([3, 77])
    x = activations(rng, m, d, channels, 50.0, dtype=np.float32)
    wt = gaussian(rng, (k, d), std=0.02)
    return {"x": x, "wt": wt, "signs": signs, "channels": channels, "m": m, "d": d, "k": k}


def fwht_workload(seed: int = 0, m: int = 4096, d: int = 4096) -> dict:
    """4096 tokens x 4096 fp16 ~ N(0,1) with 0.1% of channels scaled x100."""
    rng = rng_for(CONFIG_FWHT, seed)
    signs = rademacher(rng, d)
    channels = outlier_channels(rng, d)
    x = activations(rng, m, d, channels, 100.0)
    return {"x": x, "signs": signs, "channels": channels, "m": m, "d": d}


def decode_linear(seed: int = 0, m: int = 16, d: int = 4096, ks=(4096, 14336)) -> dict:
    """Decode-shaped linear: up to 16 fp16 tokens of width 4096 (0.1% of
    channels x100); weights for each output width in ``ks``."""
    rng = rng_for(CONFIG_DECODE, seed)
    signs = rademacher(rng, d)
    channels = outlier_channels(rng, d)
    x = activations(rng, m, d, channels, 100.0)
    wts = {int(k): gaussian(rng, (int(k), d), std=0.02) for k in ks}
    return {"x": x, "wts": wts, "signs": signs, "channels": channels, "m": m, "d": d}


def prefill_linear(seed: int = 0, m: int = 2048, d: int = 8192, k: int = 28672,
                   with_weights: bool = True) -> dict:
    """Prefill-shaped linear: 2048 fp16 tokens of width 8192 (0.1% of
    channels x100) into 28672 outputs."""
    rng = rng_for(CONFIG_PREFILL, seed)
    signs = rademacher(rng, d)
    channels = outlier_channels(rng, d)
    x = activations(rng, m, d, channels, 100.0)
    wt = gaussian(rng, (k, d), std=0.02) if with_weights else None
    return {"x": x, "wt": wt, "signs": signs, "channels": channels, "m": m, "d": d, "k": k}


def kv_cache(seed: int = 0, batch: int = 32, heads: int = 8, seq: int = 4096,
             head_dim: int = 128, per_head: int = 2, factor: float = 20.0) -> dict:
    """K and V fp16 [batch, heads, seq, head_dim] ~ N(0,1); in every head
    ``per_head`` head_dim channels are scaled by ``factor`` (drawn separately
    for K and for V, the same for every batch entry and position)."""
    rng = rng_for(CONFIG_KV, seed)
    k_ch = np.stack([np.sort(rng.choice(head_dim, per_head, replace=False)) for _ in range(heads)])
    v_ch = np.stack([np.sort(rng.choice(head_dim, per_head, replace=False)) for _ in range(heads)])
    out = {"k_channels": k_ch, "v_channels": v_ch}
    for name, ch in (("k", k_ch), ("v", v_ch)):
        t = gaussian(rng, (batch, heads, seq, head_dim))
        mult = np.ones((heads, head_dim), dtype=np.float32)
        for h in range(heads):
            mult[h, ch[h]] = np.float32(factor)
        t *= mult[None, :, None, :]
        out[name] = t.astype(np.float16)
    return out


def random_codes(rng: np.random.Generator, rows: int, d: int) -> np.ndarray:
    """Uniform random packed int4 codes [rows][d/2] (every nibble value)."""
    return rng.integers(0, 256, size=(rows, d // 2), dtype=np.uint8)


def random_scales(rng: np.random.Generator, rows: int, lo: float = 1e-3, hi: float = 1.0) -> np.ndarray:
    return rng.uniform(lo, hi, size=rows).astype(np.float16)


def random_codes8(rng: np.random.Generator, rows: int, d: int) -> np.ndarray:
    """Uniform random INT8 activation codes [rows][d] (every value in [-128, 127])."""
    return rng.integers(-128, 128, size=(rows, d), dtype=np.int8)
