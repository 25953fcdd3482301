"""Seeded synthetic inputs for the SmoothQuant W8A8 linear layer.

This module is the only code that both the GPU library's tests/bench and the
CPU oracle use.  It holds no step of the method: it only draws random numbers
and casts them to the input dtype, so both sides receive identical bits.

The workloads mirror the pages' setting (abeam.tech SmoothQuant explainer,
基本アイデア / 課題: a few activation channels carry large outliers, and they
stay in the same channels across tokens).  Every activation draw is
``X[t, j] = z[t, j] * (factor if j is an outlier channel else 1)`` with
``z ~ N(0, 1)``; weights are ``N(0, sigma)`` (sigma a standard deviation).
Outlier channel indices are drawn once per (config, layer) and reused for the
calibration draw and for every evaluation draw ("persistent").

Seeds: ``numpy.random.default_rng([config, layer_index, stream])`` with
stream 0 = outlier indices, 1 = W, 2 = calibration X, 3 = evaluation X,
4 = LayerNorm gamma/beta.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Layer:
    name: str
    K: int  # input channels
    N: int  # output channels


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    layers: tuple
    M: tuple          # evaluation token counts
    T: int            # calibration tokens
    act: str          # activation dtype
    wdt: str          # weight dtype
    ydt: str          # output dtype
    sigma: float      # weight standard deviation
    outliers: tuple   # ("count", n) or ("frac", f) of the layer's K
    factor: float     # outlier magnitude multiplier
    alphas: tuple = field(default=(0.5,))

    def layer(self, name: str) -> Layer:
        for ly in self.layers:
            if ly.name == name:
                return ly
        raise KeyError(name)

    def n_outliers(self, K: int) -> int:
        kind, v = self.outliers
        if kind == "count":
            return int(v)
        return int(round(v * K))


CONFIGS = {
    1: Config(1, "toy-512", (Layer("toy", 512, 512),), (16,), 64, "f32", "f32", "f16",
              0.02, ("count", 5), 40.0),
    2: Config(2, "opt-6.7b", (Layer("qkv", 4096, 12288), Layer("fc1", 4096, 16384),
                              Layer("fc2", 16384, 4096)),
              (1, 16, 512, 2048), 512, "f16", "f16", "f16", 0.02, ("frac", 0.005), 60.0),
    3: Config(3, "opt-13b", (Layer("qkv", 5120, 15360), Layer("fc1", 5120, 20480),
                             Layer("fc2", 20480, 5120)),
              (4096,), 512, "f16", "f16", "f16", 0.02, ("count", 6), 80.0,
              (0.4, 0.5, 0.6, 0.75)),
    4: Config(4, "opt-175b", (Layer("qkv", 12288, 36864), Layer("fc1", 12288, 49152),
                              Layer("fc2", 49152, 12288)),
              (2048, 8192), 512, "bf16", "bf16", "bf16", 0.02, ("frac", 0.001), 100.0),
    5: Config(5, "llama-70b-decode", (Layer("up", 8192, 28672), Layer("down", 28672, 8192)),
              (1, 4, 8, 16), 512, "f16", "f16", "f16", 0.015, ("count", 8), 50.0),
}


def _rng(cid: int, layer_idx: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([cid, layer_idx, stream])


def _layer_index(cfg: Config, layer: str) -> int:
    for i, ly in enumerate(cfg.layers):
        if ly.name == layer:
            return i
    raise KeyError(layer)


def _cast(a: np.ndarray, dt: str) -> torch.Tensor:
    """float32 numpy -> CPU tensor of the workload dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DTYPES[dt])


def outlier_channels(cfg: Config, layer: str) -> np.ndarray:
    ly = cfg.layer(layer)
    n = cfg.n_outliers(ly.K)
    idx = _rng(cfg.cid, _layer_index(cfg, layer), 0).choice(ly.K, size=n, replace=False)
    return np.sort(idx)


def weight(cfg: Config, layer: str) -> torch.Tensor:
    """W [K x N] in the weight dtype (row j multiplies input channel j)."""
    ly = cfg.layer(layer)
    z = _rng(cfg.cid, _layer_index(cfg, layer), 1).standard_normal((ly.K, ly.N), dtype=np.float32)
    z *= np.float32(cfg.sigma)
    return _cast(z, cfg.wdt)


def activations(cfg: Config, layer: str, rows: int, calibration: bool = False) -> torch.Tensor:
    """X [rows x K] with persistent outlier channels, in the activation dtype."""
    ly = cfg.layer(layer)
    stream = 2 if calibration else 3
    z = _rng(cfg.cid, _layer_index(cfg, layer), stream).standard_normal((rows, ly.K),
                                                                          dtype=np.float32)
    z[:, outlier_channels(cfg, layer)] *= np.float32(cfg.factor)
    return _cast(z, cfg.act)


def layernorm_params(cfg: Config, layer: str):
    """(gamma, beta) float32 [K]: gamma ~ 1 + N(0, 0.1), beta ~ N(0, 0.1)."""
    ly = cfg.layer(layer)
    r = _rng(cfg.cid, _layer_index(cfg, layer), 4)
    gamma = (1.0 + 0.1 * r.standard_normal(ly.K)).astype(np.float32)
    beta = (0.1 * r.standard_normal(ly.K)).astype(np.float32)
    return torch.from_numpy(gamma), torch.from_numpy(beta)


def random_matrix(seed: int, rows: int, cols: int, dt: str = "f32", scale: float = 1.0,
                  outlier_cols=None, factor: float = 1.0) -> torch.Tensor:
    """Generic seeded N(0, scale) matrix for shape-sweep tests."""
    z = np.random.default_rng([99, seed]).standard_normal((rows, cols), dtype=np.float32)
    z *= np.float32(scale)
    if outlier_cols is not None and len(outlier_cols):
        z[:, outlier_cols] *= np.float32(factor)
    return _cast(z, dt)


def random_int8(seed: int, rows: int, cols: int) -> np.ndarray:
    """Uniform int8 codes in [-127, 127] (the quantiser's code range)."""
    return np.random.default_rng([98, seed]).integers(-127, 128, size=(rows, cols),
                                                      dtype=np.int16).astype(np.int8)


def device_matrix(seed: int, rows: int, cols: int, dt: str, device, scale: float = 1.0,
                  outlier_cols=None, factor: float = 1.0) -> torch.Tensor:
    """Seeded N(0, scale) matrix drawn on the device (torch's generator), for
    tensors too large to draw on the host in a test's time; the values a test
    checks are copied back, so both sides still see identical bits."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    z = torch.randn(rows, cols, generator=g, device=device, dtype=DTYPES[dt])
    if scale != 1.0:
        z.mul_(scale)
    if outlier_cols is not None and len(outlier_cols):
        idx = torch.as_tensor(np.asarray(outlier_cols, dtype=np.int64), device=device)
        z[:, idx] *= factor
    return z


def device_int8(seed: int, rows: int, cols: int, device) -> torch.Tensor:
    """Seeded uniform int8 codes in [-127, 127] drawn on the device."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randint(-127, 128, (rows, cols), generator=g, device=device, dtype=torch.int8)
