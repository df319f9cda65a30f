"""Seeded synthetic inputs for the FP8 hot path (input generation only).

This module draws random tensors and rounds them to bf16; it holds none of the
method's arithmetic, and both the GPU path and the oracle are fed from it.

Every tensor is identified by (seed, tensor_id).  It is drawn in chunks of
2^22 elements; chunk c comes from ``numpy.random.default_rng([seed,
tensor_id, c])`` (float32 standard normals, or float64 Student-t), is scaled by
its standard deviation and rounded to bf16 (round to nearest even, via
torch's CPU cast).  Chunks are drawn in parallel threads, and the result does
not depend on the number of threads.

The shapes and distributions stand in for the pages' 7B-32B training
workloads (Llama2-7B, Qwen2.5-14B and a 32B model are the models the pages
train); no dataset is involved.
"""
from __future__ import annotations

import concurrent.futures
import os
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 22


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw(seed: int, tensor_id: int, shape, sigma: float = 1.0, dist: str = "normal",
         outlier_frac: float = 0.0, outlier_scale: float = 50.0) -> torch.Tensor:
    """A bf16 CPU tensor of `shape`.

    dist "normal": N(0, sigma^2).  dist "student_t": Student-t with 3 degrees
    of freedom, times sigma.  outlier_frac > 0: round(outlier_frac * cols)
    columns (chosen by a seeded permutation) are multiplied by outlier_scale
    before the bf16 rounding.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng([seed, tensor_id, c])
        if dist == "normal":
            out[lo:hi] = rng.standard_normal(hi - lo, dtype=np.float32)
        elif dist == "student_t":
            out[lo:hi] = rng.standard_t(3, hi - lo).astype(np.float32)
        else:
            raise ValueError(dist)
        if sigma != 1.0:
            out[lo:hi] *= np.float32(sigma)

    nchunks = (n + CHUNK - 1) // CHUNK
    with concurrent.futures.ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    arr = out.reshape(shape)
    if outlier_frac > 0:
        cols = shape[-1]
        k = int(round(outlier_frac * cols))
        pick = np.random.default_rng([seed, tensor_id, 1 << 30]).permutation(cols)[:k]
        arr[..., pick] *= np.float32(outlier_scale)
    t = torch.from_numpy(arr)
    return t.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bf16 tensor (CPU, as numpy)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Linear:
    name: str
    K: int            # input features
    N: int            # output features


@dataclass
class Config:
    name: str
    seed: int
    M: int                              # tokens
    linears: list = field(default_factory=list)
    x_dist: str = "normal"
    x_outlier_frac: float = 0.0
    w_sigma: float = 0.02
    dy_sigma: float = 1e-3
    backward: bool = True
    mlp_chain: bool = False             # X -> gate/up -> SwiGLU requant -> down
    recompute: bool = False             # MLP recomputation with retained statistics
    description: str = ""


def _layer(d, ffn, qkv_out):
    return [Linear("qkv", d, qkv_out), Linear("o", d, d), Linear("gate_up", d, 2 * ffn), Linear("down", ffn, d)]


CONFIGS = {
    "fc256": Config("fc256", 0, 128, [Linear("fc", 256, 256)], backward=False,
                 description="single FP8 linear forward, X [128,256] N(0,1), W [256,256] N(0,0.02)"),
    "mlp7b": Config("mlp7b", 1, 4096, [Linear("gate_up", 4096, 22016), Linear("down", 11008, 4096)],
                 backward=False, mlp_chain=True,
                 description="7B-class SwiGLU MLP forward, M=4096, d=4096, ffn=11008"),
    "layer7b": Config("layer7b", 2, 4096, _layer(4096, 11008, 12288),
                 description="7B-class layer linears forward+backward, M=4096"),
    "layer14b": Config("layer14b", 3, 8192, _layer(5120, 13824, 7168), x_dist="student_t", x_outlier_frac=0.001,
                 description="14B-class layer linears forward+backward, M=8192, Student-t(3) X with "
                             "0.1% of channels x50"),
    "layer32b": Config("layer32b", 4, 16384, _layer(5120, 27648, 7168), mlp_chain=True, recompute=True,
                 description="32B-class layer linears forward+backward, M=16384, MLP recomputation "
                             "with retained statistics"),
}


def tensor_ids(li: int):
    """(X, W, dY) tensor ids of the li-th linear of a config."""
    return 10 * li, 10 * li + 1, 10 * li + 2


def draw_x(cfg: Config, li: int) -> torch.Tensor:
    lin = cfg.linears[li]
    return draw(cfg.seed, tensor_ids(li)[0], (cfg.M, lin.K), 1.0, cfg.x_dist, cfg.x_outlier_frac)


def draw_w(cfg: Config, li: int) -> torch.Tensor:
    lin = cfg.linears[li]
    return draw(cfg.seed, tensor_ids(li)[1], (lin.N, lin.K), cfg.w_sigma)


def draw_dy(cfg: Config, li: int) -> torch.Tensor:
    lin = cfg.linears[li]
    return draw(cfg.seed, tensor_ids(li)[2], (cfg.M, lin.N), cfg.dy_sigma)
