"""Seeded synthetic workloads for the routed-MoE layer.

This module only draws random numbers and rounds them to the storage types
(binary16, bfloat16); it holds none of the layer's arithmetic, so both the GPU
library's tests/benchmark and the CPU oracle can take their inputs from it.

Workloads (shapes from the DS4 (DwarfStar 4) wiki note, "Architecture": 256
routed experts, 6 active + 1 shared, d_model 4096; prefill chunk of 2048 from
the same section; 16 batched decode sessions from TopDigg "DwarfStar (ds4)
Deep Dive", section 5.4):

  tiny      d 256,  E 16,  top-2, f = fs = 256,  T 8,    x fp32
  decode1   d 4096, E 256, top-6, f = fs = 2048, T 1,    x bf16
  decode16  as decode1, T 16, +10 router bias on a seeded pool of 88 experts
  prefill   as decode1, T 2048, bias -1.1*beta*ln(rank) (Zipf-like loads)
  stack43   43 layers of the decode1 shape, per-layer seeds 1000 + layer

Hyper-connection mixer inputs (the n = 4 streams of d around each layer, DS4
(DwarfStar 4) wiki note, "Key Techniques"), gen_hc: streams X [T, 4, d] fp32
N(0, 1) with stream i scaled by 2^(i - 1); projection phi [24, 4d] fp32
N(0, 1/128^2), so each mixer logit has unit spread at d = 4096; bias [24]:
pre/post N(0, 1), residual mixer 4 I + N(0, 0.5^2) (a near-identity mixer);
alpha = (1, 1, 1).  Streams 10..13 of the layer seed.

Every tensor comes from numpy PCG64(SeedSequence([cfg_seed, stream, variant])):
stream 0 = x, 1 = router, 2/3/4 = shared gate/up/down, 5 = bias / pool,
100 + 3*e + m = routed expert e, matrix m (0 gate, 1 up, 2 down).  Draws are
float32 standard normals scaled by 0.02 (weights) or 1 (activations), then
rounded to nearest-even into binary16 / bfloat16 where the layer stores them.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

WEIGHT_SIGMA = 0.02

STREAM_X, STREAM_ROUTER, STREAM_SH_GATE, STREAM_SH_UP, STREAM_SH_DOWN, STREAM_BIAS = 0, 1, 2, 3, 4, 5
STREAM_HC_X, STREAM_HC_PHI, STREAM_HC_BIAS, STREAM_HC_Y = 10, 11, 12, 13
HC_STREAMS = 4
HC_SINKHORN_ITERS = 20
HC_EPS = 1e-6


def expert_stream(e: int, m: int) -> int:
    return 100 + 3 * e + m


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    d: int
    E: int
    k: int
    f: int
    fs: int
    T: int
    x_dtype: str  # "f32" or "bf16"
    seed: int
    router_variant: int = 0
    x_variant: int = 0
    bias: str | None = None  # None, "hotpool", "zipf"
    hot_pool: int = 88
    hot_bias: float = 10.0
    zipf_beta: float = 1.0
    layers: int = 1


# router_variant / x_variant / zipf_beta values are the ones the committed
# script tests/golden/find_seeds.py selected with the CPU oracle (top-k gap
# > 1e-4 for every token; distinct-expert count and Zipf slope targets).
CONFIGS = {
    "tiny": Config("tiny", 256, 16, 2, 256, 256, 8, "f32", seed=0),
    "decode1": Config("decode1", 4096, 256, 6, 2048, 2048, 1, "bf16", seed=1),
    "decode16": Config("decode16", 4096, 256, 6, 2048, 2048, 16, "bf16", seed=3, bias="hotpool"),
    "prefill": Config("prefill", 4096, 256, 6, 2048, 2048, 2048, "bf16", seed=4, bias="zipf",
                      router_variant=4, zipf_beta=0.546875),
    "stack43": Config("stack43", 4096, 256, 6, 2048, 2048, 1, "bf16", seed=1000, layers=43),
}


def rng(cfg_seed: int, stream: int, variant: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_seed, stream, variant])))


def normal_f32(g: np.random.Generator, shape, scale: float) -> np.ndarray:
    a = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def gen_x(cfg: Config, variant: int | None = None, T: int | None = None, cfg_seed: int | None = None):
    """Activations [T, d]: float32 (x_dtype f32) or bfloat16 bits as uint16."""
    T = cfg.T if T is None else T
    v = cfg.x_variant if variant is None else variant
    s = cfg.seed if cfg_seed is None else cfg_seed
    a = normal_f32(rng(s, STREAM_X, v), (T, cfg.d), 1.0)
    return a if cfg.x_dtype == "f32" else f32_to_bf16_bits(a)


def gen_router(cfg: Config, variant: int | None = None, cfg_seed: int | None = None) -> np.ndarray:
    """Router weights [E, d] as binary16 bits."""
    v = cfg.router_variant if variant is None else variant
    s = cfg.seed if cfg_seed is None else cfg_seed
    return f32_to_f16_bits(normal_f32(rng(s, STREAM_ROUTER, v), (cfg.E, cfg.d), WEIGHT_SIGMA))


def gen_bias(cfg: Config, beta: float | None = None) -> np.ndarray | None:
    """Optional fp32 router bias [E] that shapes the expert load."""
    if cfg.bias is None:
        return None
    g = rng(cfg.seed, STREAM_BIAS)
    perm = g.permutation(cfg.E)
    b = np.zeros(cfg.E, dtype=np.float32)
    if cfg.bias == "hotpool":
        b[perm[: cfg.hot_pool]] = np.float32(cfg.hot_bias)
    elif cfg.bias == "zipf":
        beta = cfg.zipf_beta if beta is None else beta
        rank = np.empty(cfg.E, dtype=np.float64)
        rank[perm] = np.arange(1, cfg.E + 1, dtype=np.float64)
        b[:] = (-1.1 * beta * np.log(rank)).astype(np.float32)
    else:
        raise ValueError(cfg.bias)
    return b


def gen_shared(cfg: Config, cfg_seed: int | None = None):
    """Shared expert gate [fs, d], up [fs, d], down [d, fs] as binary16 bits."""
    s = cfg.seed if cfg_seed is None else cfg_seed
    gate = f32_to_f16_bits(normal_f32(rng(s, STREAM_SH_GATE), (cfg.fs, cfg.d), WEIGHT_SIGMA))
    up = f32_to_f16_bits(normal_f32(rng(s, STREAM_SH_UP), (cfg.fs, cfg.d), WEIGHT_SIGMA))
    down = f32_to_f16_bits(normal_f32(rng(s, STREAM_SH_DOWN), (cfg.d, cfg.fs), WEIGHT_SIGMA))
    return gate, up, down


def gen_expert(cfg: Config, e: int, cfg_seed: int | None = None):
    """Routed expert e before quantization: gate [f, d], up [f, d], down [d, f] float32."""
    s = cfg.seed if cfg_seed is None else cfg_seed
    gate = normal_f32(rng(s, expert_stream(e, 0)), (cfg.f, cfg.d), WEIGHT_SIGMA)
    up = normal_f32(rng(s, expert_stream(e, 1)), (cfg.f, cfg.d), WEIGHT_SIGMA)
    down = normal_f32(rng(s, expert_stream(e, 2)), (cfg.d, cfg.f), WEIGHT_SIGMA)
    return gate, up, down


def gen_experts(cfg: Config, experts, threads: int = 8, cfg_seed: int | None = None):
    """gen_expert over a list of experts on a thread pool (numpy drops the GIL
    while it fills arrays); returns a list in the order given."""
    experts = list(experts)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda e: gen_expert(cfg, e, cfg_seed), experts))


def stack_layer_seed(layer: int) -> int:
    return CONFIGS["stack43"].seed + layer


def stack_token_x(cfg: Config, n: int) -> np.ndarray:
    """Input row of token n to the layer stack (seed 5000 + n)."""
    a = normal_f32(rng(5000 + n, STREAM_X), (1, cfg.d), 1.0)
    return f32_to_bf16_bits(a)


def zipf_reference(E: int, s: float = 1.1) -> np.ndarray:
    """Normalised Zipf(s) probabilities over ranks 1..E (a target, not a draw)."""
    p = 1.0 / np.arange(1, E + 1, dtype=np.float64) ** s
    return p / p.sum()


def rank_frequency_slope(counts: np.ndarray) -> float:
    """Least-squares slope of log(load) against log(rank) over experts with load > 0."""
    c = np.sort(np.asarray(counts, dtype=np.float64))[::-1]
    c = c[c > 0]
    r = np.arange(1, len(c) + 1, dtype=np.float64)
    A = np.vstack([np.log(r), np.ones_like(r)]).T
    slope, _ = np.linalg.lstsq(A, np.log(c), rcond=None)[0]
    return float(slope)


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "dataclasses", "math", "np")]


def gen_hc(d: int, T: int, cfg_seed: int = 7, variant: int = 0):
    """Hyper-connection mixer inputs: streams X [T, 4, d], projection phi
    [24, 4d], bias [24], alpha (3,), sublayer output y [T, d]; float32."""
    n = HC_STREAMS
    no = 2 * n + n * n
    X = normal_f32(rng(cfg_seed, STREAM_HC_X, variant), (T, n, d), 1.0)
    X *= np.array([0.5, 1.0, 2.0, 4.0], dtype=np.float32)[None, :, None]
    phi = normal_f32(rng(cfg_seed, STREAM_HC_PHI), (no, n * d), 1.0 / 128.0)
    g = rng(cfg_seed, STREAM_HC_BIAS)
    bias = normal_f32(g, (no,), 1.0)
    bias[2 * n:] = normal_f32(g, (n * n,), 0.5) + 4.0 * np.eye(n, dtype=np.float32).ravel()
    alpha = np.ones(3, dtype=np.float32)
    y = normal_f32(rng(cfg_seed, STREAM_HC_Y, variant), (T, d), 1.0)
    return X, phi, bias, alpha, y
