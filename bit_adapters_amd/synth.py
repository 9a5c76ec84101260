"""Seeded synthetic inputs for the double-binary factorized linear layer.

This module only draws random numbers and rounds them to the storage types
(fp16 scales, bf16 / fp16 / int8 activations, bf16 base weights, int8 +-1
signs).  It holds none of the layer's arithmetic, so that both the fp64
oracle and the HIP path can consume the very same inputs.

Every tensor comes from its own numpy PCG64 stream,
``default_rng([0xDBF, config, tensor, term, variant])``, so a tensor does not
change when another one is added or resized.  Activations are drawn for the
largest token count of a configuration and sliced by prefix, so the token
sweeps are nested.

The five layer configurations follow the shapes the DBF and LoRDBA pages
work with (Llama-shaped 4096x4096 projections, the 11008x4096 MLP
up-projection, a prefill-sized 8192x8192 layer) and the distributions stated
for each of them.
"""
from __future__ import annotations

import numpy as np

TENSOR_X, TENSOR_W0, TENSOR_B1, TENSOR_B2 = 0, 1, 2, 3
TENSOR_ALPHA, TENSOR_BETA, TENSOR_GAMMA, TENSOR_XI8 = 4, 5, 6, 7
TENSOR_SIGNS_GENERIC = 8
TENSOR_WBOOL, TENSOR_SIN, TENSOR_SOUT = 9, 10, 11

# Shapes: N output features, M input features, R inner rank, L terms, and the
# token counts each configuration is run at.
CONFIGS = {
    1: dict(name="dbf-512-r256", N=512, M=512, R=256, L=1, T=(1,),
            scales="uniform", lo=0.5, hi=1.5, x="f16"),
    2: dict(name="dbf-4096-r2048", N=4096, M=4096, R=2048, L=1, T=(1, 4, 16),
            scales="absnormal", x="bf16"),
    3: dict(name="lordba-4096", N=4096, M=4096, R=None, L=1, T=(1, 4, 16),
            scales="uniform", lo=0.001, hi=0.01, x="bf16", base=True,
            ranks=(16, 64)),
    4: dict(name="mbok-11008x4096-r2048-l3", N=11008, M=4096, R=2048, L=3,
            T=(1, 8, 64, 256), scales="decay", decay=(1.0, 0.5, 0.25),
            lo=0.5, hi=1.5, x="bf16"),
    5: dict(name="dbf-8192-r6144", N=8192, M=8192, R=6144, L=1, T=(4096,),
            scales="absnormal", x="bf16"),
}


# Boolean-kernel layers of the Multi-Boolean form: K full N x M sign matrices,
# each with a rank-one pair of fp16 scales (s_out [N], s_in [M]).  The
# shapes are the Llama-7B 4096 x 4096 projection with K = 2 and the
# 11008 x 4096 MLP up-projection with K = 3 (the page finds 2 to 4 kernels
# enough).  The scales stand in for a successive SVID of an N(0, 0.02^2)
# weight: near 0.12 on each side of the first kernel (sqrt of E|W| = 0.016),
# each later kernel x0.6, with +-20% spread, positive (a leading singular
# pair of a nonnegative matrix).
BOOL_CONFIGS = {
    6: dict(name="mbok-svid-4096-k2", N=4096, M=4096, K=2, T=(1, 4, 16, 256), x="bf16"),
    7: dict(name="mbok-svid-11008x4096-k3", N=11008, M=4096, K=3, T=(1, 8, 64),
            x="bf16"),
}


def rng(config: int, tensor: int, term: int = 0, variant: int = 0):
    return np.random.default_rng([0xDBF, int(config), int(tensor), int(term),
                                  int(variant)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def signs(g: np.random.Generator, shape) -> np.ndarray:
    """i.i.d. +-1 signs with p = 0.5, as int8."""
    return (g.integers(0, 2, size=shape, dtype=np.int8) * 2 - 1).astype(np.int8)


def _scales(cfg: dict, config: int, tensor: int, term: int, n: int,
            variant: int) -> np.ndarray:
    g = rng(config, tensor, term, variant)
    kind = cfg["scales"]
    if kind == "uniform":
        v = g.uniform(cfg["lo"], cfg["hi"], n)
    elif kind == "absnormal":
        v = np.abs(g.standard_normal(n)) * 0.02 + 0.01
    elif kind == "decay":
        v = cfg["decay"][term] * g.uniform(cfg["lo"], cfg["hi"], n)
    else:
        raise ValueError(kind)
    return v.astype(np.float16)


def make_layer(config: int, R: int | None = None) -> dict:
    """The layer of a configuration: per-term int8 signs and fp16 scales, plus
    the bf16 base weight (uint16 bit patterns) in adapter configurations."""
    cfg = CONFIGS[config]
    N, M = cfg["N"], cfg["M"]
    if cfg["R"] is not None:
        R = cfg["R"]
    elif R is None:
        raise ValueError("configuration %d needs a rank" % config)
    variant = R if cfg["R"] is None else 0
    terms = []
    for i in range(cfg["L"]):
        terms.append(dict(
            b1=signs(rng(config, TENSOR_B1, i, variant), (N, R)),
            b2=signs(rng(config, TENSOR_B2, i, variant), (R, M)),
            alpha=_scales(cfg, config, TENSOR_ALPHA, i, N, variant),
            beta=_scales(cfg, config, TENSOR_BETA, i, R, variant),
            gamma=_scales(cfg, config, TENSOR_GAMMA, i, M, variant),
        ))
    layer = dict(config=config, N=N, M=M, R=R, terms=terms, w0=None)
    if cfg.get("base"):
        w = rng(config, TENSOR_W0, 0, variant).standard_normal(
            (N, M), dtype=np.float32) * np.float32(0.02)
        layer["w0"] = f32_to_bf16_bits(w)
    return layer


def make_x(config: int, T: int, kind: str | None = None) -> np.ndarray:
    """Activations [T x M]: bf16 bit patterns (uint16), fp16, or int8 in
    [-127, 127].  Drawn for the largest T of the configuration, sliced by
    prefix."""
    cfg = CONFIGS[config] if config in CONFIGS else BOOL_CONFIGS[config]
    M = cfg["M"]
    kind = kind or cfg["x"]
    tmax = max(max(cfg["T"]), T)
    if kind == "i8":
        g = rng(config, TENSOR_XI8)
        return g.integers(-127, 128, size=(tmax, M), dtype=np.int8)[:T].copy()
    g = rng(config, TENSOR_X)
    v = g.standard_normal((tmax, M), dtype=np.float32)[:T]
    if kind == "f16":
        return v.astype(np.float16)
    if kind == "bf16":
        return f32_to_bf16_bits(v)
    raise ValueError(kind)


def _bool_scale(g: np.random.Generator, k: int, n: int) -> np.ndarray:
    return (0.12 * 0.6 ** k * g.uniform(0.8, 1.2, n)).astype(np.float16)


def make_bool_layer(config: int) -> dict:
    """Boolean kernels of a configuration: int8 signs w [N x M] and fp16
    scales s_in [M], s_out [N] per kernel."""
    cfg = BOOL_CONFIGS[config]
    N, M = cfg["N"], cfg["M"]
    kernels = [dict(w=signs(rng(config, TENSOR_WBOOL, k), (N, M)),
                    s_in=_bool_scale(rng(config, TENSOR_SIN, k), k, M),
                    s_out=_bool_scale(rng(config, TENSOR_SOUT, k), k, N))
               for k in range(cfg["K"])]
    return dict(config=config, N=N, M=M, kernels=kernels)


def make_custom_bool(N: int, M: int, K: int, T: int, seed: int,
                     x_kind: str = "bf16") -> tuple[dict, np.ndarray]:
    """Boolean kernels and activations of arbitrary shape (edge cases)."""
    kernels = []
    for k in range(K):
        g = np.random.default_rng([0xDBF, 103, seed, k, N, M])
        kernels.append(dict(w=signs(g, (N, M)), s_in=_bool_scale(g, k, M),
                            s_out=_bool_scale(g, k, N)))
    g = np.random.default_rng([0xDBF, 104, seed, N, M, T])
    v = g.standard_normal((T, M), dtype=np.float32)
    x = v.astype(np.float16) if x_kind == "f16" else f32_to_bf16_bits(v)
    return dict(config=0, N=N, M=M, kernels=kernels), x


def make_custom(N: int, M: int, R: int, L: int, T: int, seed: int,
                scale_lo: float = 0.5, scale_hi: float = 1.5,
                x_kind: str = "bf16", base: bool = False) -> tuple[dict, np.ndarray]:
    """A layer and activations of arbitrary shape, for odd-shape and edge-case
    tests.  Scales are fp16 uniform[scale_lo, scale_hi]."""
    terms = []
    for i in range(L):
        g = np.random.default_rng([0xDBF, 100, seed, i, N, M, R])
        terms.append(dict(
            b1=signs(g, (N, R)), b2=signs(g, (R, M)),
            alpha=g.uniform(scale_lo, scale_hi, N).astype(np.float16),
            beta=g.uniform(scale_lo, scale_hi, R).astype(np.float16),
            gamma=g.uniform(scale_lo, scale_hi, M).astype(np.float16)))
    layer = dict(config=0, N=N, M=M, R=R, terms=terms, w0=None)
    g = np.random.default_rng([0xDBF, 101, seed, N, M, R, T])
    if base:
        layer["w0"] = f32_to_bf16_bits(
            g.standard_normal((N, M), dtype=np.float32) * np.float32(0.02))
    if x_kind == "i8":
        x = g.integers(-127, 128, size=(T, M), dtype=np.int8)
    else:
        v = g.standard_normal((T, M), dtype=np.float32)
        x = v.astype(np.float16) if x_kind == "f16" else f32_to_bf16_bits(v)
    return layer, x


def random_values(rows: int, K: int, seed: int, kind: str = "f32") -> np.ndarray:
    """Values whose signs are to be packed: N(0,1) in the requested storage
    type, with some exact zeros and negative zeros mixed in."""
    g = np.random.default_rng([0xDBF, 102, seed, rows, K])
    v = g.standard_normal((rows, K), dtype=np.float32)
    z = g.random((rows, K)) < 0.02
    v[z] = 0.0
    nz = g.random((rows, K)) < 0.02
    v[nz] = -0.0
    if kind == "f32":
        return v
    if kind == "f16":
        return v.astype(np.float16)
    if kind == "bf16":
        return f32_to_bf16_bits(v)
    if kind == "i8":
        return np.clip(np.round(v * 40), -127, 127).astype(np.int8)
    raise ValueError(kind)
