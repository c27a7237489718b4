"""Seeded synthetic inputs for the microscaling-FP4 quantizer and GEMM.

This module holds the shapes and value distributions of the workloads and
nothing of the method's arithmetic: it draws numbers and rounds them to
bf16, and both the CPU oracle and the HIP path consume exactly these bytes.

The pages train and evaluate on ViT image data, LLM corpora of up to 200B
tokens and downstream suites, none of which are available here; tensors of
the same shapes with the distributions below stand in for them.

Recipe: every tensor draws from
``np.random.default_rng(np.random.SeedSequence(0, spawn_key=(cfg, tensor)))``,
in float32 (Student-t in float64, then float32), converted to bf16 with
round-to-nearest-even on the host.  "N(0, s)" means standard deviation s.
"""
from __future__ import annotations

import numpy as np


def rng_for(cfg: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(0, spawn_key=(cfg, tensor)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std: float, cfg: int, tensor: int) -> np.ndarray:
    g = rng_for(cfg, tensor)
    x = g.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(std)
    return f32_to_bf16_bits(x)


def student_t_bf16(shape, nu: float, cfg: int, tensor: int,
                   outlier_frac: float = 0.0, outlier_scale: float = 50.0) -> np.ndarray:
    """Student-t(nu) entries; optionally round(outlier_frac * cols) whole
    columns (channels), chosen without replacement, multiplied by outlier_scale."""
    g = rng_for(cfg, tensor)
    x = g.standard_t(nu, size=shape).astype(np.float32)
    if outlier_frac > 0.0:
        cols = shape[-1]
        n_out = int(round(outlier_frac * cols))
        ch = g.choice(cols, size=n_out, replace=False)
        x[..., ch] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


# Workload table.  Each entry: the tensors (name, shape, generator kwargs) and
# the format / rotation / rounding of the configuration.
CONFIGS = {
    1: dict(name="mx-rtn-256x256x1024", fmt="mx", hadamard=False,
            tensors={"X": ((256, 1024), dict(kind="normal", std=1.0)),
                     "W": ((256, 1024), dict(kind="normal", std=0.02))}),
    2: dict(name="nv-rtn-8192x4096x4096-outliers", fmt="nv", hadamard=False,
            tensors={"X": ((8192, 4096), dict(kind="t", nu=3.0, outlier_frac=0.01, outlier_scale=50.0)),
                     "W": ((4096, 4096), dict(kind="normal", std=0.02))}),
    3: dict(name="mx-hadamard-inference", fmt="mx", hadamard=True,
            tensors={"W_up": ((14336, 4096), dict(kind="normal", std=0.02)),
                     "W_down": ((4096, 14336), dict(kind="normal", std=0.02)),
                     "x_dec_up": ((16, 4096), dict(kind="t", nu=4.0)),
                     "x_pre_up": ((4096, 4096), dict(kind="t", nu=4.0)),
                     "x_dec_down": ((16, 14336), dict(kind="t", nu=4.0)),
                     "x_pre_down": ((4096, 14336), dict(kind="t", nu=4.0))}),
    4: dict(name="mx-vit-b16-train", fmt="mx", hadamard=False,
            tensors={"X1": ((50432, 768), dict(kind="normal", std=1.0)),
                     "W1": ((3072, 768), dict(kind="normal", std=0.02)),
                     "dY1": ((50432, 3072), dict(kind="normal", std=1e-3)),
                     "X2": ((50432, 3072), dict(kind="normal", std=1.0)),
                     "W2": ((768, 3072), dict(kind="normal", std=0.02)),
                     "dY2": ((50432, 768), dict(kind="normal", std=1e-3))}),
    5: dict(name="nv-7b-train", fmt="nv", hadamard=False,
            tensors={"X": ((16384, 4096), dict(kind="t", nu=3.0)),
                     "X_down": ((16384, 11008), dict(kind="t", nu=3.0)),
                     "W_qkv": ((12288, 4096), dict(kind="normal", std=0.02)),
                     "W_o": ((4096, 4096), dict(kind="normal", std=0.02)),
                     "W_gate": ((11008, 4096), dict(kind="normal", std=0.02)),
                     "W_up": ((11008, 4096), dict(kind="normal", std=0.02)),
                     "W_down": ((4096, 11008), dict(kind="normal", std=0.02)),
                     "dY_qkv": ((16384, 12288), dict(kind="normal", std=1e-3)),
                     "dY_o": ((16384, 4096), dict(kind="normal", std=1e-3)),
                     "dY_gate": ((16384, 11008), dict(kind="normal", std=1e-3)),
                     "dY_down": ((16384, 4096), dict(kind="normal", std=1e-3))}),
    # headline: M x N x K = 4096 x 14336 x 8192, MXFP4, RTN, no rotation
    0: dict(name="mx-rtn-4096x14336x8192", fmt="mx", hadamard=False,
            tensors={"A": ((4096, 8192), dict(kind="normal", std=1.0)),
                     "B": ((14336, 8192), dict(kind="normal", std=0.02))}),
}


def make_tensor(cfg: int, name: str, rows: int | None = None) -> np.ndarray:
    """bf16 bits of tensor `name` of configuration `cfg`.  `rows` keeps only the
    first rows of the full draw (the draw itself is always the full shape, so
    a prefix is identical to the same rows of the full tensor)."""
    spec = CONFIGS[cfg]
    names = list(spec["tensors"].keys())
    shape, kw = spec["tensors"][name]
    tensor_id = names.index(name)
    kw = dict(kw)
    kind = kw.pop("kind")
    if kind == "normal":
        x = normal_bf16(shape, kw["std"], cfg, tensor_id)
    else:
        x = student_t_bf16(shape, kw["nu"], cfg, tensor_id,
                           kw.get("outlier_frac", 0.0), kw.get("outlier_scale", 50.0))
    return x if rows is None else np.ascontiguousarray(x[:rows])


def small_normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """Small seeded N(0, std) bf16 tensor for unit and parity tests."""
    g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(99,)))
    return f32_to_bf16_bits(g.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def small_t_bf16(shape, nu: float, seed: int, outlier_frac: float = 0.0,
                 outlier_scale: float = 50.0) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(98,)))
    x = g.standard_t(nu, size=shape).astype(np.float32)
    if outlier_frac > 0.0:
        cols = shape[-1]
        ch = g.choice(cols, size=max(1, int(round(outlier_frac * cols))), replace=False)
        x[..., ch] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)
