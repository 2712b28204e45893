"""Seeded synthetic workloads for the SeedLM decompress-and-multiply path.

This module only draws random numbers and lists matrix shapes. It holds none of
the method's arithmetic (no LFSR, no decoding, no packing), so that the CPU
oracle and the HIP path can both consume the same inputs without sharing code.

Draw recipe, per (config id, matrix id), from one generator
``numpy.random.default_rng([config_id, matrix_id])``, in this order:

* seeds   uniform integers in [1, 65535]      shape (rows, nb)
* coeffs  uniform integers in [-8, 7]          shape (rows, nb, P)
* exps    uniform integers in [-12, -6]        shape (rows, nb)
* x       standard normal, cast to fp16 or fp32, shape (batch, cols)

with ``nb = ceil(cols / C)``.  The pages report that runtime does not depend on
the learned values (SeedLM, paperhub.cn OpenReview discussion, answer to the
question on speed after fine-tuning), so uniform records stand in for the
compressed Llama 2/3 weights, which are not available here.  The x draws come
from a second generator ``default_rng([config_id, matrix_id, 1 + batch_index])``
so that x can be drawn without first drawing the (large) record arrays.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "MatrixSpec",
    "ConfigSpec",
    "CONFIGS",
    "gen_records",
    "gen_x",
    "gen_gaussian_matrix",
]


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    rows: int  # M: output features
    cols: int  # N: input features (the reduction axis)


@dataclass(frozen=True)
class ConfigSpec:
    config_id: int
    name: str
    C: int
    P: int
    K: int
    x_dtype: str  # "f32" or "f16"
    batches: tuple
    matrices: tuple = field(default_factory=tuple)


def _llama(q, kv, hidden, inter):
    return (
        MatrixSpec("q", q, hidden),
        MatrixSpec("k", kv, hidden),
        MatrixSpec("v", kv, hidden),
        MatrixSpec("o", hidden, q),
        MatrixSpec("gate", inter, hidden),
        MatrixSpec("up", inter, hidden),
        MatrixSpec("down", hidden, inter),
    )


CONFIGS = {
    0: ConfigSpec(0, "single 512x512, 4-bit", 8, 3, 16, "f32", (1,),
                  (MatrixSpec("w", 512, 512),)),
    1: ConfigSpec(1, "single 2048x2048, 4-bit", 8, 3, 16, "f16", (1,),
                  (MatrixSpec("w", 2048, 2048),)),
    2: ConfigSpec(2, "Llama-2-7B layer, 4-bit", 8, 3, 16, "f16", (1,),
                  _llama(4096, 4096, 4096, 11008)),
    3: ConfigSpec(3, "Llama-3-8B layer, 3-bit", 12, 4, 16, "f16", (1, 4, 16),
                  _llama(4096, 1024, 4096, 14336)),
    4: ConfigSpec(4, "Llama-3-70B layer, 4-bit", 8, 3, 16, "f16", (1, 8),
                  _llama(8192, 1024, 8192, 28672)),
}


def gen_records(config_id: int, matrix_id: int, rows: int, cols: int, C: int, P: int):
    """Seeds (uint16), coefficients (int8) and exponents (int8) for one matrix."""
    nb = math.ceil(cols / C)
    rng = np.random.default_rng([config_id, matrix_id])
    seeds = rng.integers(1, 65536, size=(rows, nb), dtype=np.uint16)
    coeffs = rng.integers(-8, 8, size=(rows, nb, P), dtype=np.int8)
    exps = rng.integers(-12, -5, size=(rows, nb), dtype=np.int8)
    return seeds, coeffs, exps


def gen_x(config_id: int, matrix_id: int, batch: int, cols: int, dtype: str):
    """Activations x[batch][cols], N(0,1), cast to fp16 ("f16") or fp32 ("f32")."""
    out = np.empty((batch, cols), dtype=np.float16 if dtype == "f16" else np.float32)
    for b in range(batch):
        rng = np.random.default_rng([config_id, matrix_id, 1 + b])
        out[b] = rng.standard_normal(cols).astype(out.dtype)
    return out


def gen_gaussian_matrix(config_id: int, matrix_id: int, rows: int, cols: int):
    """A dense N(0,1) float64 matrix (the encoder self-check input)."""
    rng = np.random.default_rng([config_id, matrix_id])
    return rng.standard_normal((rows, cols))


def gen_bf16_weights(config_id: int, matrix_id: int, rows: int, cols: int, scale: float = 1.0):
    """Dense N(0, scale^2) weights rounded to bf16 (round to nearest even).

    Returns the raw bf16 bit patterns (uint16 [rows][cols]); LLM checkpoints hold
    their weights in this format, and it is the encoder's input type.
    """
    rng = np.random.default_rng([config_id, matrix_id, 7])
    return to_bf16_bits(rng.standard_normal((rows, cols)) * scale)


def to_bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns of float values (via fp32, round to nearest even; finite)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_float64(bits: np.ndarray) -> np.ndarray:
    """The float64 values of bf16 bit patterns (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
