"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
benchmark: model shapes, weight artifacts, prompt ids and the operands of
the standalone matrix-row sweep.

Nothing here computes a step of the fixed-point forward pass; the module
only draws numbers from seeded generators and lays them out.
"""
from __future__ import annotations

import numpy as np

from .configs import (Shape, Workload, TINY, M1B, M7B, LONG8K, SMALL_SHAPES,
                      ROW_SWEEP_ROWS, ROW_SWEEP_COLS, ROW_SWEEP_BATCHES,
                      ROW_SWEEP_SEED, by_name)
from . import blob

__all__ = ["Shape", "Workload", "TINY", "M1B", "M7B", "LONG8K", "SMALL_SHAPES",
           "ROW_SWEEP_ROWS", "ROW_SWEEP_COLS", "ROW_SWEEP_BATCHES",
           "ROW_SWEEP_SEED", "by_name", "blob", "prompt_ids", "row_operands"]


def prompt_ids(vocab: int, n: int, seed: int, run: int) -> np.ndarray:
    """Prompt ids of one run: uniform in [3, vocab), so no id is one of the
    first three (unknown, opening and closing tokens in llama2.c vocabularies)."""
    g = np.random.default_rng([seed, run])
    lo = 3 if vocab > 3 else 0
    return g.integers(lo, vocab, n, dtype=np.int64).astype(np.uint32)


def row_operands(rows: int, cols: int, batch: int, seed: int,
                 x_std: float = 2.0, scale_lo: int = 1 << 14, scale_hi: int = 1 << 18):
    """Weight bytes uniform in [0, 255], Q24 scales uniform in
    [scale_lo, scale_hi], Q16 inputs round(2^16 * N(0, x_std))."""
    W = np.empty(rows * cols, dtype=np.uint8)
    blob.fill_weight_bytes(W, [seed, 1], "uniform")
    g = np.random.default_rng([seed, 2])
    s = g.integers(scale_lo, scale_hi, rows, endpoint=True, dtype=np.int64).astype(np.uint32)
    x = np.rint(g.standard_normal((batch, cols)) * x_std * 65536.0).astype(np.int64)
    return W.reshape(rows, cols), s, x


def adversarial_row_inputs(batch: int, cols: int, seed: int) -> np.ndarray:
    """i64 inputs that exercise every limb of a 64-bit word: extremes,
    powers of two and their neighbours, and random 64-bit patterns."""
    g = np.random.default_rng([seed, 3])
    specials = np.array([0, 1, -1, 2**62, -2**62, 2**63 - 1, -2**63, 2**31 - 1,
                         -2**31, 2**23, -2**23, 2**23 - 1, -2**23 - 1, 8421504,
                         -8421505, 8421377, 8421378, 127, 128, -128, -129, 255, 256],
                        dtype=np.int64)
    x = g.integers(-2**63, 2**63 - 1, (batch, cols), dtype=np.int64, endpoint=True)
    pick = g.random((batch, cols)) < 0.5
    x[pick] = g.choice(specials, int(pick.sum()))
    return x
