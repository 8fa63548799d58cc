"""Synthetic weight artifacts ("blobs") in the curta-core weight format.

The pages fix only part of the artifact ("The inference core" page,
sections "One crate, three targets" and "The Rust API"): it opens with the
tag CURTAW01, section zero holds the configuration, the lookup tables, the
tokenizer and the metadata, the second u64 of the first section-table entry
is the length of section zero, and the matrices sit in further sections.
This module makes that layout concrete.  Every value is little-endian and
every offset counts from the start of the artifact.

Header (section zero starts at offset 0)::

    0    8 bytes   tag "CURTAW01"
    8    u32[7]    config: dim, hidden, layers, heads, kv_heads, vocab, context
    36   u32       section count S (section zero included)
    40   u32       matrix count, 2 + 7 * layers
    44   u32       one over the square root of the head size, Q24
    48   u64       offset of the exponential table, u32[4097] Q30
    56   u64       offset of the SiLU table, i32[4097] Q16
    64   u64       offset of the rotary cosines, i32[context][head/2] Q24
    72   u64       offset of the rotary sines, i32[context][head/2] Q24
    80   u64       offset of the normalization weights, i32 Q24:
                   [layers][2][dim] (before attention, before the
                   feed-forward), then the final [dim]
    88   u64       offset of the tokenizer block (layout in workloads/vocab.py)
    96   u64       length of the tokenizer block (0 for a vocabulary below 260)
    104  u64       offset of the matrix descriptors
    112  16 bytes  zero
    128  section table: S entries of {u64 offset, u64 length};
                   entry 0 is {0, length of section zero}

Matrix descriptor (32 bytes)::

    u32 kind, u32 layer, u32 rows, u32 cols, u32 section, u32 zero,
    u64 offset of the weight bytes inside the section

The section holds rows*cols weight bytes (each weight plus 128, row-major)
at that offset and, 8-aligned after them, rows u32 row scales (Q24).

Kinds: 0 embedding [vocab][dim], 1 query [dim][dim], 2 key [kv_dim][dim],
3 value [kv_dim][dim], 4 attention output [dim][dim], 5 gate [hidden][dim],
6 up [hidden][dim], 7 down [dim][hidden], 8 classifier [vocab][dim].

The tables are filled from their definitions here, as the pages' converter
would fill them at conversion: e^(-i/256) at Q30, silu(-16 + i/128) at Q16,
cos and sin of pos * 10000^(-2j/head) at Q24 and 1/sqrt(head) at Q24.

This module draws numbers and lays them out; it computes no step of the
forward pass.
"""
from __future__ import annotations

import hashlib
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import Shape
from . import vocab as _vocab

TAG = b"CURTAW01"
SECTION_TABLE = 128
DESCRIPTOR_BYTES = 32
TABLE_ENTRIES = 4097

KIND_EMBED, KIND_Q, KIND_K, KIND_V, KIND_O, KIND_GATE, KIND_UP, KIND_DOWN, KIND_CLS = range(9)
LAYER_KINDS = (KIND_Q, KIND_K, KIND_V, KIND_O, KIND_GATE, KIND_UP, KIND_DOWN)

SECTION_ALIGN = 256


def _a8(n: int) -> int:
    return (n + 7) & ~7


def _align(n: int, a: int) -> int:
    return (n + a - 1) // a * a


def matrix_shape(shape: Shape, kind: int):
    d, f, kvd, v = shape.dim, shape.hidden, shape.kv_dim, shape.vocab
    return {
        KIND_EMBED: (v, d), KIND_Q: (d, d), KIND_K: (kvd, d), KIND_V: (kvd, d),
        KIND_O: (d, d), KIND_GATE: (f, d), KIND_UP: (f, d), KIND_DOWN: (d, f),
        KIND_CLS: (v, d),
    }[kind]


def matrix_list(shape: Shape):
    """(kind, layer) of every matrix, in section order."""
    out = [(KIND_EMBED, 0)]
    for l in range(shape.layers):
        out += [(k, l) for k in LAYER_KINDS]
    out.append((KIND_CLS, 0))
    return out


# ----------------------------------------------------------------------------
# conversion-time tables
# ----------------------------------------------------------------------------

def exp_table() -> np.ndarray:
    i = np.arange(TABLE_ENTRIES, dtype=np.float64)
    return np.rint(np.exp(-i / 256.0) * 2.0 ** 30).astype(np.uint32)


def silu_table() -> np.ndarray:
    x = -16.0 + np.arange(TABLE_ENTRIES, dtype=np.float64) / 128.0
    return np.rint(x / (1.0 + np.exp(-x)) * 2.0 ** 16).astype(np.int32)


def rope_tables(shape: Shape):
    half = shape.head_size // 2
    pos = np.arange(shape.context, dtype=np.float64)[:, None]
    j = np.arange(half, dtype=np.float64)[None, :]
    ang = pos * np.power(10000.0, -2.0 * j / shape.head_size)
    cos = np.rint(np.cos(ang) * 2.0 ** 24).astype(np.int32)
    sin = np.rint(np.sin(ang) * 2.0 ** 24).astype(np.int32)
    return cos, sin


def inv_sqrt_head(shape: Shape) -> int:
    return int(round(2.0 ** 24 / math.sqrt(shape.head_size)))


# ----------------------------------------------------------------------------
# seeded weight bytes
# ----------------------------------------------------------------------------

_CHUNK = 1 << 24


def _normal20_lookup() -> np.ndarray:
    """u16 -> byte: inverse CDF of clip(128 + rint(N(0, 20)), 0, 255)."""
    from scipy.special import ndtri
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return np.clip(128.0 + np.rint(20.0 * ndtri(u)), 0, 255).astype(np.uint8)


_LOOKUP = None


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill_weight_bytes(out: np.ndarray, seed, dist: str = "normal20") -> None:
    """Fill a flat uint8 view with seeded weight bytes, chunk by chunk.

    Chunk c is drawn from default_rng([*seed, c]), so the bytes do not
    depend on how many threads fill them.
    """
    global _LOOKUP
    if dist == "normal20" and _LOOKUP is None:
        _LOOKUP = _normal20_lookup()
    n = out.size
    seed = list(seed)

    def job(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng(seed + [c])
        if dist == "normal20":
            u = g.integers(0, 65536, hi - lo, dtype=np.uint16)
            np.take(_LOOKUP, u, out=out[lo:hi])
        elif dist == "uniform":
            out[lo:hi] = g.integers(0, 256, hi - lo, dtype=np.uint8)
        else:
            raise ValueError(dist)

    chunks = (n + _CHUNK - 1) // _CHUNK
    if chunks <= 1:
        for c in range(chunks):
            job(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, range(chunks)))


def _row_scales(shape: Shape, kind: int, rows: int, cols: int, rng) -> np.ndarray:
    """Q24 row scales chosen so the activations stay well below 8.0."""
    q24 = float(1 << 24)
    spread = 20.0 * math.sqrt(cols)          # std of a row dot at unit input
    L = shape.layers
    if kind == KIND_EMBED:
        base = 0.5 * q24 / 20.0              # embedding RMS 0.5
    elif kind in (KIND_O, KIND_DOWN):
        base = q24 * 0.5 / math.sqrt(2.0 * L) / spread
    elif kind == KIND_CLS:
        base = q24 * 2.0 / spread
    else:
        base = q24 / spread                  # query, key, value, gate, up: RMS 1
    jitter = rng.uniform(0.9, 1.1, rows)
    return np.rint(base * jitter).astype(np.uint32)


# ----------------------------------------------------------------------------
# the artifact
# ----------------------------------------------------------------------------

@dataclass
class BlobLayout:
    section0_len: int
    total: int
    sections: list          # [(offset, length)] including section zero
    matrices: list          # [(kind, layer, rows, cols, section, offset_in_section)]
    offsets: dict           # name -> offset inside section zero


def plan(shape: Shape, tok_len: int | None = None) -> BlobLayout:
    n_mat = 2 + 7 * shape.layers
    n_sec = 1 + n_mat
    half = shape.head_size // 2
    o = SECTION_TABLE + 16 * n_sec
    offs = {}
    o = _a8(o); offs["exp"] = o; o += 4 * TABLE_ENTRIES
    o = _a8(o); offs["silu"] = o; o += 4 * TABLE_ENTRIES
    o = _a8(o); offs["cos"] = o; o += 4 * shape.context * half
    o = _a8(o); offs["sin"] = o; o += 4 * shape.context * half
    o = _a8(o); offs["norm"] = o; o += 4 * (2 * shape.layers + 1) * shape.dim
    o = _a8(o); offs["tok"] = o
    o += _vocab.block_len(shape.vocab) if tok_len is None else tok_len
    o = _a8(o); offs["desc"] = o; o += DESCRIPTOR_BYTES * n_mat
    s0 = _a8(o)
    sections = [(0, s0)]
    mats = []
    cur = _align(s0, SECTION_ALIGN)
    for si, (kind, layer) in enumerate(matrix_list(shape), start=1):
        rows, cols = matrix_shape(shape, kind)
        length = _a8(rows * cols) + 4 * rows
        sections.append((cur, length))
        mats.append((kind, layer, rows, cols, si, 0))
        cur = _align(cur + length, SECTION_ALIGN)
    return BlobLayout(s0, cur, sections, mats, offs)


def build_blob(shape: Shape, seed: int, dist: str = "normal20",
               tables: dict | None = None, tok: bytes | None = None) -> np.ndarray:
    """The whole artifact as one uint8 array.

    `tables` may override "exp", "silu", "cos", "sin", "norm" or "inv" (used
    by tests that need special tables, for instance an identity table), and
    `tok` the tokenizer block (bytes; empty for none).
    """
    tok = _vocab.block_bytes(shape.vocab) if tok is None else bytes(tok)
    lay = plan(shape, len(tok))
    blob = np.zeros(lay.total, dtype=np.uint8)
    hdr = blob[:SECTION_TABLE]
    hdr[:8] = np.frombuffer(TAG, dtype=np.uint8)
    tables = dict(tables or {})
    inv = tables.get("inv", inv_sqrt_head(shape))

    def put(off, arr):
        b = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        blob[off:off + b.size] = b

    put(8, np.array(shape.as_tuple(), dtype=np.uint32))
    put(36, np.array([len(lay.sections), len(lay.matrices), inv], dtype=np.uint32))
    put(48, np.array([lay.offsets["exp"], lay.offsets["silu"], lay.offsets["cos"],
                      lay.offsets["sin"], lay.offsets["norm"], lay.offsets["tok"],
                      len(tok), lay.offsets["desc"]], dtype=np.uint64))
    put(SECTION_TABLE, np.array(lay.sections, dtype=np.uint64).reshape(-1))

    cos, sin = rope_tables(shape)
    put(lay.offsets["exp"], np.asarray(tables.get("exp", exp_table()), dtype=np.uint32))
    put(lay.offsets["silu"], np.asarray(tables.get("silu", silu_table()), dtype=np.int32))
    put(lay.offsets["cos"], np.asarray(tables.get("cos", cos), dtype=np.int32))
    put(lay.offsets["sin"], np.asarray(tables.get("sin", sin), dtype=np.int32))
    if "norm" in tables:
        norm = np.asarray(tables["norm"], dtype=np.int32)
    else:
        g = np.random.default_rng([seed, 0x6E6F726D])
        norm = np.rint((1.0 + 0.02 * g.standard_normal((2 * shape.layers + 1) * shape.dim))
                       * 2.0 ** 24).astype(np.int32)
    put(lay.offsets["norm"], norm)
    if tok:
        put(lay.offsets["tok"], np.frombuffer(tok, dtype=np.uint8))

    desc = np.zeros((len(lay.matrices), 8), dtype=np.uint32)
    for i, (kind, layer, rows, cols, sec, off) in enumerate(lay.matrices):
        desc[i, :6] = (kind, layer, rows, cols, sec, 0)
        desc[i, 6] = off & 0xFFFFFFFF
        desc[i, 7] = off >> 32
    put(lay.offsets["desc"], desc)

    for (kind, layer, rows, cols, sec, off) in lay.matrices:
        base, _ = lay.sections[sec]
        w = blob[base + off: base + off + rows * cols]
        fill_weight_bytes(w, [seed, sec], dist)
        g = np.random.default_rng([seed, sec, 0x7363616C])
        s = _row_scales(shape, kind, rows, cols, g)
        put(base + off + _a8(rows * cols), s)
    return blob


def sha256(blob: np.ndarray) -> str:
    return hashlib.sha256(memoryview(blob)).hexdigest()


def section_zero(blob: np.ndarray) -> np.ndarray:
    n = int(blob[SECTION_TABLE + 8: SECTION_TABLE + 16].view(np.uint64)[0])
    return blob[:n]


def matrix_view(blob: np.ndarray, shape: Shape, kind: int, layer: int = 0):
    """(weights [rows][cols] uint8, scales [rows] uint32) views into a blob."""
    lay = plan(shape, int(blob[96:104].view(np.uint64)[0]))
    for (k, l, rows, cols, sec, off) in lay.matrices:
        if k == kind and l == layer:
            base = lay.sections[sec][0] + off
            w = blob[base: base + rows * cols].reshape(rows, cols)
            s = blob[base + _a8(rows * cols): base + _a8(rows * cols) + 4 * rows].view(np.uint32)
            return w, s
    raise KeyError((kind, layer))
