"""Oracle of the compute units the turn planner charges for one position.

Test infrastructure, like the rest of oracle/: only tests/ use it.  Written
from "The inference core" page: "The turn planner" (each chunk of work adds
160 units; a turn adds 18,000) and "Compute costs" (the tables for matrices,
vector operations, attention stages and sampling).  d is the dimension, h
the hidden dimension, n a matrix's column count, q the head size and p the
positions so far (position + 1).

Readings (the library takes the same):

* a position's phases are charged as whole chunks: one chunk per matrix of
  a layer, one per stage of each head's attention, one per sampling pass and
  one per vector operation; each adds its 160.  Where a turn boundary splits
  a chunk the planner charges the rest as a new chunk (its setup and 160
  again); those extra charges, and the 18,000 of each turn, depend on where
  turns end and are not part of this function;
* at a temperature above zero sampling makes three passes (maximum, sum,
  draw), each a chunk with its setup, and each pass that ends adds the
  finishing charge of 4,000.  The page prints figures at temperature zero
  only, so this case is parity unpinned;
* phases 17 to 19 run only at positions that generate a token.
"""
from __future__ import annotations

PHASES = ("embed", "norm1", "q", "k", "v", "rotary", "attention", "o", "norm2", "gate", "up",
          "silu", "down", "residual", "fnorm", "classifier", "sampling")
CHUNK = 160


def matrix(rows: int, n: int, cache: bool = False) -> int:
    """One matrix as one chunk: its setup (summing the input vector) and every row."""
    row = 37 * (n // 8) + 8 * (n % 8) + (42 if cache else 34)
    return 6 * n + 350 + rows * row + CHUNK


def attention_head(q: int, p: int) -> int:
    """The four stages of one head, each a chunk: setup plus per-unit charges."""
    scores = 100 + p * (53 * (q // 8) + 11 * (q % 8) + 25)
    exps = 80 + p * 23
    norm = 60 + p * 8
    values = 60 + q * (11 * p + 32)
    return scores + exps + norm + values + 4 * CHUNK


def sampling(vocab: int, temperature_q16: int) -> int:
    per_entry = (11,) if temperature_q16 == 0 else (11, 36, 42)
    return sum(350 + vocab * e + 4000 + CHUNK for e in per_entry)


def position_charges(cfg, position: int, generating: bool, temperature_q16: int = 0) -> dict:
    """Phase name -> compute units for one position, summed over layers."""
    d, h, layers, heads, kv_heads, vocab, context = cfg
    q = d // heads
    kvd = kv_heads * q
    p = position + 1
    out = dict.fromkeys(PHASES, 0)
    out["embed"] = 16 * d + 512 + CHUNK
    for _ in range(layers):
        out["norm1"] += 48 * d + 1500 + CHUNK
        out["q"] += matrix(d, d)
        out["k"] += matrix(kvd, d, cache=True)
        out["v"] += matrix(kvd, d, cache=True)
        out["rotary"] += 48 * d + 512 + CHUNK
        out["attention"] += heads * attention_head(q, p)
        out["o"] += matrix(d, d)
        out["norm2"] += 56 * d + 1500 + CHUNK
        out["gate"] += matrix(h, d)
        out["up"] += matrix(h, d)
        out["silu"] += 24 * h + 512 + CHUNK
        out["down"] += matrix(d, h)
        out["residual"] += 8 * d + 128 + CHUNK
    if generating:
        out["fnorm"] = 48 * d + 1500 + CHUNK
        out["classifier"] = matrix(vocab, d)
        out["sampling"] = sampling(vocab, temperature_q16)
    return out


def split_setup(phase: str, cfg) -> tuple:
    """The charges a turn boundary adds when it splits a chunk of this phase
    (the setup and 160 again); several for attention, one per stage."""
    d, h, layers, heads, kv_heads, vocab, context = cfg
    n = h if phase == "down" else d
    if phase in ("q", "k", "v", "o", "gate", "up", "down", "classifier"):
        return (6 * n + 350 + CHUNK,)
    if phase == "attention":
        return (100 + CHUNK, 80 + CHUNK, 60 + CHUNK)
    if phase == "sampling":
        return (350 + CHUNK,)
    return ()
