"""A synthetic tokenizer vocabulary for section zero of the artifact.

The pages' models ship a llama2.c tokenizer (one byte string and one score
per token id) that the converter stores in section zero ("The inference
core" page, "The forward pass, in order", phases 0 to 2, and "Tokenizing"
under "Compute costs").  None of those vocabularies is here, so this module
draws one with the same structure from a fixed seed:

* ids 0, 1, 2: the unknown, opening and closing tokens (a vocabulary of
  fewer than 260 tokens gets no block: it cannot hold the byte tokens);
* ids 3 to 258: the 256 byte tokens, written ``<0xXX>``;
* then single characters (ASCII letters, digits, punctuation, the space and
  a few multi-byte UTF-8 characters), as many as the vocabulary holds;
* then merged tokens, each the concatenation of two earlier non-special
  tokens, with scores that mostly fall in the order the merges were drawn
  and now and then repeat the previous score (ties).

Block layout (little-endian, at the offset the artifact header gives)::

    u32 n (the vocabulary size), u32 the longest token in bytes
    u32 score[n]           merge priority; the higher merges first
    u32 start[n + 1]       token i is pool[start[i] : start[i + 1]]
    u32 sorted_ids[n]      ids in the byte order of their strings (shorter
                           first where one is a prefix of the other)
    pool bytes, then zeros up to a multiple of 8

This module draws and lays out data; it computes no step of tokenizing.
"""
from __future__ import annotations

import functools

import numpy as np

SPECIAL = (b"<unk>", b"<s>", b"</s>")
VOCAB_SEED = 0x766F63616200
MAX_PIECE = 16

_CHARS = ([bytes([c]) for c in b" etaoinshrdlcumwfgypbvkjxqzETAOINSHRDLCUMWFGYPBVKJXQZ"]
          + [bytes([c]) for c in b".,!?';:-0123456789()\n"]
          + [s.encode() for s in ("é", "ü", "ñ", "中", "日")])


@functools.lru_cache(maxsize=8)
def build_vocab(n: int, seed: int = VOCAB_SEED):
    """(pieces, scores) of a vocabulary of n tokens; None below 260 tokens,
    which cannot hold the 256 byte tokens and a character."""
    if n < 260:
        return None
    rng = np.random.default_rng(seed)
    pieces = list(SPECIAL) + [b"<0x%02X>" % i for i in range(256)]
    scores = [0] * len(pieces)
    chars = []
    for ch in _CHARS:
        if len(pieces) >= n:
            break
        chars.append(len(pieces))
        pieces.append(ch)
        scores.append(0)
    # characters drawn by frequency (earlier in the list is more frequent),
    # or an earlier merged token
    cw = np.array([1.0 / (1 + k) for k in range(len(chars))])
    cw /= cw.sum()
    merged_ids = []
    have = set(pieces)
    score = 1 << 30
    tries = 0

    def draw():
        if merged_ids and rng.random() < 0.4:
            return merged_ids[int(rng.integers(0, len(merged_ids)))]
        return chars[int(rng.choice(len(chars), p=cw))]
    while len(pieces) < n:
        tries += 1
        if tries > 100 * n:
            raise RuntimeError("vocabulary generator stalled")
        merged = pieces[draw()] + pieces[draw()]
        if len(merged) > MAX_PIECE or merged in have:
            continue
        if rng.random() > 0.02:
            score -= int(rng.integers(1, 1000))
        merged_ids.append(len(pieces))
        pieces.append(merged)
        scores.append(score)
        have.add(merged)
    return tuple(pieces), tuple(scores)


@functools.lru_cache(maxsize=8)
def block_bytes(n: int) -> bytes:
    """The tokenizer block of the vocabulary of n tokens (empty below 260)."""
    v = build_vocab(n)
    if v is None:
        return b""
    return block_from(*v)


def block_from(pieces, scores) -> bytes:
    """The tokenizer block of a given vocabulary (pieces: byte strings)."""
    n = len(pieces)
    start = np.zeros(n + 1, dtype=np.uint32)
    start[1:] = np.cumsum([len(p) for p in pieces])
    order = sorted(range(n), key=lambda i: pieces[i])
    body = (np.array([n, max(len(p) for p in pieces)], dtype=np.uint32).tobytes()
            + np.array(scores, dtype=np.uint32).tobytes() + start.tobytes()
            + np.array(order, dtype=np.uint32).tobytes() + b"".join(pieces))
    return body + bytes(-len(body) % 8)


def block_len(n: int) -> int:
    return len(block_bytes(n))


def sample_text(n_chars: int, seed: int, extra: bool = True) -> bytes:
    """Seeded prompt text: words of the vocabulary's characters and spaces,
    with characters outside it (tab, sharp s, an emoji) when `extra`."""
    rng = np.random.default_rng(seed)
    chars = [c for c in _CHARS if c != b"\n"]
    if extra:
        chars += ["\t".encode(), "ß".encode(), "😀".encode()]
    out = []
    for _ in range(n_chars):
        k = int(rng.integers(0, len(chars)))
        out.append(chars[min(k, int(rng.integers(0, len(chars))))])
    return b"".join(out)
