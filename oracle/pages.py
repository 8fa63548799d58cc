"""Oracle of the page's own state format (CURTAST2) and the way back.

Test infrastructure, like the rest of oracle/: only tests/ use it.  Written
from "The inference core" page, "The resumable state": a 128-byte header
(tag, phase, layer, row, position, token, prompt bytes, prompt tokens, max
tokens, temperature, generated, text bytes, five tokenizer fields, the
generator, the turn count, the largest score, the chosen entry, the pass,
the sum, the remainder, the attention stage and index) and the buffers in
the table's order, each 8-byte aligned, with cache positions
min(prompt bytes + max tokens + 1, context).

Readings (the same ones the library takes): the caches are
[layer][position][kv head * head + element]; after tokenizing the
tokenizer's next byte is the prompt's length and its other fields zero; a
frozen run has no page form.  The library's state is read through the
oracle's own layout (oracle.state_layout) and header offsets.
"""
from __future__ import annotations

import struct

import numpy as np

import oracle as O
from oracle import tokenizer as T

TAG = b"CURTAST2"


def a8(n: int) -> int:
    return (n + 7) // 8 * 8


def layout(cfg, prompt_bytes: int, max_tokens: int) -> dict:
    dim, hidden, layers, heads, kv_heads, vocab, context = cfg
    kvd = kv_heads * (dim // heads)
    cp = min(prompt_bytes + max_tokens + 1, context)
    L, o = {"cachepos": cp}, 128
    for name, size in (("prompt", prompt_bytes), ("ids", 4 * (prompt_bytes + 2)),
                       ("out", 4 * max_tokens), ("text", 128 * max_tokens),
                       ("x", 8 * dim), ("w1", 8 * dim), ("w2", 8 * dim), ("w3", 8 * dim),
                       ("gate", 8 * hidden), ("up", 8 * hidden), ("logits", 8 * vocab),
                       ("scores", 8 * cp), ("keys", 4 * layers * cp * kvd),
                       ("values", 4 * layers * cp * kvd)):
        L[name] = o
        o += a8(size)
    L["total"] = o
    return L


def _u32(b, off):
    return struct.unpack_from("<I", b, off)[0]


def export(section0, cfg, state: np.ndarray, prompt: bytes) -> np.ndarray:
    info = O.state_info(state)[1]
    n_ids, mx = info["n_ids"], info["max_tokens"]
    S = O.state_layout(cfg, n_ids, mx)
    P = layout(cfg, len(prompt), mx)
    dim, hidden, layers, heads, kv_heads, vocab, context = cfg
    hd = dim // heads
    out = np.zeros(P["total"], dtype=np.uint8)
    ids = state[S["ids"]: S["ids"] + 4 * n_ids].view(np.uint32)
    gen = state[S["out"]: S["out"] + 4 * info["generated"]].view(np.uint32)
    text = T.output_text(T.Vocab(section0), ids, gen)
    hdr = bytearray(128)
    hdr[0:8] = TAG
    for off, v in ((8, info["phase"]), (12, info["layer"]), (16, _u32(state, 16)),
                   (20, info["position"]), (24, info["token"]), (28, len(prompt)),
                   (32, n_ids), (36, mx), (40, info["temperature_q16"]),
                   (44, info["generated"]), (48, len(text)), (52, len(prompt))):
        struct.pack_into("<I", hdr, off, v)
    hdr[72:128] = bytes(state[72:128])
    out[:128] = np.frombuffer(bytes(hdr), np.uint8)
    out[P["prompt"]: P["prompt"] + len(prompt)] = np.frombuffer(prompt, np.uint8)
    out[P["ids"]: P["ids"] + 4 * n_ids] = state[S["ids"]: S["ids"] + 4 * n_ids]
    out[P["out"]: P["out"] + 4 * mx] = state[S["out"]: S["out"] + 4 * mx]
    out[P["text"]: P["text"] + len(text)] = np.frombuffer(text, np.uint8)
    for name, n in (("x", dim), ("w1", dim), ("w2", dim), ("w3", dim), ("gate", hidden),
                    ("up", hidden), ("logits", vocab), ("scores", S["cache_positions"])):
        out[P[name]: P[name] + 8 * n] = state[S[name]: S[name] + 8 * n]
    cs = S["cache_positions"]
    for name in ("keys", "values"):
        mine = state[S[name]: S[name] + 4 * layers * kv_heads * cs * hd].view(np.int32)
        mine = mine.reshape(layers, kv_heads, cs, hd)
        theirs = out[P[name]: P[name] + 4 * layers * P["cachepos"] * kv_heads * hd].view(np.int32)
        theirs = theirs.reshape(layers, P["cachepos"], kv_heads, hd)
        theirs[:, :cs] = mine.transpose(0, 2, 1, 3)
    return out


def import_(cfg, pages: np.ndarray) -> np.ndarray:
    prompt_bytes, n_ids, mx = _u32(pages, 28), _u32(pages, 32), _u32(pages, 36)
    P = layout(cfg, prompt_bytes, mx)
    S = O.state_layout(cfg, n_ids, mx)
    dim, hidden, layers, heads, kv_heads, vocab, context = cfg
    hd = dim // heads
    st = O.aligned_zeros(S["total"])
    st[0:8] = np.frombuffer(b"FPI8ST01", np.uint8)
    st[8:28] = pages[8:28]
    st[32:48] = pages[32:48]
    st[48:52] = np.frombuffer(struct.pack("<I", S["cache_positions"]), np.uint8)
    st[72:128] = pages[72:128]
    st[S["ids"]: S["ids"] + 4 * n_ids] = pages[P["ids"]: P["ids"] + 4 * n_ids]
    st[S["out"]: S["out"] + 4 * mx] = pages[P["out"]: P["out"] + 4 * mx]
    cs = S["cache_positions"]
    for name, n in (("x", dim), ("w1", dim), ("w2", dim), ("w3", dim), ("gate", hidden),
                    ("up", hidden), ("logits", vocab), ("scores", cs)):
        st[S[name]: S[name] + 8 * n] = pages[P[name]: P[name] + 8 * n]
    for name in ("keys", "values"):
        theirs = pages[P[name]: P[name] + 4 * layers * P["cachepos"] * kv_heads * hd]
        theirs = theirs.view(np.int32).reshape(layers, P["cachepos"], kv_heads, hd)
        mine = st[S[name]: S[name] + 4 * layers * kv_heads * cs * hd].view(np.int32)
        mine.reshape(layers, kv_heads, cs, hd)[:] = theirs[:, :cs].transpose(0, 2, 1, 3)
    return st
