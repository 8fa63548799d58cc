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


# ---------------------------------------------------------------------------
# Phases 0 to 2 in the page's state, resumable ("The forward pass, in order",
# phases 0-2, with the header's tokenizer fields of "The resumable state").
#
# Readings (the library takes the same): a unit of tokenizing is phase 0
# whole; one character of phase 1, or the step that ends phase 1; one pair
# looked up in a merge scan, or the end of a scan, which applies the best
# merge or, when there is none, checks the context and ends phase 2.  The
# fields at 52-68 hold the next prompt byte (phase 1), the pair being looked
# up, the position, score key and token id of the best merge found in this
# scan (position 0xFFFFFFFF for none).  A prompt that does not fit is error
# 7 at the end of phase 2, the state left as it stood.

NONE = 0xFFFFFFFF


def init(cfg, prompt: bytes, max_tokens: int, temperature_q16: int, seed: int):
    """(error, a fresh state in the page's format at phase 0)."""
    context = cfg[6]
    if len(prompt) > 1024 or 0 in prompt or not 1 <= max_tokens <= context or \
            temperature_q16 > 16 * 65536:
        return 6, None
    P = layout(cfg, len(prompt), max_tokens)
    st = np.zeros(P["total"], dtype=np.uint8)
    hdr = bytearray(128)
    hdr[0:8] = TAG
    struct.pack_into("<I", hdr, 28, len(prompt))
    struct.pack_into("<I", hdr, 36, max_tokens)
    struct.pack_into("<I", hdr, 40, temperature_q16)
    struct.pack_into("<Q", hdr, 72, seed if seed else 0x9E3779B97F4A7C15)
    st[:128] = np.frombuffer(bytes(hdr), np.uint8)
    st[P["prompt"]: P["prompt"] + len(prompt)] = np.frombuffer(prompt, np.uint8)
    return 0, st


def tokenize_units(section0, cfg, st: np.ndarray, budget: int) -> int:
    """Runs up to `budget` units of phases 0-2; 0, or 7 (no fit), 3 (past them)."""
    v = T.Vocab(section0)
    pb, mx = _u32(st, 28), _u32(st, 36)
    P = layout(cfg, pb, mx)
    prompt = bytes(st[P["prompt"]: P["prompt"] + pb])
    ids = st[P["ids"]: P["ids"] + 4 * (pb + 2)].view(np.uint32)

    def get(off):
        return _u32(st, off)

    def put(off, val):
        st[off: off + 4] = np.frombuffer(struct.pack("<I", val), np.uint8)
    if get(8) > 2:
        return 3
    while budget > 0:
        budget -= 1
        phase, n = get(8), get(32)
        if phase == 0:
            ids[0] = 1
            n = 1
            if pb:
                sp = v.lookup(b" ")
                ids[1] = sp if sp >= 0 else ord(" ") + 3
                n = 2
            put(32, n); put(8, 1); put(52, 0)
        elif phase == 1:
            i = get(52)
            if i >= pb:
                put(8, 2); put(56, 0); put(60, NONE); put(64, 0); put(68, 0)
                continue
            ch = T.characters(prompt[i:])[0]
            t = v.lookup(ch)
            for tok in ([t] if t >= 0 else [b + 3 for b in ch]):
                ids[n] = tok
                n += 1
            put(32, n); put(52, i + len(ch))
        else:
            k = get(56)
            if k + 1 < n:
                t = v.lookup(v.pieces[ids[k]] + v.pieces[ids[k + 1]])
                if t >= 0 and (get(60) == NONE or v.score[t] > get(64)):
                    put(60, k); put(64, v.score[t]); put(68, t)
                put(56, k + 1)
                continue
            best = get(60)
            if best != NONE:
                ids[best] = get(68)
                ids[best + 1: n - 1] = ids[best + 2: n].copy()
                ids[n - 1] = 0
                put(32, n - 1); put(56, 0); put(60, NONE); put(64, 0); put(68, 0)
                continue
            if n + mx - 1 > cfg[6]:
                return 7
            put(56, 0); put(60, 0)
            put(8, 3); put(20, 0); put(24, int(ids[0]))
            return 0
    return 0
