"""Oracle of the tokenizer: phases 0 to 2 and the text of generated tokens.

Test infrastructure, like the rest of oracle/: only tests/,
__graft_entry__.smoke() and bench.py's CPU baseline use it; the library
never does.  Plain Python loops over small inputs (prompts of at most 1,024
bytes), written from "The inference core" page:

* "The forward pass, in order", phase 0: the ids start with the opening
  token (1), followed by the space token if the prompt is not empty;
* phase 1: each UTF-8 character is looked up as one string; one that is not
  in the vocabulary falls back to its bytes, each as id byte + 3;
* phase 2: repeatedly, among all neighbouring pairs whose joined string is a
  token, the best-scoring one is merged; when none is left, the ids plus max
  tokens have to fit in the context;
* "Sampling", its closing rules for text: a token contributes its bytes,
  except that a space at its start is dropped when it directly follows the
  opening token, a <0xXX> token stands for the single byte XX (two hex
  digits, either case), and tokens 1 and 2 contribute nothing.

Readings where the page is silent (the same ones the library takes):

* a character is a lead byte and the continuation bytes after it, at most
  four bytes in all (a continuation byte with no lead stands alone);
* among pairs of the highest score the leftmost merges;
* the pairs include the opening token's;
* a prompt has at most 1,024 bytes and no zero byte, and max tokens lies in
  1 to the context (else error 6); ids + max tokens - 1 above the context is
  error 7, as for a state;
* the space token is looked up like a character; without one, the space
  falls back to its byte token.

The tokenizer block (section zero, at the header's offset 88, length at 96)
is read here on its own terms: n, longest, score[n], start[n + 1],
sorted_ids[n], pool.
"""
from __future__ import annotations

import struct

INVALID_FORMAT, INVALID_PROMPT, CONTEXT_EXCEEDED = 2, 6, 7


class Vocab:
    def __init__(self, section0: bytes):
        s0 = bytes(section0)
        self.config = struct.unpack_from("<7I", s0, 8)
        off, length = struct.unpack_from("<QQ", s0, 88)
        if length == 0:
            raise ValueError("no tokenizer block")
        blk = s0[off:off + length]
        n, self.longest = struct.unpack_from("<II", blk, 0)
        p = 8
        self.score = list(struct.unpack_from(f"<{n}I", blk, p)); p += 4 * n
        start = struct.unpack_from(f"<{n + 1}I", blk, p); p += 4 * (n + 1)
        p += 4 * n  # the sorted ids: a lookup here is a dictionary
        pool = blk[p:]
        self.pieces = [pool[start[i]:start[i + 1]] for i in range(n)]
        self.index = {}
        for i, piece in enumerate(self.pieces):
            self.index.setdefault(piece, i)

    def lookup(self, b: bytes) -> int:
        return self.index.get(b, -1)


def characters(text: bytes):
    """The prompt's UTF-8 characters: a lead byte and up to three
    continuation bytes after it."""
    out = []
    i = 0
    while i < len(text):
        j = i + 1
        while j < len(text) and j - i < 4 and (text[j] & 0xC0) == 0x80:
            j += 1
        out.append(text[i:j])
        i = j
    return out


def encode(v: Vocab, prompt: bytes, max_tokens: int):
    """(error, ids) of phases 0 to 2."""
    context = v.config[6]
    if len(prompt) > 1024 or 0 in prompt or max_tokens < 1 or max_tokens > context:
        return INVALID_PROMPT, None
    ids = [1]
    if prompt:
        sp = v.lookup(b" ")
        ids.append(sp if sp >= 0 else ord(" ") + 3)
    for ch in characters(prompt):
        t = v.lookup(ch)
        if t >= 0:
            ids.append(t)
        else:
            ids.extend(b + 3 for b in ch)
    while True:
        best, where, best_id = None, -1, -1
        for i in range(len(ids) - 1):
            t = v.lookup(v.pieces[ids[i]] + v.pieces[ids[i + 1]])
            if t >= 0 and (best is None or v.score[t] > best):
                best, where, best_id = v.score[t], i, t
        if where < 0:
            break
        ids[where:where + 2] = [best_id]
    if len(ids) + max_tokens - 1 > context:
        return CONTEXT_EXCEEDED, None
    return 0, ids


def token_text(v: Vocab, prev: int, token: int) -> bytes:
    """The text a generated token adds after the token prev."""
    if token in (1, 2):
        return b""
    piece = v.pieces[token]
    if prev == 1 and piece[:1] == b" ":
        piece = piece[1:]
    hexd = b"0123456789ABCDEFabcdef"
    if (len(piece) == 6 and piece[:3] == b"<0x" and piece[5:] == b">"
            and piece[3] in hexd and piece[4] in hexd):
        return bytes([int(piece[3:5].decode(), 16)])
    return piece


def output_text(v: Vocab, prompt_ids, generated) -> bytes:
    """The text of generated tokens, the first one after the prompt's last id."""
    out, prev = [], int(prompt_ids[-1])
    for t in generated:
        out.append(token_text(v, prev, int(t)))
        prev = int(t)
    return b"".join(out)
