"""The tokenizer of section zero (phases 0 to 2, and the text of generated
tokens), CPU only: the oracle against a vocabulary worked by hand and
against properties of the rules, and the library's host tokenizer against
the oracle.  Sections cited are those of "The inference core" page.
"""
import ast
import os

import numpy as np
import pytest

import oracle as O
from oracle import tokenizer as T
import workloads as W
from workloads import blob as Bl
from workloads import vocab as V
from fixed_point_int8_amd import binding as B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tokenizer_example.txt")


def read_golden():
    vocab, enc, text = {}, [], []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, rest = line.split(" ", 1)
        if kind == "vocab":
            i, sc, piece = rest.split(" ", 2)
            vocab[int(i)] = (int(sc), ast.literal_eval(piece))
        elif kind == "encode":
            end = rest.index("' ") + 1 if "' " in rest else len(rest)
            prompt = ast.literal_eval(rest[:end])
            enc.append((prompt, [int(x) for x in rest[end:].split()]))
        else:
            prev, tok, hx = rest.split()
            text.append((int(prev), int(tok), b"" if hx == "-" else bytes.fromhex(hx)))
    return vocab, enc, text


def hand_blob():
    vocab, enc, text = read_golden()
    pieces = [b"<unk>", b"<s>", b"</s>"] + [b"<0x%02X>" % i for i in range(256)]
    scores = [0] * len(pieces)
    for i in range(259, 300):
        sc, piece = vocab.get(i, (0, b"~%02d" % (i - 273)))
        pieces.append(piece)
        scores.append(sc)
    shape = W.SMALL_SHAPES["gqa"]
    assert shape.vocab == 300
    return Bl.build_blob(shape, 60, tok=V.block_from(pieces, scores)), enc, text


def test_hand_example_oracle():
    blob, enc, text = hand_blob()
    v = T.Vocab(Bl.section_zero(blob))
    for prompt, ids in enc:
        assert T.encode(v, prompt, 4) == (0, ids), prompt
    for prev, tok, want in text:
        assert T.token_text(v, prev, tok) == want, (prev, tok)


def test_hand_example_library():
    blob, enc, text = hand_blob()
    s0 = Bl.section_zero(blob)
    for prompt, ids in enc:
        e, got = B.fpi8_tokenize(s0, prompt, 4)
        assert e == 0 and list(got) == ids, prompt
    for prev, tok, want in text:
        assert B.fpi8_token_text(s0, prev, tok) == (0, want), (prev, tok)


@pytest.mark.parametrize("n", [512, 2048, 32000])
def test_rules_hold_on_synthetic_vocabularies(n):
    # After phase 2 no adjacent pair joins into a token (checked pair by
    # pair); characters without a token are their bytes + 3; and the texts
    # of the prompt's tokens after the opening one give the prompt back (the
    # leading-space rule takes off the space phase 0 put in).
    shape = W.Shape(64, 96, 1, 4, 4, n, 2048)
    v = T.Vocab(Bl.section_zero(Bl.build_blob(shape, 61)))
    for seed in range(12):
        prompt = V.sample_text(int(np.random.default_rng(seed).integers(0, 200)), seed)
        e, ids = T.encode(v, prompt, 1)
        assert e == 0
        assert ids[0] == 1
        for a, b in zip(ids, ids[1:]):
            assert v.lookup(v.pieces[a] + v.pieces[b]) < 0
        out = b"".join(T.token_text(v, p, t) for p, t in zip(ids, ids[1:]))
        assert out == prompt
        for ch in T.characters(prompt):
            if v.lookup(ch) < 0:
                want = [b + 3 for b in ch]
                assert any(ids[i:i + len(want)] == want for i in range(len(ids))), ch


@pytest.mark.parametrize("n", [300, 512, 2048, 32000])
def test_library_matches_oracle(n):
    shape = W.Shape(64, 96, 1, 4, 4, n, 4096)
    s0 = Bl.section_zero(Bl.build_blob(shape, 62))
    v = T.Vocab(s0)
    rng = np.random.default_rng(n)
    for seed in range(20):
        prompt = V.sample_text(int(rng.integers(0, 400)), 1000 + seed)
        e, ids = B.fpi8_tokenize(s0, prompt, 7)
        assert (e, list(ids)) == T.encode(v, prompt, 7)
    for _ in range(300):
        prev, tok = (int(x) for x in rng.integers(0, n, 2))
        assert B.fpi8_token_text(s0, prev, tok) == (0, T.token_text(v, prev, tok))
    for tok in range(3, 259):
        assert B.fpi8_token_text(s0, 5, tok) == (0, bytes([tok - 3]))


def test_errors_agree():
    shape = W.Shape(64, 96, 1, 4, 4, 512, 40)
    s0 = Bl.section_zero(Bl.build_blob(shape, 63))
    v = T.Vocab(s0)
    cases = [(b"a" * 1025, 1), (b"ab\x00c", 1), (b"abc", 0), (b"abc", 41),
             (b"a" * 1024, 1), (b"hello there", 30), (b"a b c d e f g h i j k l m n o", 30)]
    for prompt, mx in cases:
        want = T.encode(v, prompt, mx)
        e, ids = B.fpi8_tokenize(s0, prompt, mx)
        assert e == want[0], (prompt[:20], mx, e, want[0])
        if e == 0:
            assert list(ids) == want[1]
    assert T.encode(v, b"a" * 1025, 1)[0] == 6
    assert T.encode(v, b"abc", 0)[0] == 6
    assert B.fpi8_token_text(s0, 0, 512)[0] == 6
    # a vocabulary below 260 tokens has no tokenizer block
    small = Bl.section_zero(Bl.build_blob(W.SMALL_SHAPES["h8"], 64))
    assert B.fpi8_tokenize(small, b"abc", 1)[0] == 2
    with pytest.raises(ValueError):
        T.Vocab(small)


def test_blob_check_rejects_bad_tokenizer_blocks():
    # The oracle's and the library's artifact checks both refuse a block
    # whose strings repeat or are out of order, a piece beyond 128 bytes, a
    # count other than the vocabulary, or a wrong longest length.
    shape = W.SMALL_SHAPES["gqa"]
    pieces, scores = V.build_vocab(300)
    good = Bl.build_blob(shape, 65)
    assert O.blob_check(good)[0] == 0 and B.fpi8_blob_check(good)[0] == 0

    def check(block):
        bl = Bl.build_blob(shape, 65, tok=block)
        assert O.blob_check(bl)[0] == 2
        assert B.fpi8_blob_check(bl)[0] == 2
    p = list(pieces)
    p[299] = p[298]                                        # a string twice
    check(V.block_from(p, scores))
    p = list(pieces)
    p[299] = b"x" * 129                                    # too long
    check(V.block_from(p, scores))
    blk = bytearray(V.block_from(pieces, scores))
    blk[0:4] = np.uint32(299).tobytes()                    # count
    check(bytes(blk))
    blk = bytearray(V.block_from(pieces, scores))
    blk[4:8] = np.uint32(7).tobytes()                      # longest
    check(bytes(blk))
    blk = bytearray(V.block_from(pieces, scores))
    o = 8 + 8 * 300 + 4                                    # sorted ids: swap two
    a, b = bytes(blk[o:o + 4]), bytes(blk[o + 4:o + 8])
    blk[o:o + 4], blk[o + 4:o + 8] = b, a
    check(bytes(blk))


def test_output_text_matches_oracle():
    # A text prompt through the whole pass on the CPU: the library's text of
    # the generated tokens equals the oracle's.
    shape = W.TINY.shape
    blob = Bl.build_blob(shape, 66)
    s0 = Bl.section_zero(blob)
    v = T.Vocab(s0)
    for temp, seed in ((0, 1), (65536, 2), (3 * 65536, 3)):
        prompt = V.sample_text(12, 70 + seed)
        e, ids = T.encode(v, prompt, 8)
        assert e == 0
        e, st = O.init_state(shape.as_tuple(), ids, 8, temp, seed)
        assert e == 0 and O.run_to_end(blob, st) == 0
        toks = O.state_info(st)[1]["generated"]
        L = O.state_layout(shape.as_tuple(), len(ids), 8)
        gen = st[L["out"]: L["out"] + 4 * toks].view(np.uint32)
        assert B.fpi8_output_text(s0, st) == (0, T.output_text(v, ids, gen))
