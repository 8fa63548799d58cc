"""A run's state in the page's own format (CURTAST2) and back, CPU only.

Pinned by the run-account sizes "The inference core" page prints in "The
resumable state" (tests/golden/state_sizes.txt), by the page's buffer table
read on its own terms in oracle/pages.py, and by round trips that continue
the pass from an imported state.
"""
import numpy as np
import pytest

import oracle as O
from oracle import pages as OP
from oracle import tokenizer as T
import workloads as W
from workloads import blob as Bl
from fixed_point_int8_amd import binding as B
from conftest import read_table

PROMPT = b"Once upon a time"


COLUMNS = ("model", "dim", "hidden", "layers", "heads", "kv_heads", "vocab", "context",
           "prompt_bytes", "max_tokens", "cache_positions", "account_bytes")


def sizes():
    return [dict(zip(COLUMNS, r)) for r in read_table("state_sizes.txt")]


def test_sizes_are_the_pages_run_accounts():
    # the page's run account is a 256-byte header and the core state
    for row in sizes():
        cfg = tuple(int(row[k]) for k in ("dim", "hidden", "layers", "heads", "kv_heads",
                                          "vocab", "context"))
        pb, mx = int(row["prompt_bytes"]), int(row["max_tokens"])
        assert B.fpi8_pages_state_size(cfg, pb, mx) + 256 == int(row["account_bytes"])
        assert OP.layout(cfg, pb, mx)["total"] + 256 == int(row["account_bytes"])
        assert OP.layout(cfg, pb, mx)["cachepos"] == int(row["cache_positions"])


def run_state(shape, seed, max_tokens, units, temp=0):
    """A run of the prompt stopped after `units` units of work, before its end."""
    blob = Bl.build_blob(shape, seed)
    s0 = Bl.section_zero(blob)
    e, ids = T.encode(T.Vocab(s0), PROMPT, max_tokens)
    assert e == 0
    e, st = O.init_state(shape.as_tuple(), ids, max_tokens, temp, seed)
    assert e == 0
    assert O.turn_units(blob, st, units) == 0
    info = O.state_info(st)[1]
    assert not info["complete"] and info["generated"] > 0
    return blob, s0, st


@pytest.mark.parametrize("name,max_tokens,units", [("stories260K", 12, 100_001),
                                                    ("stories15M", 8, 700_003)])
def test_export_matches_oracle_and_the_printed_size(name, max_tokens, units):
    # The models the page sizes, with "Once upon a time" and the synthetic
    # vocabulary: a state stopped inside a position, exported by the library
    # and by the oracle, byte for byte, at the printed account size.
    row = next(r for r in sizes() if r["model"] == name and int(r["prompt_bytes"]) == 16)
    shape = W.Shape(*(int(row[k]) for k in ("dim", "hidden", "layers", "heads", "kv_heads",
                                             "vocab", "context")))
    blob, s0, st = run_state(shape, 70, max_tokens, units, temp=65536)
    cfg = shape.as_tuple()
    e, pg = B.fpi8_state_export(s0, st, PROMPT, cfg)
    assert e == 0
    assert pg.size + 256 == int(row["account_bytes"])
    assert np.array_equal(pg, OP.export(s0, cfg, st, PROMPT))
    assert bytes(pg[:8]) == b"CURTAST2"
    assert pg[28:32].view(np.uint32)[0] == 16 and pg[52:56].view(np.uint32)[0] == 16
    # back: the same state, and the pass goes on from it as from the original
    e, back = B.fpi8_state_import(cfg, pg)
    assert e == 0 and np.array_equal(back, st)
    assert np.array_equal(OP.import_(cfg, pg), st)
    a, b = st.copy(), back.copy()
    assert O.run_to_end(blob, a) == 0 and O.run_to_end(blob, b) == 0
    assert np.array_equal(a, b)


def test_cache_order_and_text():
    # The page's key cache holds [layer][position][kv head * head + element]
    # and its text buffer the generated tokens' text.
    shape = W.SMALL_SHAPES["gqa"]
    blob, s0, st = run_state(shape, 71, 6, 45_001)
    cfg = shape.as_tuple()
    e, pg = B.fpi8_state_export(s0, st, PROMPT, cfg)
    assert e == 0
    info = O.state_info(st)[1]
    S = O.state_layout(cfg, info["n_ids"], info["max_tokens"])
    P = OP.layout(cfg, len(PROMPT), info["max_tokens"])
    hd, cs = shape.head_size, S["cache_positions"]
    mine = st[S["keys"]: S["keys"] + 4 * shape.layers * shape.kv_heads * cs * hd].view(
        np.int32).reshape(shape.layers, shape.kv_heads, cs, hd)
    theirs = pg[P["keys"]: P["keys"] + 4 * shape.layers * P["cachepos"] * shape.kv_dim].view(
        np.int32).reshape(shape.layers, P["cachepos"], shape.kv_dim)
    for l in range(shape.layers):
        for t in range(cs):
            for kh in range(shape.kv_heads):
                assert np.array_equal(theirs[l, t, kh * hd:(kh + 1) * hd], mine[l, kh, t])
    assert not theirs[:, cs:].any()
    n_text = int(pg[48:52].view(np.uint32)[0])
    assert bytes(pg[P["text"]: P["text"] + n_text]) == B.fpi8_output_text(s0, st)[1]
    assert bytes(pg[P["prompt"]: P["prompt"] + len(PROMPT)]) == PROMPT


def test_export_errors():
    shape = W.SMALL_SHAPES["gqa"]
    blob, s0, st = run_state(shape, 72, 4, 40_001)
    cfg = shape.as_tuple()
    assert B.fpi8_state_export(s0, st, b"ab", cfg)[0] == 6        # fewer bytes than the ids need
    bad = st.copy()
    bad[28:32] = np.frombuffer(np.uint32(8).tobytes(), np.uint8)  # a frozen run
    assert B.fpi8_state_export(s0, bad, PROMPT, cfg)[0] == 3
    e, pg = B.fpi8_state_export(s0, st, PROMPT, cfg)
    assert e == 0
    pg2 = pg.copy()
    pg2[8:12] = np.frombuffer(np.uint32(1).tobytes(), np.uint8)   # still tokenizing
    assert B.fpi8_state_import(cfg, pg2)[0] == 3
    pg2 = pg.copy()
    pg2[0] = ord("X")
    assert B.fpi8_state_import(cfg, pg2)[0] == 3
