"""The compute units the turn planner charges for one position, CPU only.

The oracle (oracle/charges.py) is pinned by the table "One position, added
up" that "The inference core" page prints under "Compute costs"
(tests/golden/position_charges.txt): with every chunk whole, each printed
row equals the oracle's charge plus a whole number of chunk setups that
turn boundaries split off again, and no more splits than the turns have
boundaries.  The library's charges are then compared with the oracle's.
"""
import itertools

import numpy as np
import pytest

from oracle import charges as CH
from fixed_point_int8_amd import binding as B
from conftest import read_table

MODELS = {  # (shape, position, turns) the page names
    "stories260K": ((64, 172, 5, 8, 4, 512, 512), 511, 5),
    "stories15M": ((288, 768, 6, 6, 6, 32000, 256), 255, 62),
}


def printed():
    rows = read_table("position_charges.txt")
    return {name: {r[0]: int(r[1 + j]) for r in rows} for j, name in enumerate(MODELS)}


def fewest_splits(diff, setups):
    """The fewest chunk setups that add up to diff, or None."""
    if not setups:
        return None
    best = None
    ranges = [range(diff // s + 1) for s in setups[:-1]]
    for counts in itertools.product(*ranges):
        rest = diff - sum(c * s for c, s in zip(counts, setups))
        if rest >= 0 and rest % setups[-1] == 0:
            k = sum(counts) + rest // setups[-1]
            best = k if best is None else min(best, k)
    return best


@pytest.mark.parametrize("name", list(MODELS))
def test_charges_against_the_printed_position(name):
    cfg, pos, turns = MODELS[name]
    table = printed()[name]
    got = CH.position_charges(cfg, pos, True, 0)
    assert sum(table[k] for k in table if k != "total") == table["total"]
    assert table["fixed"] == 18_000 * turns
    splits = 0
    exact = 0
    for phase in CH.PHASES:
        diff = table[phase] - got[phase]
        assert diff >= 0, (phase, diff)
        if diff == 0:
            exact += 1
            continue
        k = fewest_splits(diff, CH.split_setup(phase, cfg))
        assert k is not None, (phase, diff)
        splits += k
    assert splits <= turns - 1
    # phases no turn boundary can split (vector operations) are exact
    for phase in ("embed", "norm1", "rotary", "norm2", "silu", "residual", "fnorm"):
        assert table[phase] == got[phase], phase
    # every row but attention and down at stories260K, and the query matrix
    # besides the vector operations at stories15M, is split by no turn
    assert exact >= {"stories260K": 15, "stories15M": 8}[name]


def test_whole_chunk_forms():
    # The per-phase charges written out for one small case by hand from the
    # page's tables: d = 16, h = 24, one layer, 2 heads of 8, 1 key/value
    # head, vocab 10, position 2 (p = 3).
    cfg = (16, 24, 1, 2, 1, 10, 8)
    c = CH.position_charges(cfg, 2, True, 0)
    row16, row24 = 37 * 2 + 34, 37 * 3 + 34
    assert c["q"] == 6 * 16 + 350 + 16 * row16 + 160
    assert c["k"] == 6 * 16 + 350 + 8 * (row16 + 8) + 160
    assert c["down"] == 6 * 24 + 350 + 16 * row24 + 160
    head = (100 + 3 * 78) + (80 + 3 * 23) + (60 + 3 * 8) + (60 + 8 * (33 + 32)) + 4 * 160
    assert c["attention"] == 2 * head
    assert c["sampling"] == 350 + 10 * 11 + 4000 + 160
    warm = CH.position_charges(cfg, 2, True, 65536)["sampling"]
    assert warm == 3 * (350 + 4000 + 160) + 10 * (11 + 36 + 42)
    prompt = CH.position_charges(cfg, 2, False, 0)
    assert prompt["fnorm"] == prompt["classifier"] == prompt["sampling"] == 0


def test_library_matches_oracle():
    rng = np.random.default_rng(5)
    cfgs = [cfg for cfg, _, _ in MODELS.values()] + [
        (4096, 11008, 32, 32, 32, 32000, 4096), (2048, 5632, 22, 32, 32, 32000, 2048),
        (160, 392, 2, 5, 5, 1000, 48), (120, 200, 2, 6, 3, 300, 24)]
    for cfg in cfgs:
        for _ in range(20):
            pos = int(rng.integers(0, cfg[6]))
            gen = bool(rng.integers(0, 2))
            temp = int(rng.choice([0, 1, 65536, 16 << 16]))
            e, out = B.fpi8_position_charges(cfg, pos, gen, temp)
            assert e == 0
            want = CH.position_charges(cfg, pos, gen, temp)
            assert [int(v) for v in out] == [want[p] for p in CH.PHASES], (cfg, pos, gen, temp)


def test_library_errors():
    cfg = MODELS["stories260K"][0]
    assert B.fpi8_position_charges(cfg, 512, True)[0] == 6           # at the context
    assert B.fpi8_position_charges(cfg, 0, True, 16 * 65536 + 1)[0] == 6
    assert B.fpi8_position_charges((64, 172, 5, 7, 4, 512, 512), 0, True)[0] == 1
