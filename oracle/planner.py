"""Oracle of the turn planner: plan_turn and quote_turns for an ids-in state.

Test infrastructure, like the rest of oracle/: only tests/ use it; the
library never does.  Written from "The inference core" page, sections "The
turn planner" (what a turn may hold and when it stops) and "Compute costs"
(the charge of every kind of chunk), with the same cursor semantics as the
oracle's turn of units (fpi8_ref_turn_units): a unit is a matrix row, a
position of attention stages 0-2 or an output element of stage 3, a
vocabulary entry of a sampling pass, or a phase that is one vector
operation.

A turn starts with 18,000 units charged for the instruction.  It then adds
chunks, each the setup of its kind, 160 for the cursor, and its units'
charges, until one of these: the next chunk does not fit what is left of
1,350,000; the next chunk needs a third matrix section; the run is complete.

Readings where the page is silent (the library takes the same):

* the 18,000 count against the 1,350,000, so chunks share what is left
  after them (1,332,000);
* a chunk takes as many units as fit; a chunk with no unit that fits ends
  the turn.  A vector operation is one unit with no setup.  The chunk whose
  last unit ends a sampling pass also carries the pass's finishing charge
  of 4,000, which must fit too;
* a chunk that continues an item begun in an earlier turn pays its setup
  and 160 again;
* a matrix chunk, and the embedding (it reads a row of the embedding
  matrix), need the section that holds their matrix; attention, the vector
  operations and sampling read section zero only;
* the run is complete when it has generated max tokens; stop tokens (1 and
  2) cannot be known ahead, so a turn planned past one simply ends there;
* above temperature zero sampling makes three passes (maximum, sum, draw),
  each a chunk kind of its own with setup 350, per entry 11, 36 and 42, and
  each ending with the finishing charge (parity unpinned by the page, which
  prints temperature-zero figures only).  The draw stops at the entry the
  remainder falls inside, which shows only when it runs: the planner charges
  it for every entry left (an upper bound) and ends the turn with the chunk
  that ends the draw, so the turn ends exactly at the next position's start
  whatever the draw's length (ends_with_draw; such a turn runs as a turn that
  finishes the position, the others as a turn of their units).

Only states at phase 3 or later (ids already fed) are planned; the
tokenizing turns of a text prompt are not.
"""
from __future__ import annotations

import numpy as np

BUDGET = 1_350_000
TURN = 18_000
CHUNK = 160

# header offsets of the ids-in state ("The resumable state", same fields)
H_PHASE, H_LAYER, H_ROW, H_POSITION = 8, 12, 16, 20
H_NIDS, H_MAX, H_TEMP, H_GENERATED = 32, 36, 40, 44
H_PASS, H_STAGE, H_INDEX = 100, 120, 124


def _u32(a: np.ndarray, off: int) -> int:
    return int(a[off: off + 4].view(np.uint32)[0])


def _u64(a: np.ndarray, off: int) -> int:
    return int(a[off: off + 8].view(np.uint64)[0])


def artifact_layout(section_zero: np.ndarray):
    """(cfg, section of each matrix as {(kind, layer): section}) from the
    artifact's header and matrix descriptors (32 bytes each: kind, layer,
    rows, cols, section, zero, offset)."""
    cfg = tuple(int(v) for v in section_zero[8:36].view(np.uint32))
    n = _u32(section_zero, 40)
    at = _u64(section_zero, 104)
    sec = {}
    for i in range(n):
        d = section_zero[at + 32 * i: at + 32 * i + 24].view(np.uint32)
        sec[(int(d[0]), int(d[1]))] = int(d[4])
    return cfg, sec


def _row_charge(n: int, cache: bool = False) -> int:
    return 37 * (n // 8) + 8 * (n % 8) + (42 if cache else 34)


class Item:
    """One piece of the pass: a matrix, an attention stage of one head, a
    sampling pass or a vector operation, with the cursor fields that name it."""

    def __init__(self, phase, layer, units, setup, per, finish=0, section=None, head=0, stage=0,
                 sample_pass=0, ends_token=False):
        self.phase, self.layer, self.units = phase, layer, units
        self.setup, self.per, self.finish, self.section = setup, per, finish, section
        self.head, self.stage, self.sample_pass = head, stage, sample_pass
        self.ends_token = ends_token
        self.position = 0
        self.done_before = 0


def position_items(cfg, sec, position, generating, temperature_q16):
    """The items of one position in the page's phase order (3, then 4-16 per
    layer, then 17-19 where a token is generated)."""
    d, h, layers, heads, kv_heads, vocab, context = cfg
    q = d // heads
    kvd = kv_heads * q
    p = position + 1
    out = [Item(3, 0, 1, 0, 16 * d + 512, section=sec[(0, 0)])]
    for l in range(layers):
        out.append(Item(4, l, 1, 0, 48 * d + 1500))
        out.append(Item(5, l, d, 6 * d + 350, _row_charge(d), section=sec[(1, l)]))
        out.append(Item(6, l, kvd, 6 * d + 350, _row_charge(d, True), section=sec[(2, l)]))
        out.append(Item(7, l, kvd, 6 * d + 350, _row_charge(d, True), section=sec[(3, l)]))
        out.append(Item(8, l, 1, 0, 48 * d + 512))
        for hh in range(heads):
            out.append(Item(9, l, p, 100, 53 * (q // 8) + 11 * (q % 8) + 25, head=hh, stage=0))
            out.append(Item(9, l, p, 80, 23, head=hh, stage=1))
            out.append(Item(9, l, p, 60, 8, head=hh, stage=2))
            out.append(Item(9, l, q, 60, 11 * p + 32, head=hh, stage=3))
        out.append(Item(10, l, d, 6 * d + 350, _row_charge(d), section=sec[(4, l)]))
        out.append(Item(11, l, 1, 0, 56 * d + 1500))
        out.append(Item(12, l, h, 6 * d + 350, _row_charge(d), section=sec[(5, l)]))
        out.append(Item(13, l, h, 6 * d + 350, _row_charge(d), section=sec[(6, l)]))
        out.append(Item(14, l, 1, 0, 24 * h + 512))
        out.append(Item(15, l, d, 6 * h + 350, _row_charge(h), section=sec[(7, l)]))
        out.append(Item(16, l, 1, 0, 8 * d + 128))
    if generating:
        out.append(Item(17, 0, 1, 0, 48 * d + 1500))
        out.append(Item(18, 0, vocab, 6 * d + 350, _row_charge(d), section=sec[(8, 0)]))
        per = (11,) if temperature_q16 == 0 else (11, 36, 42)
        for k, e in enumerate(per):
            out.append(Item(19, 0, vocab, 350, e, finish=4000, sample_pass=k,
                            ends_token=k == len(per) - 1))
    return out


def _order(phase: int, layer: int) -> int:
    """Rank of a (phase, layer) cursor inside a position: 3; 4-16 of layer 0,
    of layer 1, ...; then 17, 18, 19 (the state keeps layer 0 there)."""
    if phase == 3:
        return 0
    if phase <= 16:
        return 1 + 13 * layer + (phase - 4)
    return 1 << 30 | (phase - 17)


def _remaining_items(cfg, sec, st):
    """(item, units already done) from the state's cursor to the end of the run."""
    phase, layer, row = _u32(st, H_PHASE), _u32(st, H_LAYER), _u32(st, H_ROW)
    pos = _u32(st, H_POSITION)
    n_ids, mx, temp = _u32(st, H_NIDS), _u32(st, H_MAX), _u32(st, H_TEMP)
    gen = _u32(st, H_GENERATED)
    stage, index, spass = _u32(st, H_STAGE), _u32(st, H_INDEX), _u32(st, H_PASS)
    first = True
    while gen < mx:
        generating = pos >= n_ids - 1
        for it in position_items(cfg, sec, pos, generating, temp):
            it.position = pos
            done = 0
            if first:
                # items before the cursor are done; the cursor's own item is
                # done up to its row (matrix), head/stage/index (attention)
                # or pass/entry (sampling)
                key = _order(it.phase, it.layer)
                cur = _order(phase, layer)
                if key < cur:
                    continue
                if key == cur:
                    if it.phase == 9:
                        if (it.head, it.stage) < (row, stage):
                            continue
                        if (it.head, it.stage) == (row, stage):
                            done = index
                    elif it.phase == 19:
                        if it.sample_pass < spass:
                            continue
                        if it.sample_pass == spass:
                            done = row
                    elif it.units > 1:
                        done = row
            it.done_before = done
            yield it, done
            if it.ends_token:
                gen += 1
        first = False
        pos += 1


def chunks(section_zero: np.ndarray, st: np.ndarray):
    """Every chunk from the state's cursor to the end of the run, planned turn
    by turn: tuples (turn, item, position, units, charge, sections of the
    turn so far, whether the chunk ends its item).  Turn 0 is the next one.
    The 18,000 of each turn are not chunks."""
    cfg, sec = artifact_layout(section_zero)
    n_ids = _u32(st, H_NIDS)
    turn = 0
    left = BUDGET - TURN
    sections = []
    in_turn = 0  # chunks in this turn
    pos = _u32(st, H_POSITION)
    for it, done in _remaining_items(cfg, sec, st):
        rest = it.units - done
        while rest > 0:
            k = 0
            if not (it.section is not None and it.section not in sections and len(sections) == 2):
                room = left - it.setup - CHUNK
                if room > 0:
                    k = min(rest, room // it.per)
                    if k == rest and it.finish and k * it.per + it.finish > room:
                        k = rest - 1
            if k <= 0:
                if in_turn == 0:
                    raise ValueError("a chunk that fits no turn")
                turn += 1
                left = BUDGET - TURN
                sections = []
                in_turn = 0
                continue
            cost = it.setup + CHUNK + k * it.per + (it.finish if k == rest else 0)
            left -= cost
            if it.section is not None and it.section not in sections:
                sections.append(it.section)
            rest -= k
            in_turn += 1
            yield turn, it, it.position, k, cost, list(sections), rest == 0
            if rest == 0 and it.phase == 19 and it.sample_pass == 2:
                # a draw's length shows only when it runs: the turn ends here
                turn += 1
                left = BUDGET - TURN
                sections = []
                in_turn = 0


def plan_turn(section_zero: np.ndarray, st: np.ndarray) -> dict:
    """The next turn of the run in state st: the compute units charged, the
    matrix sections read in the order reached, the units of work it runs and
    the most tokens it can complete."""
    if _u32(st, H_PHASE) == 20:
        return {"estimated_cu": 0, "sections": [], "units": 0, "max_generated": 0, "ends_with_draw": 0}
    cu, units, tokens, sections, draw = TURN, 0, 0, [], 0
    for turn, it, pos, k, cost, secs, ends in chunks(section_zero, st):
        if turn > 0:
            break
        cu += cost
        units += k
        sections = secs
        if it.ends_token and ends:
            tokens += 1
        draw = 1 if (ends and it.phase == 19 and it.sample_pass == 2) else 0
    return {"estimated_cu": cu, "sections": sections, "units": units, "max_generated": tokens,
            "ends_with_draw": draw}


def quote_turns(section_zero: np.ndarray, st: np.ndarray) -> int:
    """The count of turns the run in state st takes to generate max tokens
    (fewer if it meets a stop token): plan_turn stepped to the end."""
    if _u32(st, H_PHASE) == 20:
        return 0
    last = -1
    for turn, *_ in chunks(section_zero, st):
        last = turn
    return last + 1
