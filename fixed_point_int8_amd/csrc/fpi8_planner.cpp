// fpi8_planner.cpp - the turn planner of "The inference core" page, on the
// host: how far the next turn of a run goes (fpi8_plan_turn) and how many
// turns a run takes (fpi8_quote_turns).
//
// "The turn planner": a turn is charged 18,000 units for the instruction,
// then chunks of work, each 160 units for the cursor plus its own charges
// ("Compute costs"), until the next chunk does not fit what is left of the
// turn's 1,350,000 units, or needs a third matrix section, or the run is
// complete.  A chunk is a run of rows of one matrix (setup 6n + 350, per
// row 37 floor(n/8) + 8 (n mod 8) + 34, or + 42 for a key or value row
// stored in the cache), a run of units of one attention stage of one head
// (setups 100, 80, 60, 60; per unit 53 floor(q/8) + 11 (q mod 8) + 25, 23
// and 8 per position so far, 11 p + 32 per output element), a run of
// vocabulary entries of one sampling pass (setup 350; 11, 36 or 42 per entry;
// 4,000 when the pass ends), or one whole vector operation (embedding
// 16d + 512, the normalizations 48d + 1,500, rotary 48d + 512, residual with
// the feed-forward normalization 56d + 1,500, SiLU 24h + 512, residual
// 8d + 128).
//
// Readings (the page is silent): the 18,000 count against the 1,350,000; a
// chunk takes as many units as fit and a chunk that fits none ends the turn;
// a chunk continuing an item begun in an earlier turn pays its setup and 160
// again; the chunk that ends a sampling pass carries the 4,000, which must
// fit too; matrix chunks and the embedding need their matrix's section
// (from the artifact's descriptors), the rest only section zero; the run is
// complete at max tokens (stop tokens cannot be foreseen); above temperature
// zero there are three passes, each ending with the 4,000, and a turn ends
// with the chunk that ends a draw pass: the draw stops at the entry the
// remainder falls inside, known only when it runs, so the plan charges every
// entry left (an upper bound) and the turn's end is the next position's
// start whatever the draw's length.  Units of work are those of
// fpi8_turn_units, so a planned turn runs as a turn of its units, or, when
// it ends with a draw, as a turn that finishes the position.
#include <stdint.h>
#include <string.h>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

using namespace fpi8;

namespace {

constexpr uint64_t kBudget = 1350000, kTurnCharge = 18000, kChunkCharge = 160;

uint32_t rd32(const uint8_t *p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}
uint64_t rd64(const uint8_t *p) {
  uint64_t v;
  memcpy(&v, p, 8);
  return v;
}

// The section holding each matrix: [0] embedding, [1 + 7 l + k] layer l's
// k-th matrix (query .. down), [1 + 7 L] classifier; read from the matrix
// descriptors of section zero.
bool read_sections(const uint8_t *s0, uint64_t len, Cfg *c, uint32_t *sec, uint32_t nsec_max) {
  if (len < 144 || memcmp(s0, "CURTAW01", 8) != 0) return false;
  uint32_t w[7];
  for (int i = 0; i < 7; i++) w[i] = rd32(s0 + 8 + 4 * i);
  if (!cfg_from_words(w, c)) return false;
  const uint32_t nmat = rd32(s0 + 40);
  if (nmat != 2 + 7 * c->layers || nmat > nsec_max) return false;
  const uint64_t at = rd64(s0 + 104);
  if (at > len || 32ull * nmat > len - at) return false;
  for (uint32_t i = 0; i < nmat; i++) sec[i] = 0;
  for (uint32_t i = 0; i < nmat; i++) {
    const uint8_t *d = s0 + at + 32ull * i;
    const uint32_t kind = rd32(d), layer = rd32(d + 4), section = rd32(d + 16);
    uint32_t slot;
    if (kind == 0 || kind == 8) {
      if (layer != 0) return false;
      slot = kind == 0 ? 0 : 1 + 7 * c->layers;
    } else if (kind <= 7) {
      if (layer >= c->layers) return false;
      slot = 1 + 7 * layer + (kind - 1);
    } else {
      return false;
    }
    if (section == 0 || sec[slot] != 0) return false;
    sec[slot] = section;
  }
  return true;
}

// The chunks of a run, turn by turn.  take() offers an item: `units` still
// to do, its setup, per-unit and finishing charges and its section (0 for
// section zero alone).  It returns false once the caller needs no more.
struct Turns {
  bool plan_only;              // stop at the end of the first turn
  uint64_t left = kBudget - kTurnCharge;
  uint32_t secs[2] = {0, 0};
  uint32_t nsec = 0;
  uint64_t chunks_in_turn = 0;
  uint64_t turns = 0;          // turns ended so far
  bool stopped = false;
  bool stuck = false;          // a chunk that fits no turn
  // the first turn
  uint64_t cu = kTurnCharge, units = 0;
  uint32_t tokens = 0, first_secs[2] = {0, 0}, first_nsec = 0, first_draw = 0;
  bool last_draw = false;      // the last chunk ended a draw pass

  bool has(uint32_t s) const { return s == 0 || (nsec > 0 && secs[0] == s) || (nsec > 1 && secs[1] == s); }

  void end_turn() {
    if (turns == 0) {
      first_nsec = nsec;
      first_secs[0] = secs[0];
      first_secs[1] = secs[1];
      first_draw = last_draw ? 1 : 0;
    }
    turns++;
    left = kBudget - kTurnCharge;
    nsec = 0;
    chunks_in_turn = 0;
    if (plan_only) stopped = true;
  }

  // draw: the item is a draw pass, whose true length shows only when it
  // runs; the turn ends with the chunk that ends it.
  bool take(uint64_t n, uint64_t setup, uint64_t per, uint64_t finish, uint32_t section, bool ends_token,
            bool draw = false) {
    while (n > 0 && !stopped) {
      uint64_t k = 0;
      if (has(section) || nsec < 2) {
        if (left > setup + kChunkCharge) {
          const uint64_t room = left - setup - kChunkCharge;
          k = room / per < n ? room / per : n;
          if (k == n && finish && k * per + finish > room) k = n - 1;
        }
      }
      if (k == 0) {
        if (chunks_in_turn == 0) {
          stuck = true;
          stopped = true;
          return false;
        }
        end_turn();
        continue;
      }
      const uint64_t cost = setup + kChunkCharge + k * per + (k == n ? finish : 0);
      left -= cost;
      if (!has(section)) secs[nsec++] = section;
      chunks_in_turn++;
      if (turns == 0) {
        cu += cost;
        units += k;
        if (k == n && ends_token) tokens++;
      }
      last_draw = draw && k == n;
      n -= k;
      if (last_draw) end_turn();
    }
    return !stopped;
  }
};

uint64_t row_charge(uint64_t n, bool cache) { return 37 * (n / 8) + 8 * (n % 8) + (cache ? 42 : 34); }

// Walks the work from the state's cursor to max tokens, offering each item
// to t (the cursor's own item offered with what it has left).
void walk(const Cfg &c, const uint32_t *sec, const uint8_t *h, Turns &t) {
  const uint64_t d = c.dim, hd = c.hidden, q = c.head, kvd = c.kvd, L = c.layers;
  uint32_t phase = rd32(h + 8), layer = rd32(h + 12), row = rd32(h + 16);
  uint32_t pos = rd32(h + 20);
  const uint32_t n_ids = rd32(h + 32), mx = rd32(h + 36), temp = rd32(h + 40);
  uint32_t gen = rd32(h + 44);
  uint32_t stage = rd32(h + 120), index = rd32(h + 124), pass = rd32(h + 100);
  const int passes = temp == 0 ? 1 : 3;
  const uint64_t per_entry[3] = {11, 36, 42};
  while (gen < mx) {
    const uint64_t p = (uint64_t)pos + 1;
    const bool generating = pos + 1 >= n_ids;
    // phase 3
    if (phase == 3 && !t.take(1, 0, 16 * d + 512, 0, sec[0], false)) return;
    for (uint32_t l = (phase >= 4 && phase <= 16) ? layer : 0; l < L && (phase <= 16); l++) {
      const uint32_t *ls = sec + 1 + 7 * l;
      // the first phase of this layer to run, and what the cursor's item has done
      const uint32_t from = (phase >= 4 && phase <= 16 && l == layer) ? phase : 4;
      auto left_of = [&](uint32_t ph, uint64_t units) { return ph == from ? units - row : units; };
      if (from <= 4 && !t.take(1, 0, 48 * d + 1500, 0, 0, false)) return;
      if (from <= 5 && !t.take(left_of(5, d), 6 * d + 350, row_charge(d, false), 0, ls[0], false)) return;
      if (from <= 6 && !t.take(left_of(6, kvd), 6 * d + 350, row_charge(d, true), 0, ls[1], false)) return;
      if (from <= 7 && !t.take(left_of(7, kvd), 6 * d + 350, row_charge(d, true), 0, ls[2], false)) return;
      if (from <= 8 && !t.take(1, 0, 48 * d + 512, 0, 0, false)) return;
      if (from <= 9) {
        const uint64_t su[4] = {100, 80, 60, 60};
        const uint64_t pu[4] = {53 * (q / 8) + 11 * (q % 8) + 25, 23, 8, 11 * p + 32};
        const uint64_t n[4] = {p, p, p, q};
        for (uint32_t hh = from == 9 ? row : 0; hh < c.heads; hh++)
          for (uint32_t s = (from == 9 && hh == row) ? stage : 0; s < 4; s++) {
            const uint64_t done = (from == 9 && hh == row && s == stage) ? index : 0;
            if (!t.take(n[s] - done, su[s], pu[s], 0, 0, false)) return;
          }
      }
      if (from <= 10 && !t.take(left_of(10, d), 6 * d + 350, row_charge(d, false), 0, ls[3], false)) return;
      if (from <= 11 && !t.take(1, 0, 56 * d + 1500, 0, 0, false)) return;
      if (from <= 12 && !t.take(left_of(12, hd), 6 * d + 350, row_charge(d, false), 0, ls[4], false)) return;
      if (from <= 13 && !t.take(left_of(13, hd), 6 * d + 350, row_charge(d, false), 0, ls[5], false)) return;
      if (from <= 14 && !t.take(1, 0, 24 * hd + 512, 0, 0, false)) return;
      if (from <= 15 && !t.take(left_of(15, d), 6 * hd + 350, row_charge(hd, false), 0, ls[6], false)) return;
      if (from <= 16 && !t.take(1, 0, 8 * d + 128, 0, 0, false)) return;
      phase = 4;
      row = 0;
      stage = index = 0;
    }
    if (generating) {
      if (phase <= 17 && !t.take(1, 0, 48 * d + 1500, 0, 0, false)) return;
      if (phase <= 18) {
        const uint64_t done = phase == 18 ? row : 0;
        if (!t.take(c.vocab - done, 6 * d + 350, row_charge(d, false), 0, sec[1 + 7 * L], false)) return;
      }
      for (int k = (phase == 19 ? (int)pass : 0); k < passes; k++) {
        const uint64_t done = (phase == 19 && k == (int)pass) ? row : 0;
        if (!t.take(c.vocab - done, 350, per_entry[k], 4000, 0, k == passes - 1, k == 2)) return;
      }
      gen++;
    }
    pos++;
    phase = 3;
    layer = 0;
    row = 0;
    stage = index = pass = 0;
  }
}

int32_t plan(const uint8_t *s0, uint64_t s0_len, const uint8_t *state, uint64_t state_len,
             Turns &t, bool *complete) {
  if (!s0 || !state) return FPI8_BUFFER_TOO_SMALL;
  Cfg c;
  static constexpr uint32_t kMaxMats = 2 + 7 * 1024;
  static thread_local uint32_t sec[kMaxMats];
  if (!read_sections(s0, s0_len, &c, sec, kMaxMats)) return FPI8_INVALID_FORMAT;
  if (state_len < ST_HEADER || (reinterpret_cast<uintptr_t>(state) & 7) != 0) return FPI8_INVALID_STATE;
  StateLayout L;
  const int h = check_header(c, state, state_len, &L);
  if (h == -1) {
    *complete = true;
    return 0;
  }
  if (h) return h;
  *complete = false;
  walk(c, sec, state, t);
  if (t.stuck) return FPI8_INVALID_CONFIG;  // a single unit larger than a turn
  if (!t.stopped && t.chunks_in_turn > 0) t.end_turn();
  return 0;
}

}  // namespace

extern "C" {

int32_t fpi8_plan_turn(const uint8_t *h_section_zero, uint64_t section_zero_len, const uint8_t *h_state,
                       uint64_t state_len, fpi8_turn_plan *out) {
  if (!out) return FPI8_BUFFER_TOO_SMALL;
  memset(out, 0, sizeof *out);
  Turns t;
  t.plan_only = true;
  bool complete = false;
  const int32_t e = plan(h_section_zero, section_zero_len, h_state, state_len, t, &complete);
  if (e || complete) return e;
  out->estimated_cu = (uint32_t)t.cu;
  out->section_count = t.first_nsec;
  out->sections[0] = t.first_secs[0];
  out->sections[1] = t.first_secs[1];
  out->max_generated = t.tokens;
  out->ends_with_draw = t.first_draw;
  out->units = t.units;
  return 0;
}

int32_t fpi8_quote_turns(const uint8_t *h_section_zero, uint64_t section_zero_len, const uint8_t *h_state,
                         uint64_t state_len, uint64_t *turns) {
  if (!turns) return FPI8_BUFFER_TOO_SMALL;
  *turns = 0;
  Turns t;
  t.plan_only = false;
  bool complete = false;
  const int32_t e = plan(h_section_zero, section_zero_len, h_state, state_len, t, &complete);
  if (e || complete) return e;
  *turns = t.turns;
  return 0;
}

}  // extern "C"
