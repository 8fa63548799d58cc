// fpi8_tokenizer.cpp - the tokenizer of section zero, on the host: phases 0
// to 2 of "The inference core" page ("The forward pass, in order") and the
// text of generated tokens ("Sampling", last paragraph), over the block
// layout the artifact header points at (offset 88, length 96):
//   u32 n, u32 longest, u32 score[n], u32 start[n + 1], u32 sorted_ids[n],
//   pool bytes (token i is pool[start[i], start[i + 1])).
// Lookups are binary searches over sorted_ids, as the page's cost table
// describes them ("Tokenizing").
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

namespace fpi8 {

namespace {

uint32_t rd32(const uint8_t *p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}

// Orders byte strings as the sorted ids are: bytewise, a prefix first.
int compare(const uint8_t *a, uint32_t na, const uint8_t *b, uint32_t nb) {
  const int c = memcmp(a, b, na < nb ? na : nb);
  if (c != 0) return c;
  return na < nb ? -1 : na > nb ? 1 : 0;
}

}  // namespace

// Checks a tokenizer block of `len` bytes for a vocabulary of `vocab`
// tokens and fills `v`: the counts fit the block, the pieces lie in the
// pool, no piece is empty or longer than 128 bytes (a generated token's
// text fits its 128 bytes of output text), the longest is recorded right,
// and sorted_ids is a permutation in strictly increasing order (no two
// tokens share a string).
bool vocab_parse(const uint8_t *blk, uint64_t len, uint32_t vocab, Vocab *v) {
  if (len < 8) return false;
  const uint32_t n = rd32(blk), longest = rd32(blk + 4);
  if (n != vocab || n < 259) return false;
  const uint64_t head = 8 + 4ull * n + 4ull * (n + 1) + 4ull * n;
  if (head > len) return false;
  v->n = n;
  v->longest = longest;
  v->score = blk + 8;
  v->start = blk + 8 + 4ull * n;
  v->sorted = blk + 8 + 8ull * n + 4;
  v->pool = blk + head;
  const uint64_t pool_len = len - head;
  uint32_t prev = 0, most = 0;
  for (uint32_t i = 0; i <= n; i++) {
    const uint32_t s = rd32(v->start + 4ull * i);
    if (s < prev || s > pool_len) return false;
    if (i > 0) {
      const uint32_t piece = s - prev;
      if (piece == 0 || piece > 128) return false;
      most = piece > most ? piece : most;
    }
    prev = s;
  }
  if (most != longest) return false;
  std::vector<uint8_t> seen(n, 0);
  for (uint32_t k = 0; k < n; k++) {
    const uint32_t id = rd32(v->sorted + 4ull * k);
    if (id >= n || seen[id]) return false;
    seen[id] = 1;
    if (k > 0) {
      const uint32_t p = rd32(v->sorted + 4ull * (k - 1));
      if (compare(v->piece(p), v->piece_len(p), v->piece(id), v->piece_len(id)) >= 0) return false;
    }
  }
  return true;
}

// The id of the token whose string is s[0, n), or -1.
int64_t vocab_lookup(const Vocab &v, const uint8_t *s, uint32_t n) {
  uint32_t lo = 0, hi = v.n;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2;
    const uint32_t id = rd32(v.sorted + 4ull * mid);
    const int c = compare(v.piece(id), v.piece_len(id), s, n);
    if (c == 0) return id;
    if (c < 0) lo = mid + 1; else hi = mid;
  }
  return -1;
}

// Section zero's configuration and its tokenizer block, checked: 0 or 2.
int32_t vocab_of(const uint8_t *s0, uint64_t s0_len, Model *m, Vocab *v) {
  if (!s0) return FPI8_INVALID_FORMAT;
  int e = parse_section0(s0, s0_len, UINT64_MAX, m);  // section zero alone
  if (e) return e;
  const uint64_t tok = rd32(s0 + 88) | (uint64_t)rd32(s0 + 92) << 32;
  const uint64_t len = rd32(s0 + 96) | (uint64_t)rd32(s0 + 100) << 32;
  if (len == 0 || !vocab_parse(s0 + tok, len, m->cfg.vocab, v)) return FPI8_INVALID_FORMAT;
  return 0;
}

}  // namespace fpi8

using namespace fpi8;

namespace {

// The text token adds after prev into out (at most 128 bytes); its length.
uint32_t piece_text(const Vocab &v, uint32_t prev, uint32_t token, uint8_t *out) {
  const uint8_t *p = v.piece(token);
  uint32_t n = v.piece_len(token);
  if (token == 1 || token == 2) return 0;              // no text
  if (n > 0 && prev == 1 && p[0] == ' ') { p++; n--; }  // after the opening token
  auto hex = [](uint8_t c, uint8_t *d) {
    if (c >= '0' && c <= '9') { *d = c - '0'; return true; }
    if (c >= 'A' && c <= 'F') { *d = c - 'A' + 10; return true; }
    if (c >= 'a' && c <= 'f') { *d = c - 'a' + 10; return true; }
    return false;
  };
  uint8_t hi, lo;
  if (n == 6 && memcmp(p, "<0x", 3) == 0 && p[5] == '>' && hex(p[3], &hi) && hex(p[4], &lo)) {
    out[0] = (uint8_t)(hi * 16 + lo);  // a byte token: that one byte
    return 1;
  }
  memcpy(out, p, n);
  return n;
}

}  // namespace

extern "C" {

int32_t fpi8_tokenize(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *prompt,
                      uint32_t prompt_len, uint32_t max_tokens, uint32_t *ids, uint32_t capacity,
                      uint32_t *n_ids) {
  Model m;
  Vocab v;
  int e = vocab_of(h_section0, section0_len, &m, &v);
  if (e) return e;
  const uint32_t context = m.cfg.context;
  if ((prompt_len > 0 && !prompt) || prompt_len > 1024 || max_tokens == 0 || max_tokens > context)
    return FPI8_INVALID_PROMPT;
  for (uint32_t i = 0; i < prompt_len; i++)
    if (prompt[i] == 0) return FPI8_INVALID_PROMPT;
  // Phase 0: the opening token, then a single space's token when the
  // prompt has text.
  std::vector<uint32_t> t;
  t.reserve(prompt_len + 2);
  t.push_back(1);
  const uint8_t space = ' ';
  if (prompt_len > 0) {
    const int64_t s = vocab_lookup(v, &space, 1);
    t.push_back(s >= 0 ? (uint32_t)s : space + 3u);
  }
  // Phase 1: one UTF-8 character at a time (a lead byte and up to three
  // continuation bytes), looked up whole, else one token per byte.
  for (uint32_t i = 0; i < prompt_len;) {
    uint32_t j = i + 1;
    while (j < prompt_len && j - i < 4 && (prompt[j] & 0xC0) == 0x80) j++;
    const int64_t id = vocab_lookup(v, prompt + i, j - i);
    if (id >= 0) {
      t.push_back((uint32_t)id);
    } else {
      for (uint32_t k = i; k < j; k++) t.push_back(prompt[k] + 3u);
    }
    i = j;
  }
  // Phase 2: the adjacent pair whose merged string is the highest-scoring
  // token (the leftmost among equals) becomes that token, until none is.
  std::vector<uint8_t> buf(2 * 128);
  for (;;) {
    int64_t best_at = -1, best_id = -1;
    uint32_t best_score = 0;
    for (size_t i = 0; i + 1 < t.size(); i++) {
      const uint32_t a = t[i], b = t[i + 1];
      const uint32_t na = v.piece_len(a), nb = v.piece_len(b);
      memcpy(buf.data(), v.piece(a), na);
      memcpy(buf.data() + na, v.piece(b), nb);
      const int64_t id = vocab_lookup(v, buf.data(), na + nb);
      if (id < 0) continue;
      const uint32_t sc = rd32(v.score + 4ull * id);
      if (best_at < 0 || sc > best_score) {
        best_at = (int64_t)i;
        best_id = id;
        best_score = sc;
      }
    }
    if (best_at < 0) break;
    t[best_at] = (uint32_t)best_id;
    t.erase(t.begin() + best_at + 1);
  }
  // Then the prompt's tokens and max tokens must fit the context.
  if (uint64_t(t.size()) + max_tokens - 1 > context) return FPI8_CONTEXT_EXCEEDED;
  if (n_ids) *n_ids = (uint32_t)t.size();
  if (!ids || capacity < t.size()) return FPI8_BUFFER_TOO_SMALL;
  memcpy(ids, t.data(), 4 * t.size());
  return 0;
}

int32_t fpi8_token_text(const uint8_t *h_section0, uint64_t section0_len, uint32_t prev,
                        uint32_t token, uint8_t *out, uint32_t capacity, uint32_t *len) {
  Model m;
  Vocab v;
  int e = vocab_of(h_section0, section0_len, &m, &v);
  if (e) return e;
  if (token >= v.n || prev >= v.n) return FPI8_INVALID_PROMPT;
  uint8_t piece[128];
  const uint32_t n = piece_text(v, prev, token, piece);
  if (len) *len = n;
  if (n > 0 && (!out || capacity < n)) return FPI8_BUFFER_TOO_SMALL;
  if (n > 0) memcpy(out, piece, n);
  return 0;
}

int32_t fpi8_output_text(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *state,
                         uint64_t state_len, uint8_t *out, uint64_t capacity, uint64_t *len) {
  Model m;
  Vocab v;
  int32_t e = vocab_of(h_section0, section0_len, &m, &v);
  if (e) return e;
  uint32_t count = 0;
  const uint32_t *toks = fpi8_output_tokens(state, state_len, &count);
  if (!toks) return FPI8_INVALID_STATE;
  fpi8_info info;
  fpi8_state_info(state, state_len, &info);
  if (info.n_ids == 0) return FPI8_INVALID_STATE;
  // the first generated token follows the prompt's last id
  uint32_t ids_last;
  memcpy(&ids_last, state + ST_HEADER + 4ull * (info.n_ids - 1), 4);
  uint64_t n = 0;
  uint8_t piece[128];
  uint32_t prev = ids_last;
  for (uint32_t i = 0; i < count; i++) {
    uint32_t tok;
    memcpy(&tok, toks + i, 4);
    if (tok >= v.n || prev >= v.n) return FPI8_INVALID_PROMPT;
    const uint32_t k = piece_text(v, prev, tok, piece);
    if (out && n + k <= capacity) memcpy(out + n, piece, k);
    n += k;
    prev = tok;
  }
  if (len) *len = n;
  return n > capacity || (n > 0 && !out) ? FPI8_BUFFER_TOO_SMALL : 0;
}

}  // extern "C"
