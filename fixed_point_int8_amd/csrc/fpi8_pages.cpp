// fpi8_pages.cpp - a run's state in the page's own format and back (host).
//
// "The inference core" page, "The resumable state", lays the core state out
// as a 128-byte header tagged CURTAST2 (phase, layer, row, position, token,
// the prompt's length in bytes, the count of prompt tokens, max tokens,
// temperature, tokens generated, output text bytes, five tokenizer fields,
// the generator, the turn count, then the attention and sampling fields),
// followed by the prompt bytes, the prompt tokens (prompt bytes + 2), the
// output tokens, the output text (max tokens x 128), the activations and
// three working vectors, gate and up, logits, scores and the key and value
// caches, each 8-byte aligned, with cache positions min(prompt bytes + max
// tokens + 1, context).  This library's state holds the same words with the
// ids fed in: no prompt bytes or text, cache positions ids + max - 1, and a
// key/value order of [layer][kv head][position][element].  Readings: the
// page's caches are [layer][position][kv head * head + element] (its table
// gives layers x cache positions x key and value dimension); after phase 2
// the tokenizer's next byte is the prompt's length and its other fields are
// zero; the page's state has no error field, so a frozen run has no page
// form.
//
// A state in the page's format can also start before tokenizing
// (fpi8_pages_init) and run phases 0 to 2 in units (fpi8_pages_tokenize),
// with the header's five tokenizer fields as the cursor.  Readings: a unit
// is phase 0 whole; one character of phase 1, or the step that ends it;
// one pair looked up in a merge scan, or the scan's end, which applies the
// best merge found or, with none, checks the context and moves to phase 3.
// The fields hold the next prompt byte, the pair being looked up, and the
// position (0xFFFFFFFF before any), score key and id of the scan's best
// merge; a higher score replaces it, so the leftmost of equals merges.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

using namespace fpi8;

namespace {

uint32_t rd32(const uint8_t *p) { uint32_t v; memcpy(&v, p, 4); return v; }
void wr32(uint8_t *p, uint32_t v) { memcpy(p, &v, 4); }
uint64_t a8(uint64_t n) { return (n + 7) & ~7ull; }

const char kPagesTag[8] = {'C', 'U', 'R', 'T', 'A', 'S', 'T', '2'};

// Byte offsets of the page's buffers.
struct PagesLayout {
  uint64_t prompt, ids, out, text, x, w1, w2, w3, gate, up, logits, scores, keys, values, total;
  uint32_t cachepos;
};

bool pages_layout(const Cfg &c, uint32_t prompt_bytes, uint32_t max_tokens, PagesLayout *L) {
  if (prompt_bytes > 1024 || max_tokens == 0 || max_tokens > c.context) return false;
  uint64_t cp = (uint64_t)prompt_bytes + max_tokens + 1;
  L->cachepos = (uint32_t)(cp > c.context ? c.context : cp);
  uint64_t o = ST_HEADER;
  L->prompt = o; o += a8(prompt_bytes);
  L->ids = o;    o += a8(4ull * (prompt_bytes + 2));
  L->out = o;    o += a8(4ull * max_tokens);
  L->text = o;   o += a8(128ull * max_tokens);
  L->x = o;      o += 8ull * c.dim;
  L->w1 = o;     o += 8ull * c.dim;
  L->w2 = o;     o += 8ull * c.dim;
  L->w3 = o;     o += 8ull * c.dim;
  L->gate = o;   o += 8ull * c.hidden;
  L->up = o;     o += 8ull * c.hidden;
  L->logits = o; o += 8ull * c.vocab;
  L->scores = o; o += 8ull * L->cachepos;
  const uint64_t cache = a8(4ull * c.layers * L->cachepos * c.kvd);
  L->keys = o;   o += cache;
  L->values = o; o += cache;
  L->total = o;
  return true;
}

// Copies one cache between the two orders for positions below npos.
void copy_cache(const Cfg &c, const uint8_t *src, uint32_t src_cp, bool src_pages, uint8_t *dst,
                uint32_t dst_cp, bool dst_pages, uint32_t npos) {
  for (uint32_t l = 0; l < c.layers; l++)
    for (uint32_t kh = 0; kh < c.kv_heads; kh++)
      for (uint32_t t = 0; t < npos; t++) {
        const uint64_t so = src_pages ? ((uint64_t)l * src_cp + t) * c.kvd + (uint64_t)kh * c.head
                                      : (((uint64_t)l * c.kv_heads + kh) * src_cp + t) * c.head;
        const uint64_t d = dst_pages ? ((uint64_t)l * dst_cp + t) * c.kvd + (uint64_t)kh * c.head
                                     : (((uint64_t)l * c.kv_heads + kh) * dst_cp + t) * c.head;
        memcpy(dst + 4 * d, src + 4 * so, 4ull * c.head);
      }
}

constexpr uint32_t kNone = 0xFFFFFFFFu;

// Header words of the page's state used here.
enum : uint32_t {
  PG_PHASE = 8, PG_POSITION = 20, PG_TOKEN = 24, PG_PROMPT = 28, PG_NIDS = 32, PG_MAX = 36,
  PG_TEMP = 40, PG_NEXT_BYTE = 52, PG_PAIR = 56, PG_BEST_AT = 60, PG_BEST_SCORE = 64,
  PG_BEST_ID = 68, PG_SEED = 72
};

}  // namespace

extern "C" {

int32_t fpi8_pages_init(const uint32_t cfg[7], const uint8_t *prompt, uint32_t prompt_len,
                        uint32_t max_tokens, uint32_t temperature_q16, uint64_t seed, uint8_t *out,
                        uint64_t out_len) {
  Cfg c;
  PagesLayout P;
  if (!cfg || !cfg_from_words(cfg, &c)) return FPI8_INVALID_CONFIG;
  if ((prompt_len > 0 && !prompt) || !pages_layout(c, prompt_len, max_tokens, &P) ||
      temperature_q16 > (16u << 16))
    return FPI8_INVALID_PROMPT;
  for (uint32_t i = 0; i < prompt_len; i++)
    if (prompt[i] == 0) return FPI8_INVALID_PROMPT;
  if (!out || out_len != P.total) return FPI8_BUFFER_TOO_SMALL;
  memset(out, 0, out_len);
  memcpy(out, kPagesTag, 8);
  wr32(out + PG_PROMPT, prompt_len);
  wr32(out + PG_MAX, max_tokens);
  wr32(out + PG_TEMP, temperature_q16);
  // a zero seed starts the generator at 0x9E3779B97F4A7C15 ("Sampling")
  const uint64_t g = seed ? seed : 0x9E3779B97F4A7C15ull;
  memcpy(out + PG_SEED, &g, 8);
  if (prompt_len) memcpy(out + P.prompt, prompt, prompt_len);
  return 0;
}

int32_t fpi8_pages_tokenize(const uint8_t *h_section0, uint64_t section0_len, uint8_t *pages,
                            uint64_t pages_len, uint64_t max_units, uint64_t *units_done) {
  if (units_done) *units_done = 0;
  Model m;
  Vocab v;
  int32_t e = vocab_of(h_section0, section0_len, &m, &v);
  if (e) return e;
  const Cfg &c = m.cfg;
  if (!pages || pages_len < ST_HEADER || memcmp(pages, kPagesTag, 8) != 0) return FPI8_INVALID_STATE;
  const uint32_t pb = rd32(pages + PG_PROMPT), mx = rd32(pages + PG_MAX);
  PagesLayout P;
  if (!pages_layout(c, pb, mx, &P) || P.total != pages_len) return FPI8_INVALID_STATE;
  const uint8_t *prompt = pages + P.prompt;
  uint8_t *ids = pages + P.ids;  // u32[prompt bytes + 2], unaligned-safe access
  auto id_at = [&](uint32_t i) { return rd32(ids + 4ull * i); };
  auto set_id = [&](uint32_t i, uint32_t t) { wr32(ids + 4ull * i, t); };
  // the cursor must lie where phases 0 to 2 can leave it
  uint32_t phase = rd32(pages + PG_PHASE), n = rd32(pages + PG_NIDS);
  if (phase > 2) return FPI8_INVALID_STATE;
  const uint32_t cap = pb + 2;
  if (phase > 0 && (n < 1 || n > cap)) return FPI8_INVALID_STATE;
  // in phase 1 the tokens so far are at most the opening and space tokens
  // and one per byte read, so the rest of the prompt still fits the buffer
  if (phase == 1 && (rd32(pages + PG_NEXT_BYTE) > pb ||
                     n > (pb > 0 ? 2u : 1u) + rd32(pages + PG_NEXT_BYTE)))
    return FPI8_INVALID_STATE;
  if (phase == 2) {
    const uint32_t at = rd32(pages + PG_BEST_AT);
    if (rd32(pages + PG_PAIR) >= n || (at != kNone && at + 1 >= n) ||
        (at != kNone && rd32(pages + PG_BEST_ID) >= v.n))
      return FPI8_INVALID_STATE;
  }
  for (uint32_t i = 0; phase > 0 && i < n; i++)
    if (id_at(i) >= v.n) return FPI8_INVALID_STATE;
  uint8_t joined[256];
  uint64_t done = 0;
  e = 0;
  while (done < max_units) {
    if (phase == 0) {
      // the opening token, then a single space's token when there is text
      set_id(0, 1);
      n = 1;
      if (pb > 0) {
        const uint8_t space = ' ';
        const int64_t s = vocab_lookup(v, &space, 1);
        set_id(n++, s >= 0 ? (uint32_t)s : space + 3u);
      }
      wr32(pages + PG_NIDS, n);
      wr32(pages + PG_NEXT_BYTE, 0);
      phase = 1;
    } else if (phase == 1) {
      const uint32_t i = rd32(pages + PG_NEXT_BYTE);
      if (i >= pb) {
        phase = 2;
        wr32(pages + PG_PAIR, 0);
        wr32(pages + PG_BEST_AT, kNone);
        wr32(pages + PG_BEST_SCORE, 0);
        wr32(pages + PG_BEST_ID, 0);
      } else {
        // one UTF-8 character: a lead byte and up to three continuation bytes
        uint32_t j = i + 1;
        while (j < pb && j - i < 4 && (prompt[j] & 0xC0) == 0x80) j++;
        const int64_t t = vocab_lookup(v, prompt + i, j - i);
        if (t >= 0) {
          set_id(n++, (uint32_t)t);
        } else {
          for (uint32_t k = i; k < j; k++) set_id(n++, prompt[k] + 3u);
        }
        wr32(pages + PG_NIDS, n);
        wr32(pages + PG_NEXT_BYTE, j);
      }
    } else {
      const uint32_t k = rd32(pages + PG_PAIR);
      if (k + 1 < n) {
        // one pair of the scan
        const uint32_t a = id_at(k), b = id_at(k + 1);
        const uint32_t na = v.piece_len(a), nb = v.piece_len(b);
        memcpy(joined, v.piece(a), na);
        memcpy(joined + na, v.piece(b), nb);
        const int64_t t = vocab_lookup(v, joined, na + nb);
        if (t >= 0) {
          const uint32_t sc = v.at(v.score, (uint32_t)t);
          if (rd32(pages + PG_BEST_AT) == kNone || sc > rd32(pages + PG_BEST_SCORE)) {
            wr32(pages + PG_BEST_AT, k);
            wr32(pages + PG_BEST_SCORE, sc);
            wr32(pages + PG_BEST_ID, (uint32_t)t);
          }
        }
        wr32(pages + PG_PAIR, k + 1);
      } else if (rd32(pages + PG_BEST_AT) != kNone) {
        // the scan's end: its best pair becomes one token
        const uint32_t at = rd32(pages + PG_BEST_AT);
        set_id(at, rd32(pages + PG_BEST_ID));
        memmove(ids + 4ull * (at + 1), ids + 4ull * (at + 2), 4ull * (n - at - 2));
        set_id(n - 1, 0);
        wr32(pages + PG_NIDS, --n);
        wr32(pages + PG_PAIR, 0);
        wr32(pages + PG_BEST_AT, kNone);
        wr32(pages + PG_BEST_SCORE, 0);
        wr32(pages + PG_BEST_ID, 0);
      } else {
        // no pair merges: the prompt's tokens and max tokens must fit
        if ((uint64_t)n + mx - 1 > c.context) { e = FPI8_CONTEXT_EXCEEDED; break; }
        wr32(pages + PG_PAIR, 0);
        wr32(pages + PG_BEST_AT, 0);
        wr32(pages + PG_POSITION, 0);
        wr32(pages + PG_TOKEN, id_at(0));
        phase = 3;
      }
    }
    wr32(pages + PG_PHASE, phase);
    done++;
    if (phase == 3) break;
  }
  if (units_done) *units_done = done;
  return e;
}

uint64_t fpi8_pages_state_size(const uint32_t cfg[7], uint32_t prompt_bytes, uint32_t max_tokens) {
  Cfg c;
  PagesLayout L;
  if (!cfg || !cfg_from_words(cfg, &c) || !pages_layout(c, prompt_bytes, max_tokens, &L))
    return UINT64_MAX;
  return L.total;
}

int32_t fpi8_state_export(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *state,
                          uint64_t state_len, const uint8_t *prompt, uint32_t prompt_len,
                          uint8_t *out, uint64_t out_len) {
  Model m;
  if (!h_section0) return FPI8_INVALID_FORMAT;
  int32_t e = parse_section0(h_section0, section0_len, UINT64_MAX, &m);
  if (e) return e;
  const Cfg &c = m.cfg;
  fpi8_info info;
  if (!state || fpi8_state_info(state, state_len, &info) != 0 || info.error != 0 || info.phase < 3 ||
      info.phase > 20)
    return FPI8_INVALID_STATE;
  StateLayout S;
  if (!state_layout(c, info.n_ids, info.max_tokens, &S) || S.total != state_len)
    return FPI8_INVALID_STATE;
  if ((prompt_len > 0 && !prompt) || prompt_len > 1024 || info.n_ids > prompt_len + 2)
    return FPI8_INVALID_PROMPT;
  PagesLayout P;
  pages_layout(c, prompt_len, info.max_tokens, &P);
  if (!out || out_len != P.total) return FPI8_BUFFER_TOO_SMALL;
  // the text of the generated tokens (fpi8_output_text's rules)
  std::vector<uint8_t> text(128ull * info.max_tokens);
  uint64_t text_len = 0;
  e = fpi8_output_text(h_section0, section0_len, state, state_len, text.data(), text.size(),
                       &text_len);
  if (e) return e;
  memset(out, 0, out_len);
  memcpy(out, kPagesTag, 8);
  memcpy(out + 8, state + 8, 20);                          // phase, layer, row, position, token
  wr32(out + 28, prompt_len);
  memcpy(out + 32, state + 32, 16);                        // prompt tokens, max, temperature, generated
  wr32(out + 48, (uint32_t)text_len);
  wr32(out + 52, prompt_len);                              // the tokenizer has read the prompt
  memcpy(out + 72, state + 72, ST_HEADER - 72);            // generator, turns, attention, sampling
  if (prompt_len) memcpy(out + P.prompt, prompt, prompt_len);
  memcpy(out + P.ids, state + S.ids, 4ull * info.n_ids);
  memcpy(out + P.out, state + S.out, 4ull * info.max_tokens);
  memcpy(out + P.text, text.data(), text_len);
  memcpy(out + P.x, state + S.x, S.logits - S.x);          // x, three working vectors, gate, up
  memcpy(out + P.logits, state + S.logits, 8ull * c.vocab);
  memcpy(out + P.scores, state + S.scores, 8ull * S.cachepos);
  copy_cache(c, state + S.keys, S.cachepos, false, out + P.keys, P.cachepos, true, S.cachepos);
  copy_cache(c, state + S.values, S.cachepos, false, out + P.values, P.cachepos, true, S.cachepos);
  return 0;
}

int32_t fpi8_state_import(const uint32_t cfg[7], const uint8_t *pages, uint64_t pages_len,
                          uint8_t *state, uint64_t state_len) {
  Cfg c;
  if (!cfg || !cfg_from_words(cfg, &c)) return FPI8_INVALID_CONFIG;
  if (!pages || pages_len < ST_HEADER || memcmp(pages, kPagesTag, 8) != 0) return FPI8_INVALID_STATE;
  const uint32_t prompt_len = rd32(pages + 28), n_ids = rd32(pages + 32), mx = rd32(pages + 36);
  const uint32_t phase = rd32(pages + 8);
  PagesLayout P;
  StateLayout S;
  if (!pages_layout(c, prompt_len, mx, &P) || P.total != pages_len) return FPI8_INVALID_STATE;
  if (phase < 3 || phase > 20 || n_ids == 0 || n_ids > prompt_len + 2 ||
      !state_layout(c, n_ids, mx, &S))
    return FPI8_INVALID_STATE;
  if (!state || state_len != S.total) return FPI8_BUFFER_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(state) & 7) != 0) return FPI8_INVALID_STATE;
  memset(state, 0, state_len);
  memcpy(state, kStateTag, 8);
  memcpy(state + 8, pages + 8, 20);
  memcpy(state + 32, pages + 32, 16);
  wr32(state + ST_CACHEPOS, S.cachepos);
  memcpy(state + 72, pages + 72, ST_HEADER - 72);
  memcpy(state + S.ids, pages + P.ids, 4ull * n_ids);
  memcpy(state + S.out, pages + P.out, 4ull * mx);
  memcpy(state + S.x, pages + P.x, S.logits - S.x);
  memcpy(state + S.logits, pages + P.logits, 8ull * c.vocab);
  memcpy(state + S.scores, pages + P.scores, 8ull * S.cachepos);
  copy_cache(c, pages + P.keys, P.cachepos, true, state + S.keys, S.cachepos, false, S.cachepos);
  copy_cache(c, pages + P.values, P.cachepos, true, state + S.values, S.cachepos, false, S.cachepos);
  return 0;
}

}  // extern "C"
