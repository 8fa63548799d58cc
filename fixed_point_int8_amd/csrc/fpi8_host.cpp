// fpi8_host.cpp - host side of libfpi8: configuration, the run state, the
// weight artifact.  These functions touch no GPU.
//
// The state is the one of "The inference core" page, section "The resumable
// state": a 128-byte header, then 8-byte aligned buffers in the page's
// order.  With token ids fed in, the prompt bytes and output text are absent,
// the prompt-token buffer holds the ids and cache positions are
// ids + max_tokens - 1.  Keys and values are [layer][kv head][position][elem].
#include <string.h>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

namespace fpi8 {

static inline uint64_t up8(uint64_t n) { return (n + 7) & ~uint64_t(7); }
static inline uint32_t ld32(const uint8_t *p) { uint32_t v; memcpy(&v, p, 4); return v; }
static inline uint64_t ld64(const uint8_t *p) { uint64_t v; memcpy(&v, p, 8); return v; }
static inline void st32(uint8_t *p, uint32_t v) { memcpy(p, &v, 4); }
static inline void st64(uint8_t *p, uint64_t v) { memcpy(p, &v, 8); }

const char kStateTag[8] = {'F', 'P', 'I', '8', 'S', 'T', '0', '1'};

// Ranges of the seven configuration values (the page states none): all at
// least one, dim and hidden at most 65,536, layers at most 1,024, vocab at
// most 2^24, context at most 2^20, dim a multiple of heads, an even head
// size, heads a multiple of kv_heads.
bool cfg_from_words(const uint32_t w[7], Cfg *c) {
  c->dim = w[0]; c->hidden = w[1]; c->layers = w[2]; c->heads = w[3];
  c->kv_heads = w[4]; c->vocab = w[5]; c->context = w[6];
  for (int i = 0; i < 7; i++)
    if (w[i] == 0) return false;
  if (c->dim > 65536u || c->hidden > 65536u || c->layers > 1024u || c->vocab > (1u << 24) ||
      c->context > (1u << 20))
    return false;
  if (c->dim % c->heads != 0) return false;
  c->head = c->dim / c->heads;
  if ((c->head & 1u) != 0) return false;
  if (c->heads % c->kv_heads != 0) return false;
  c->kvd = c->kv_heads * c->head;
  return true;
}

bool state_layout(const Cfg &c, uint32_t n_ids, uint32_t max_tokens, StateLayout *L) {
  if (n_ids == 0 || max_tokens == 0 || max_tokens > c.context) return false;
  if (uint64_t(n_ids) + max_tokens - 1 > c.context) return false;
  L->cachepos = n_ids + max_tokens - 1;
  uint64_t o = ST_HEADER;
  L->ids = o;     o += up8(4ull * n_ids);
  L->out = o;     o += up8(4ull * max_tokens);
  L->x = o;       o += up8(8ull * c.dim);
  L->w1 = o;      o += up8(8ull * c.dim);
  L->w2 = o;      o += up8(8ull * c.dim);
  L->w3 = o;      o += up8(8ull * c.dim);
  L->gate = o;    o += up8(8ull * c.hidden);
  L->up = o;      o += up8(8ull * c.hidden);
  L->logits = o;  o += up8(8ull * c.vocab);
  L->scores = o;  o += up8(8ull * L->cachepos);
  L->keys = o;    o += up8(4ull * c.layers * L->cachepos * c.kvd);
  L->values = o;  o += up8(4ull * c.layers * L->cachepos * c.kvd);
  L->total = o;
  return true;
}

// Checks one header read back from the device.  Returns 0 for a run that
// can advance, -1 for a complete run, 3 for anything else.
int check_header(const Cfg &c, const uint8_t *h, uint64_t stride, StateLayout *L) {
  if (memcmp(h, kStateTag, 8) != 0) return FPI8_INVALID_STATE;
  uint32_t n_ids = ld32(h + ST_NIDS), mx = ld32(h + ST_MAX);
  if (!state_layout(c, n_ids, mx, L) || L->total > stride) return FPI8_INVALID_STATE;
  if (ld32(h + ST_CACHEPOS) != L->cachepos) return FPI8_INVALID_STATE;
  if (ld32(h + ST_ERROR) != 0) return FPI8_INVALID_STATE;
  // The cursor: phase 3 (a position's start), 4-16 with a layer, 17-19
  // only where the position generates, or 20 (complete); inside a matrix
  // phase a row below its rows, inside attention a head, a stage 0-3 and an
  // index below the stage's units (with a sum of exponentials once stage 1
  // has ended), inside sampling a pass 0-2 (1 and 2 above temperature zero)
  // and an entry below the vocabulary (in the draw pass a remainder below
  // the sum).  Every other sub-phase field is zero.
  const uint32_t phase = ld32(h + ST_PHASE), layer = ld32(h + ST_LAYER);
  if (phase == 20 && layer == 0) return -1;
  if (phase < 3 || phase > 19) return FPI8_INVALID_STATE;
  if ((phase >= 4 && phase <= 16) ? layer >= c.layers : layer != 0) return FPI8_INVALID_STATE;
  uint32_t pos = ld32(h + ST_POSITION), gen = ld32(h + ST_GENERATED);
  if (phase >= 17 && pos + 1 < n_ids) return FPI8_INVALID_STATE;
  if (pos >= L->cachepos) return FPI8_INVALID_STATE;
  if (gen != (pos + 1 > n_ids ? pos + 1 - n_ids : 0)) return FPI8_INVALID_STATE;
  const uint32_t temp = ld32(h + ST_TEMP);
  if (ld32(h + ST_TOKEN) >= c.vocab || temp > (16u << 16)) return FPI8_INVALID_STATE;
  const uint32_t row = ld32(h + ST_ROW), stage = ld32(h + ST_STAGE), index = ld32(h + ST_INDEX);
  const uint32_t pass = ld32(h + ST_PASS);
  uint64_t sum, rem;
  memcpy(&sum, h + ST_SUM, 8);
  memcpy(&rem, h + ST_REMAINDER, 8);
  if (phase == 9) {
    if (row >= c.heads || stage > 3 || index >= (stage < 3 ? pos + 1 : c.head) || pass != 0)
      return FPI8_INVALID_STATE;
    if (stage >= 2 && sum == 0) return FPI8_INVALID_STATE;
  } else if (phase == 19) {
    if (pass > 2 || (pass > 0 && temp == 0) || row >= c.vocab || stage != 0 || index != 0)
      return FPI8_INVALID_STATE;
    if (pass == 2 && rem >= sum) return FPI8_INVALID_STATE;
  } else {
    uint32_t rows = 1;  // a phase that is one vector operation has no rows
    switch (phase) {
      case 5: case 10: case 15: rows = c.dim; break;
      case 6: case 7: rows = c.kvd; break;
      case 12: case 13: rows = c.hidden; break;
      case 18: rows = c.vocab; break;
      default: break;
    }
    if (row >= rows || stage != 0 || index != 0 || pass != 0) return FPI8_INVALID_STATE;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// The artifact (see include/fpi8.h for the layout).

static bool fits(uint64_t off, uint64_t size, uint64_t limit) {
  return off <= limit && size <= limit - off;
}

static void dims_of(const Cfg &c, uint32_t kind, uint32_t *rows, uint32_t *cols) {
  switch (kind) {
    case M_EMBED: case M_CLS: *rows = c.vocab; *cols = c.dim; break;
    case M_Q: case M_O: *rows = c.dim; *cols = c.dim; break;
    case M_K: case M_V: *rows = c.kvd; *cols = c.dim; break;
    case M_GATE: case M_UP: *rows = c.hidden; *cols = c.dim; break;
    default: *rows = c.dim; *cols = c.hidden; break;
  }
}

// Parses section zero.  `blob_len` is the length of the whole artifact (its
// matrix sections must lie inside it).  Fills `m` on success.
int parse_section0(const uint8_t *s0, uint64_t s0_len, uint64_t blob_len, Model *m) {
  if (s0_len < 128 + 16 || memcmp(s0, "CURTAW01", 8) != 0) return FPI8_INVALID_FORMAT;
  uint32_t words[7];
  for (int i = 0; i < 7; i++) words[i] = ld32(s0 + 8 + 4 * i);
  if (!cfg_from_words(words, &m->cfg)) return FPI8_INVALID_CONFIG;
  const Cfg &c = m->cfg;
  uint32_t nsec = ld32(s0 + 36), nmat = ld32(s0 + 40);
  m->inv = ld32(s0 + 44);
  uint64_t zero_len = ld64(s0 + 128 + 8);
  if (ld64(s0 + 128) != 0 || zero_len > blob_len || zero_len > s0_len) return FPI8_INVALID_FORMAT;
  if (nsec < 2 || nsec > 65536u || !fits(128, 16ull * nsec, zero_len)) return FPI8_INVALID_FORMAT;
  if (nmat != 2 + 7 * c.layers) return FPI8_INVALID_FORMAT;
  const uint64_t rope = 4ull * c.context * (c.head / 2);
  const uint64_t offs[6] = {ld64(s0 + 48), ld64(s0 + 56), ld64(s0 + 64), ld64(s0 + 72),
                            ld64(s0 + 80), ld64(s0 + 104)};
  const uint64_t sizes[6] = {4ull * 4097, 4ull * 4097, rope, rope,
                             4ull * (2ull * c.layers + 1) * c.dim, 32ull * nmat};
  for (int i = 0; i < 6; i++)
    if ((offs[i] & 7) != 0 || !fits(offs[i], sizes[i], zero_len)) return FPI8_INVALID_FORMAT;
  uint64_t tok = ld64(s0 + 88), tok_len = ld64(s0 + 96);
  if ((tok & 7) != 0 || !fits(tok, tok_len, zero_len)) return FPI8_INVALID_FORMAT;
  Vocab v;
  if (tok_len != 0 && !vocab_parse(s0 + tok, tok_len, c.vocab, &v)) return FPI8_INVALID_FORMAT;
  m->off_exp = offs[0]; m->off_silu = offs[1]; m->off_cos = offs[2]; m->off_sin = offs[3];
  m->off_norm = offs[4];
  if (ld32(s0 + offs[0]) == 0) return FPI8_INVALID_FORMAT;  // EXP[0] = 0: a zero sum is possible
  m->mats.assign(nmat, MatLoc{});
  std::vector<uint8_t> seen(nmat, 0);
  bool missing = false;
  for (uint32_t i = 0; i < nmat; i++) {
    const uint8_t *d = s0 + offs[5] + 32ull * i;
    uint32_t kind = ld32(d), layer = ld32(d + 4), rows = ld32(d + 8), cols = ld32(d + 12);
    uint32_t sec = ld32(d + 16);
    uint64_t off = ld64(d + 24);
    if (kind >= M_KINDS) return FPI8_INVALID_FORMAT;
    uint32_t er, ec;
    dims_of(c, kind, &er, &ec);
    if (rows != er || cols != ec) return FPI8_INVALID_FORMAT;
    uint32_t slot;
    if (kind == M_EMBED || kind == M_CLS) {
      if (layer != 0) return FPI8_INVALID_FORMAT;
      slot = kind == M_EMBED ? 0 : 1 + 7 * c.layers;
    } else {
      if (layer >= c.layers) return FPI8_INVALID_FORMAT;
      slot = 1 + 7 * layer + (kind - M_Q);
    }
    if (seen[slot]) return FPI8_INVALID_FORMAT;
    seen[slot] = 1;
    if (sec == 0 || sec >= nsec || (off & 7) != 0) return FPI8_INVALID_FORMAT;
    uint64_t so = ld64(s0 + 128 + 16ull * sec), sl = ld64(s0 + 128 + 16ull * sec + 8);
    if ((so & 7) != 0) return FPI8_INVALID_FORMAT;
    uint64_t wbytes = uint64_t(rows) * cols;
    uint64_t need = up8(wbytes) + 4ull * rows;
    if (!fits(so, sl, blob_len) || !fits(off, need, sl)) { missing = true; continue; }
    MatLoc &ml = m->mats[slot];
    ml.w = so + off;
    ml.s = so + off + up8(wbytes);
    ml.rows = rows;
    ml.cols = cols;
  }
  if (missing) return FPI8_MISSING_WEIGHTS;
  return 0;
}

}  // namespace fpi8

using namespace fpi8;

extern "C" {

uint64_t fpi8_state_size(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens) {
  Cfg c;
  StateLayout L;
  if (!cfg || !cfg_from_words(cfg, &c) || !state_layout(c, n_ids, max_tokens, &L))
    return UINT64_MAX;
  return L.total;
}

int32_t fpi8_state_offsets(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens,
                           uint64_t out[13]) {
  Cfg c;
  StateLayout L;
  if (!cfg || !cfg_from_words(cfg, &c)) return FPI8_INVALID_CONFIG;
  if (!state_layout(c, n_ids, max_tokens, &L)) return FPI8_INVALID_PROMPT;
  const uint64_t v[13] = {L.ids, L.out, L.x, L.w1, L.w2, L.w3, L.gate, L.up,
                          L.logits, L.scores, L.keys, L.values, L.total};
  memcpy(out, v, sizeof v);
  return 0;
}

int32_t fpi8_blob_check(const uint8_t *blob, uint64_t len, uint32_t cfg_out[7]) {
  if (!blob) return FPI8_INVALID_FORMAT;
  Model m;
  int32_t e = parse_section0(blob, len, len, &m);
  if (e == 0 && cfg_out) {
    const uint32_t v[7] = {m.cfg.dim, m.cfg.hidden, m.cfg.layers, m.cfg.heads,
                           m.cfg.kv_heads, m.cfg.vocab, m.cfg.context};
    memcpy(cfg_out, v, sizeof v);
  }
  return e;
}

int32_t fpi8_init_state(const uint32_t cfg[7], uint8_t *state, uint64_t state_len,
                        const uint32_t *ids, uint32_t n_ids, uint32_t max_tokens,
                        uint32_t temperature_q16, uint64_t seed) {
  Cfg c;
  if (!cfg || !cfg_from_words(cfg, &c)) return FPI8_INVALID_CONFIG;
  if (n_ids == 0 || !ids || max_tokens == 0 || max_tokens > c.context ||
      temperature_q16 > (16u << 16))
    return FPI8_INVALID_PROMPT;
  for (uint32_t i = 0; i < n_ids; i++)
    if (ids[i] >= c.vocab) return FPI8_INVALID_PROMPT;
  if (uint64_t(n_ids) + max_tokens - 1 > c.context) return FPI8_CONTEXT_EXCEEDED;
  StateLayout L;
  state_layout(c, n_ids, max_tokens, &L);
  if (!state || state_len != L.total) return FPI8_BUFFER_TOO_SMALL;
  if ((reinterpret_cast<uintptr_t>(state) & 7) != 0) return FPI8_INVALID_STATE;
  memset(state, 0, state_len);
  memcpy(state, kStateTag, 8);
  st32(state + ST_PHASE, 3);
  st32(state + ST_TOKEN, ids[0]);
  st32(state + ST_NIDS, n_ids);
  st32(state + ST_MAX, max_tokens);
  st32(state + ST_TEMP, temperature_q16);
  st32(state + ST_CACHEPOS, L.cachepos);
  // A zero seed starts the generator at 0x9E3779B97F4A7C15 ("Sampling").
  st64(state + ST_GENERATOR, seed != 0 ? seed : 0x9E3779B97F4A7C15ull);
  memcpy(state + L.ids, ids, 4ull * n_ids);
  return 0;
}

int32_t fpi8_state_info(const uint8_t *state, uint64_t len, fpi8_info *out) {
  if (!state || !out || (reinterpret_cast<uintptr_t>(state) & 7) != 0 || len < ST_HEADER ||
      memcmp(state, kStateTag, 8) != 0)
    return FPI8_INVALID_STATE;
  out->phase = ld32(state + ST_PHASE);
  out->layer = ld32(state + ST_LAYER);
  out->position = ld32(state + ST_POSITION);
  out->token = ld32(state + ST_TOKEN);
  out->n_ids = ld32(state + ST_NIDS);
  out->max_tokens = ld32(state + ST_MAX);
  out->temperature_q16 = ld32(state + ST_TEMP);
  out->generated = ld32(state + ST_GENERATED);
  out->cache_positions = ld32(state + ST_CACHEPOS);
  out->error = ld32(state + ST_ERROR);
  out->complete = out->phase == 20;
  out->reserved = 0;
  out->generator = ld64(state + ST_GENERATOR);
  out->turns = ld64(state + ST_TURNS);
  return 0;
}

const uint32_t *fpi8_output_tokens(const uint8_t *state, uint64_t len, uint32_t *count) {
  fpi8_info info;
  if (fpi8_state_info(state, len, &info) != 0) return nullptr;
  uint64_t out = ST_HEADER + up8(4ull * info.n_ids);
  if (out + 4ull * info.max_tokens > len || info.generated > info.max_tokens) return nullptr;
  if (count) *count = info.generated;
  return reinterpret_cast<const uint32_t *>(state + out);
}

}  // extern "C"
