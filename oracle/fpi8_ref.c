/*
 * fpi8_ref.c - the oracle of the fixed-point forward pass (plain C, CPU).
 *
 * TEST INFRASTRUCTURE: the literal, slow reading of the curta-core inference
 * core ("The inference core" page) that the GPU library is checked against.
 * Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * The page defines the method by its integer arithmetic, so this file is
 * that arithmetic written out in the page's order: the phases of "The
 * forward pass, in order", the stages of "Attention, stage by stage" and the
 * passes of "Sampling".  Where the page leaves a step open, the reading taken
 * is stated at the step.  Loops over the rows of a matrix may run on several
 * threads; every output word is still computed whole, in the stated order.
 *
 * Build: gcc -std=c11 -O2 -fopenmp -shared -fPIC fpi8_ref.c -o libfpi8_ref.so
 */
#include "fpi8_ref.h"

#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* 64-bit helpers.  Wrapping arithmetic is done on uint64_t (defined in C);
 * the conversion back to int64_t is modulo 2^64 (GCC's documented rule).   */

static inline int64_t wadd(int64_t a, int64_t b) { return (int64_t)((uint64_t)a + (uint64_t)b); }
static inline int64_t wsub(int64_t a, int64_t b) { return (int64_t)((uint64_t)a - (uint64_t)b); }
static inline int64_t wmul(int64_t a, int64_t b) { return (int64_t)((uint64_t)a * (uint64_t)b); }

/* Arithmetic (flooring) right shift, written without relying on the
 * implementation-defined shift of a negative value. */
static inline int64_t asr(int64_t v, unsigned s) {
  return v >= 0 ? (int64_t)((uint64_t)v >> s) : (int64_t)~((~(uint64_t)v) >> s);
}

static inline uint32_t rd32(const uint8_t *p) { uint32_t v; memcpy(&v, p, 4); return v; }
static inline uint64_t rd64(const uint8_t *p) { uint64_t v; memcpy(&v, p, 8); return v; }
static inline void wr32(uint8_t *p, uint32_t v) { memcpy(p, &v, 4); }
static inline void wr64(uint8_t *p, uint64_t v) { memcpy(p, &v, 8); }
static inline uint64_t a8(uint64_t n) { return (n + 7) & ~(uint64_t)7; }

static int g_threads = 1;

int32_t fpi8_ref_set_threads(int32_t n) {
  if (n < 1) n = 1;
#ifdef _OPENMP
  g_threads = n;
#else
  g_threads = 1;
#endif
  return g_threads;
}

/* ---------------------------------------------------------------------- */
/* Primitives                                                             */

/* "RMS normalization": integer square root, the largest r with r*r <= n.
 * Binary search over r in [0, 2^32), where r*r cannot overflow. */
uint64_t fpi8_ref_isqrt(uint64_t n) {
  uint64_t lo = 0, hi = 0xFFFFFFFFull;
  while (lo < hi) {
    uint64_t mid = lo + (hi - lo + 1) / 2;
    if (mid * mid <= n) lo = mid; else hi = mid - 1;
  }
  return lo;
}

/* "A matrix row": sum of the inputs once per vector, the unsigned bytes
 * times the inputs, then y = ((acc - 128*sum) * scale) >> 24, all in
 * wrapping 64-bit arithmetic.  The scale is an unsigned 32-bit value and
 * enters the product zero-extended. */
int64_t fpi8_ref_row(const uint8_t *w, uint32_t scale, const int64_t *x, uint32_t n) {
  int64_t sum = 0, acc = 0;
  for (uint32_t c = 0; c < n; c++) sum = wadd(sum, x[c]);
  for (uint32_t c = 0; c < n; c++) acc = wadd(acc, wmul((int64_t)w[c], x[c]));
  int64_t t = wsub(acc, wmul(128, sum));
  return asr(wmul(t, (int64_t)(uint64_t)scale), 24);
}

void fpi8_ref_rows(const uint8_t *W, const uint32_t *scales, uint32_t rows,
                   uint32_t cols, const int64_t *x, uint32_t batch, int64_t *y) {
  for (uint32_t b = 0; b < batch; b++) {
    const int64_t *xb = x + (uint64_t)b * cols;
    int64_t *yb = y + (uint64_t)b * rows;
    int64_t r;
#pragma omp parallel for schedule(static) num_threads(g_threads) if (g_threads > 1)
    for (r = 0; r < (int64_t)rows; r++)
      yb[r] = fpi8_ref_row(W + (uint64_t)r * cols, scales[r], xb, cols);
  }
}

/* "RMS normalization": rms = isqrt(sum(x*x) / d + 42,950), at least 1;
 * y = ((x * w) / rms) >> 8 with the division truncating toward zero.
 * Reading: the squares wrap like every 64-bit product and are summed as
 * unsigned 64-bit words, and the mean is an unsigned division; the weight
 * (i32) is sign-extended. */
void fpi8_ref_rmsnorm(const int64_t *x, const int32_t *w, uint32_t d, int64_t *y) {
  uint64_t ss = 0;
  for (uint32_t i = 0; i < d; i++) ss += (uint64_t)wmul(x[i], x[i]);
  uint64_t rms = fpi8_ref_isqrt(ss / d + 42950u);
  if (rms < 1) rms = 1;
  for (uint32_t i = 0; i < d; i++) {
    int64_t p = wmul(x[i], (int64_t)w[i]);
    y[i] = asr(p / (int64_t)rms, 8);
  }
}

/* Phase 8: a pair (a, b) turned by the angle whose cosine and sine are c
 * and s at Q24: a' = (a*c - b*s) >> 24, b' = (a*s + b*c) >> 24. */
void fpi8_ref_rotate(int64_t *a, int64_t *b, int32_t c, int32_t s) {
  int64_t A = *a, B = *b;
  *a = asr(wsub(wmul(A, c), wmul(B, s)), 24);
  *b = asr(wadd(wmul(A, s), wmul(B, c)), 24);
}

/* "Lookup tables", exponential: a difference selects entry d >> 8, and
 * every difference past the table's end selects its last entry, 4,096.
 * Reading: d is a non-negative difference, taken as an unsigned word. */
uint32_t fpi8_ref_exp_index(uint64_t d) {
  uint64_t i = d >> 8;
  return i > 4096 ? 4096u : (uint32_t)i;
}

/* "Lookup tables", SiLU: 16 or more returns the input, -16 or less returns
 * zero, otherwise entry (x + 16) >> 9 in Q16, that is (x + 2^20) >> 9. */
int64_t fpi8_ref_silu(int64_t x, const int32_t *tab) {
  const int64_t sixteen = (int64_t)16 << 16;
  if (x >= sixteen) return x;
  if (x <= -sixteen) return 0;
  return (int64_t)tab[(x + sixteen) >> 9];
}

/* "Attention, stage by stage", one head, p = npos positions:
 *   scores: s_j = (((q . K_j) >> 16) * inv) >> 24, keep the largest;
 *   exponentials: e_j = EXP[index(max - s_j)], keep their sum;
 *   normalization: p_j = (e_j << 24) / sum;
 *   weighted values: o_i = (sum_j p_j * V_j,i) >> 24.
 * The one scores buffer carries s, then e, then p, as the state has one.
 * inv enters zero-extended; cached words are sign-extended.
 *
 * A head can stop after any unit of a stage ("The resumable state"): one
 * position in stages 0 to 2, one output element in stage 3.  The cursor is
 * the stage, the index of the next unit, the largest score and the sum of
 * exponentials; the scores buffer and the outputs hold the rest. */
typedef struct {
  uint32_t stage, index;
  int64_t max;
  uint64_t sum;
} attn_cursor;

/* One unit at the cursor; returns 1 when it was the head's last. */
static int attention_unit(const int64_t *q, const int32_t *K, const int32_t *V, uint32_t npos,
                          uint32_t head, uint64_t stride, uint32_t inv_sqrt_head,
                          const uint32_t *exp_tab, int64_t *scores, int64_t *out,
                          attn_cursor *c) {
  const uint32_t j = c->index;
  switch (c->stage) {
    case 0: {
      const int32_t *k = K + (uint64_t)j * stride;
      int64_t dot = 0;
      for (uint32_t i = 0; i < head; i++) dot = wadd(dot, wmul(q[i], (int64_t)k[i]));
      int64_t s = asr(wmul(asr(dot, 16), (int64_t)(uint64_t)inv_sqrt_head), 24);
      scores[j] = s;
      if (j == 0 || s > c->max) c->max = s;
      break;
    }
    case 1: {
      if (j == 0) c->sum = 0;
      uint64_t d = (uint64_t)c->max - (uint64_t)scores[j];
      uint32_t e = exp_tab[fpi8_ref_exp_index(d)];
      scores[j] = (int64_t)e;
      c->sum += e;
      break;
    }
    case 2:
      scores[j] = (int64_t)(((uint64_t)scores[j] << 24) / c->sum);
      break;
    default: {
      int64_t acc = 0;
      for (uint32_t t = 0; t < npos; t++)
        acc = wadd(acc, wmul(scores[t], (int64_t)V[(uint64_t)t * stride + j]));
      out[j] = asr(acc, 24);
      break;
    }
  }
  c->index = j + 1;
  if (c->index < (c->stage < 3 ? npos : head)) return 0;
  c->index = 0;
  return c->stage++ == 3;
}

void fpi8_ref_attention_head(const int64_t *q, const int32_t *K, const int32_t *V,
                             uint32_t npos, uint32_t head, uint64_t stride,
                             uint32_t inv_sqrt_head, const uint32_t *exp_tab,
                             int64_t *scores, int64_t *out,
                             int64_t *max_out, uint64_t *sum_out) {
  attn_cursor c = {0, 0, 0, 0};
  while (!attention_unit(q, K, V, npos, head, stride, inv_sqrt_head, exp_tab, scores, out, &c)) {
  }
  if (max_out) *max_out = c.max;
  if (sum_out) *sum_out = c.sum;
}

/* "Sampling": xorshift64* with the run's seed as its first state. */
uint64_t fpi8_ref_xorshift64s(uint64_t *state) {
  uint64_t x = *state;
  x ^= x >> 12;
  x ^= x << 25;
  x ^= x >> 27;
  *state = x;
  return x * 0x2545F4914F6CDD1Dull;
}

/* Temperature step of the sum and draw passes: the difference divided by
 * the temperature.  Reading: both are Q16, so the quotient at Q16 is
 * floor(d * 2^16 / T), computed exactly in 128 bits, then indexed like a
 * score difference. */
static uint32_t temp_index(uint64_t d, uint32_t t) {
  unsigned __int128 q = ((unsigned __int128)d << 16) / t;
  unsigned __int128 i = q >> 8;
  return i > 4096 ? 4096u : (uint32_t)i;
}

/* "Sampling": the maximum pass (the lowest index wins a tie, the first
 * found in a forward scan); at temperature zero its index is the token.
 * Above zero: the sum pass, one advance of the generator, the draw modulo
 * the sum, and the walk that subtracts each entry's exponential.
 *
 * A pass can stop after any vocabulary entry ("The resumable state"): the
 * cursor is the pass, the next entry, the largest logit, the entry chosen so
 * far, the sum of exponentials and what is left of the draw.  The generator
 * advances when the sum pass ends. */
typedef struct {
  uint32_t pass, row, chosen;
  int64_t max;
  uint64_t sum, rem;
} sample_cursor;

/* One entry at the cursor; returns 1 when the token is chosen (c->chosen). */
static int sample_unit(const int64_t *logits, uint32_t vocab, uint32_t temperature_q16,
                       const uint32_t *exp_tab, uint64_t *generator, sample_cursor *c) {
  const uint32_t i = c->row;
  c->row = i + 1;
  if (c->pass == 0) {
    if (i == 0 || logits[i] > c->max) { c->max = logits[i]; c->chosen = i; }
    if (c->row < vocab) return 0;
    if (temperature_q16 == 0) return 1;
    c->pass = 1;
    c->row = 0;
    return 0;
  }
  const uint64_t e = exp_tab[temp_index((uint64_t)c->max - (uint64_t)logits[i], temperature_q16)];
  if (c->pass == 1) {
    if (i == 0) c->sum = 0;
    c->sum += e;
    if (c->row < vocab) return 0;
    c->rem = fpi8_ref_xorshift64s(generator) % c->sum;
    c->pass = 2;
    c->row = 0;
    return 0;
  }
  if (c->rem < e || c->row == vocab) { /* the second is not reached: rem < sum */
    c->chosen = i;
    return 1;
  }
  c->rem -= e;
  return 0;
}

uint32_t fpi8_ref_sample(const int64_t *logits, uint32_t vocab, uint32_t temperature_q16,
                         const uint32_t *exp_tab, uint64_t *generator) {
  sample_cursor c = {0, 0, 0, 0, 0, 0};
  while (!sample_unit(logits, vocab, temperature_q16, exp_tab, generator, &c)) {
  }
  return c.chosen;
}

/* ---------------------------------------------------------------------- */
/* Configuration ("WebAssembly exports": seven u32 values in order).
 * Reading of the order: dim, hidden, layers, heads, kv_heads, vocab,
 * context.  Ranges (the page gives none): every count at least one, the
 * head size even (rotary pairs), heads a multiple of kv_heads, dim and
 * hidden at most 65,536, layers at most 1,024, vocab at most 2^24 and
 * context at most 2^20.                                                   */

typedef struct {
  uint32_t dim, hidden, layers, heads, kv_heads, vocab, context;
  uint32_t head, kvd;
} cfg_t;

static int cfg_read(const uint32_t c[7], cfg_t *o) {
  o->dim = c[0]; o->hidden = c[1]; o->layers = c[2]; o->heads = c[3];
  o->kv_heads = c[4]; o->vocab = c[5]; o->context = c[6];
  if (!o->dim || !o->hidden || !o->layers || !o->heads || !o->kv_heads || !o->vocab ||
      !o->context) return 0;
  if (o->dim > 65536 || o->hidden > 65536 || o->layers > 1024 || o->vocab > (1u << 24) ||
      o->context > (1u << 20)) return 0;
  if (o->dim % o->heads) return 0;
  o->head = o->dim / o->heads;
  if (o->head % 2) return 0;
  if (o->heads % o->kv_heads) return 0;
  o->kvd = o->kv_heads * o->head;
  return 1;
}

/* ---------------------------------------------------------------------- */
/* "The resumable state": a 128-byte header, then buffers each starting at
 * a multiple of eight bytes, in the page's order.  With ids fed in, the
 * prompt bytes and output text are absent and the prompt-token buffer holds
 * the ids; cache positions are n_ids + max_tokens - 1.  Keys and values are
 * laid out [layer][kv head][cache position][head element].              */

#define H_TAG 0
#define H_PHASE 8
#define H_LAYER 12
#define H_ROW 16
#define H_POSITION 20
#define H_TOKEN 24
#define H_ERROR 28
#define H_NIDS 32
#define H_MAX 36
#define H_TEMP 40
#define H_GENERATED 44
#define H_CACHEPOS 48
#define H_GENERATOR 72
#define H_TURNS 80
#define H_MAXSCORE 88
#define H_CHOSEN 96
#define H_PASS 100
#define H_SUM 104
#define H_REMAINDER 112
#define H_STAGE 120
#define H_INDEX 124
#define HEADER 128

static const char STATE_TAG[8] = {'F', 'P', 'I', '8', 'S', 'T', '0', '1'};

/* The shared tail of the buffer table: activations and three working
 * vectors, gate and up, logits, scores, keys, values. */
static uint64_t tail_layout(const cfg_t *c, uint64_t o, uint32_t cachepos, fpi8_ref_layout *L) {
  L->x = o; o += a8(8ull * c->dim);
  L->w1 = o; o += a8(8ull * c->dim);
  L->w2 = o; o += a8(8ull * c->dim);
  L->w3 = o; o += a8(8ull * c->dim);
  L->gate = o; o += a8(8ull * c->hidden);
  L->up = o; o += a8(8ull * c->hidden);
  L->logits = o; o += a8(8ull * c->vocab);
  L->scores = o; o += a8(8ull * cachepos);
  L->keys = o; o += a8(4ull * c->layers * cachepos * c->kvd);
  L->values = o; o += a8(4ull * c->layers * cachepos * c->kvd);
  return o;
}

static int layout_ids(const cfg_t *c, uint32_t n_ids, uint32_t max_tokens, fpi8_ref_layout *L) {
  if (n_ids == 0 || max_tokens == 0 || max_tokens > c->context) return 0;
  if ((uint64_t)n_ids + max_tokens - 1 > c->context) return 0;
  memset(L, 0, sizeof *L);
  L->cache_positions = n_ids + max_tokens - 1;
  uint64_t o = HEADER;
  L->ids = o; o += a8(4ull * n_ids);
  L->out = o; o += a8(4ull * max_tokens);
  L->total = tail_layout(c, o, L->cache_positions, L);
  return 1;
}

uint64_t fpi8_ref_state_size(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens) {
  cfg_t c;
  fpi8_ref_layout L;
  if (!cfg_read(cfg, &c) || !layout_ids(&c, n_ids, max_tokens, &L)) return UINT64_MAX;
  return L.total;
}

int32_t fpi8_ref_state_layout(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens,
                              fpi8_ref_layout *out) {
  cfg_t c;
  if (!cfg_read(cfg, &c)) return FPI8_REF_INVALID_CONFIG;
  if (!layout_ids(&c, n_ids, max_tokens, out)) return FPI8_REF_INVALID_PROMPT;
  return 0;
}

/* Size of a run account in the page's own layout ("The resumable state"):
 * 256 bytes of account header, the 128-byte state header, the prompt bytes,
 * room for bytes + 2 prompt tokens, the output tokens, 128 text bytes per
 * output token, then the buffers both layouts share.  The cache holds
 * prompt bytes + max tokens + 1 positions, never more than the context. */
uint64_t fpi8_ref_pages_state_size(const uint32_t cfg[7], uint32_t prompt_bytes,
                                   uint32_t max_tokens) {
  cfg_t c;
  if (!cfg_read(cfg, &c) || prompt_bytes > 1024 || max_tokens == 0 || max_tokens > c.context)
    return UINT64_MAX;
  uint64_t cp = (uint64_t)prompt_bytes + max_tokens + 1;
  if (cp > c.context) cp = c.context;
  fpi8_ref_layout L;
  uint64_t o = HEADER;
  o += a8(prompt_bytes);
  o += a8(4ull * (prompt_bytes + 2));
  o += a8(4ull * max_tokens);
  o += a8(128ull * max_tokens);
  return 256 + tail_layout(&c, o, (uint32_t)cp, &L);
}

int32_t fpi8_ref_init_state(const uint32_t cfg[7], uint8_t *state, uint64_t state_len,
                            const uint32_t *ids, uint32_t n_ids, uint32_t max_tokens,
                            uint32_t temperature_q16, uint64_t seed) {
  cfg_t c;
  fpi8_ref_layout L;
  if (!cfg_read(cfg, &c)) return FPI8_REF_INVALID_CONFIG;
  if (n_ids == 0 || max_tokens == 0 || max_tokens > c.context ||
      temperature_q16 > (16u << 16)) return FPI8_REF_INVALID_PROMPT;
  for (uint32_t i = 0; i < n_ids; i++)
    if (ids[i] >= c.vocab) return FPI8_REF_INVALID_PROMPT;
  if ((uint64_t)n_ids + max_tokens - 1 > c.context) return FPI8_REF_CONTEXT_EXCEEDED;
  layout_ids(&c, n_ids, max_tokens, &L);
  if (state_len != L.total) return FPI8_REF_BUFFER_TOO_SMALL;
  if (((uintptr_t)state) & 7) return FPI8_REF_INVALID_STATE;
  memset(state, 0, state_len);
  memcpy(state + H_TAG, STATE_TAG, 8);
  wr32(state + H_PHASE, 3);
  wr32(state + H_TOKEN, ids[0]);
  wr32(state + H_NIDS, n_ids);
  wr32(state + H_MAX, max_tokens);
  wr32(state + H_TEMP, temperature_q16);
  wr32(state + H_CACHEPOS, L.cache_positions);
  /* "Sampling": seed 0 is replaced by the golden-ratio constant
   * 0x9E3779B97F4A7C15.  Reading: the replacement is made when the state
   * is opened. */
  wr64(state + H_GENERATOR, seed ? seed : 0x9E3779B97F4A7C15ull);
  memcpy(state + L.ids, ids, 4ull * n_ids);
  return 0;
}

int32_t fpi8_ref_state_info(const uint8_t *state, uint64_t len, fpi8_ref_info *o) {
  if (((uintptr_t)state) & 7 || len < HEADER || memcmp(state, STATE_TAG, 8))
    return FPI8_REF_INVALID_STATE;
  memset(o, 0, sizeof *o);
  o->phase = rd32(state + H_PHASE);
  o->layer = rd32(state + H_LAYER);
  o->position = rd32(state + H_POSITION);
  o->token = rd32(state + H_TOKEN);
  o->error = rd32(state + H_ERROR);
  o->n_ids = rd32(state + H_NIDS);
  o->max_tokens = rd32(state + H_MAX);
  o->temperature_q16 = rd32(state + H_TEMP);
  o->generated = rd32(state + H_GENERATED);
  o->cache_positions = rd32(state + H_CACHEPOS);
  o->generator = rd64(state + H_GENERATOR);
  o->turns = rd64(state + H_TURNS);
  o->complete = o->phase == 20;
  return 0;
}

/* ---------------------------------------------------------------------- */
/* The artifact.  Layout (the page fixes the tag, section zero and the
 * section table whose first entry's second u64 is section zero's length):
 *   0 tag CURTAW01 | 8 u32[7] config | 36 u32 sections | 40 u32 matrices
 *   44 u32 inv sqrt head (Q24) | 48 u64 exp | 56 u64 silu | 64 u64 cos
 *   72 u64 sin | 80 u64 norm | 88 u64 tokenizer | 96 u64 tokenizer length
 *   104 u64 matrix descriptors | 128 section table {u64 offset, u64 length}
 * Descriptor (32 B): kind, layer, rows, cols, section, 0, u64 offset.     */

#define SECTION_TABLE 128
enum { K_EMBED, K_Q, K_K, K_V, K_O, K_GATE, K_UP, K_DOWN, K_CLS, K_KINDS };

typedef struct {
  const uint8_t *w;
  const uint32_t *s; /* may be unaligned in a hostile artifact: read via memcpy */
  const uint8_t *s_bytes;
  uint32_t rows, cols;
} mat_t;

typedef struct {
  cfg_t c;
  const uint32_t *exp_tab;
  const int32_t *silu_tab, *cos_tab, *sin_tab, *norm;
  uint32_t inv;
  mat_t embed, cls;
  mat_t *layer; /* [layers][7] */
} model_t;

static void mat_dims(const cfg_t *c, uint32_t kind, uint32_t *r, uint32_t *k) {
  switch (kind) {
    case K_EMBED: case K_CLS: *r = c->vocab; *k = c->dim; break;
    case K_Q: case K_O: *r = c->dim; *k = c->dim; break;
    case K_K: case K_V: *r = c->kvd; *k = c->dim; break;
    case K_GATE: case K_UP: *r = c->hidden; *k = c->dim; break;
    default: *r = c->dim; *k = c->hidden; break; /* K_DOWN */
  }
}

static int in_range(uint64_t off, uint64_t size, uint64_t limit) {
  return off <= limit && size <= limit - off;
}

/* The tokenizer block of section zero, when the artifact has one (its
 * layout is this artifact format's: u32 n, u32 longest, u32 score[n], u32
 * start[n+1], u32 sorted_ids[n], pool): n is the vocabulary and holds the
 * 3 special and 256 byte tokens, every token has 1 to 128 bytes inside the
 * pool (a generated token's text has 128 bytes of output text), longest is
 * the longest, and sorted_ids lists every id once in increasing byte order
 * of the strings (a prefix first), so no two tokens share a string. */
static int piece_cmp(const uint8_t *pool, const uint8_t *start, uint32_t a, uint32_t b) {
  uint32_t a0 = rd32(start + 4ull * a), a1 = rd32(start + 4ull * a + 4);
  uint32_t b0 = rd32(start + 4ull * b), b1 = rd32(start + 4ull * b + 4);
  uint32_t la = a1 - a0, lb = b1 - b0;
  for (uint32_t i = 0; i < la && i < lb; i++)
    if (pool[a0 + i] != pool[b0 + i]) return pool[a0 + i] < pool[b0 + i] ? -1 : 1;
  return la < lb ? -1 : la > lb ? 1 : 0;
}

static int tokenizer_ok(const uint8_t *t, uint64_t len, uint32_t vocab) {
  if (len < 8) return 0;
  uint32_t n = rd32(t), longest = rd32(t + 4);
  if (n != vocab || n < 259) return 0;
  uint64_t head = 8 + 12ull * n + 4;
  if (head > len) return 0;
  const uint8_t *start = t + 8 + 4ull * n, *sorted = start + 4ull * (n + 1), *pool = t + head;
  uint32_t most = 0;
  for (uint32_t i = 0; i < n; i++) {
    uint32_t a = rd32(start + 4ull * i), b = rd32(start + 4ull * i + 4);
    if (b <= a || b - a > 128 || b > len - head) return 0;
    if (b - a > most) most = b - a;
  }
  if (rd32(start) != 0 && rd32(start) > len - head) return 0;
  if (most != longest) return 0;
  uint8_t *seen = (uint8_t *)calloc(n, 1);
  if (!seen) return 0;
  int ok = 1;
  for (uint32_t k = 0; k < n && ok; k++) {
    uint32_t id = rd32(sorted + 4ull * k);
    if (id >= n || seen[id]) { ok = 0; break; }
    seen[id] = 1;
    if (k > 0 && piece_cmp(pool, start, rd32(sorted + 4ull * (k - 1)), id) >= 0) ok = 0;
  }
  free(seen);
  return ok;
}

/* Parses and checks an artifact.  mats (if not NULL) receives the matrix
 * table: [0] embedding, [1 + 7*l + (kind-1)] layer matrices, [1 + 7L]
 * classifier. */
static int32_t parse(const uint8_t *blob, uint64_t len, model_t *m, mat_t *mats) {
  if (len < SECTION_TABLE + 16 || memcmp(blob, "CURTAW01", 8)) return FPI8_REF_INVALID_FORMAT;
  uint32_t raw[7];
  for (int i = 0; i < 7; i++) raw[i] = rd32(blob + 8 + 4 * i);
  if (!cfg_read(raw, &m->c)) return FPI8_REF_INVALID_CONFIG;
  const cfg_t *c = &m->c;
  uint32_t nsec = rd32(blob + 36), nmat = rd32(blob + 40);
  m->inv = rd32(blob + 44);
  uint64_t s0 = rd64(blob + SECTION_TABLE + 8);
  if (rd64(blob + SECTION_TABLE) != 0 || s0 > len) return FPI8_REF_INVALID_FORMAT;
  if (nsec < 2 || nsec > 65536 || !in_range(SECTION_TABLE, 16ull * nsec, s0))
    return FPI8_REF_INVALID_FORMAT;
  if (nmat != 2 + 7 * c->layers) return FPI8_REF_INVALID_FORMAT;
  uint64_t o_exp = rd64(blob + 48), o_silu = rd64(blob + 56), o_cos = rd64(blob + 64);
  uint64_t o_sin = rd64(blob + 72), o_norm = rd64(blob + 80), o_tok = rd64(blob + 88);
  uint64_t n_tok = rd64(blob + 96), o_desc = rd64(blob + 104);
  uint64_t rope = 4ull * c->context * (c->head / 2);
  uint64_t offs[6] = {o_exp, o_silu, o_cos, o_sin, o_norm, o_desc};
  uint64_t sizes[6] = {4 * 4097, 4 * 4097, rope, rope, 4ull * (2ull * c->layers + 1) * c->dim,
                       32ull * nmat};
  for (int i = 0; i < 6; i++)
    if ((offs[i] & 7) || !in_range(offs[i], sizes[i], s0)) return FPI8_REF_INVALID_FORMAT;
  if ((o_tok & 7) || !in_range(o_tok, n_tok, s0)) return FPI8_REF_INVALID_FORMAT;
  if (n_tok && !tokenizer_ok(blob + o_tok, n_tok, c->vocab)) return FPI8_REF_INVALID_FORMAT;
  m->exp_tab = (const uint32_t *)(blob + o_exp);
  m->silu_tab = (const int32_t *)(blob + o_silu);
  m->cos_tab = (const int32_t *)(blob + o_cos);
  m->sin_tab = (const int32_t *)(blob + o_sin);
  m->norm = (const int32_t *)(blob + o_norm);
  /* Reading: an exponential table whose first entry is zero could make the
   * sum of exponentials zero; such an artifact is rejected. */
  if (m->exp_tab[0] == 0) return FPI8_REF_INVALID_FORMAT;

  uint8_t seen[1 + 7 * 1024 + 1];
  memset(seen, 0, nmat);
  int32_t missing = 0;
  for (uint32_t i = 0; i < nmat; i++) {
    const uint8_t *d = blob + o_desc + 32ull * i;
    uint32_t kind = rd32(d), layer = rd32(d + 4), rows = rd32(d + 8), cols = rd32(d + 12);
    uint32_t sec = rd32(d + 16);
    uint64_t off = rd64(d + 24);
    if (kind >= K_KINDS) return FPI8_REF_INVALID_FORMAT;
    uint32_t er, ek;
    mat_dims(c, kind, &er, &ek);
    if (rows != er || cols != ek) return FPI8_REF_INVALID_FORMAT;
    uint32_t slot;
    if (kind == K_EMBED || kind == K_CLS) {
      if (layer != 0) return FPI8_REF_INVALID_FORMAT;
      slot = kind == K_EMBED ? 0 : 1 + 7 * c->layers;
    } else {
      if (layer >= c->layers) return FPI8_REF_INVALID_FORMAT;
      slot = 1 + 7 * layer + (kind - 1);
    }
    if (seen[slot]) return FPI8_REF_INVALID_FORMAT;
    seen[slot] = 1;
    if (sec == 0 || sec >= nsec || (off & 7)) return FPI8_REF_INVALID_FORMAT;
    uint64_t so = rd64(blob + SECTION_TABLE + 16ull * sec);
    uint64_t sl = rd64(blob + SECTION_TABLE + 16ull * sec + 8);
    if (so & 7) return FPI8_REF_INVALID_FORMAT;
    uint64_t need = a8((uint64_t)rows * cols) + 4ull * rows;
    /* "Core errors", MissingWeights: a section absent from the artifact or
     * shorter than the matrix it holds. */
    if (!in_range(so, sl, len) || !in_range(off, need, sl)) { missing = 1; continue; }
    if (mats) {
      mat_t *t = &mats[slot];
      t->w = blob + so + off;
      t->s_bytes = blob + so + off + a8((uint64_t)rows * cols);
      t->s = (const uint32_t *)t->s_bytes;
      t->rows = rows;
      t->cols = cols;
    }
  }
  if (missing) return FPI8_REF_MISSING_WEIGHTS;
  return 0;
}

int32_t fpi8_ref_blob_check(const uint8_t *blob, uint64_t len, uint32_t cfg_out[7]) {
  model_t m;
  int32_t e = parse(blob, len, &m, NULL);
  if (e == 0 && cfg_out) {
    for (int i = 0; i < 7; i++) cfg_out[i] = rd32(blob + 8 + 4 * i);
  }
  return e;
}

/* ---------------------------------------------------------------------- */
/* The forward pass of one position ("The forward pass, in order").        */

typedef struct {
  uint8_t *st;
  fpi8_ref_layout L;
  int64_t *x, *w1, *w2, *w3, *gate, *up, *logits, *scores;
  int32_t *keys, *values;
  uint32_t *ids, *out;
  int64_t *tmp; /* key or value rows on their way to the cache (not state) */
} run_t;

/* Index of a cache word: [layer][kv head][position][element]. */
static uint64_t cache_index(const cfg_t *c, uint32_t cachepos, uint32_t l, uint32_t kvh,
                            uint32_t pos, uint32_t i) {
  return (((uint64_t)l * c->kv_heads + kvh) * cachepos + pos) * c->head + i;
}

static int fits32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }

static int32_t fail(run_t *r, uint32_t phase, uint32_t layer) {
  wr32(r->st + H_PHASE, phase);
  wr32(r->st + H_LAYER, layer);
  wr32(r->st + H_ERROR, FPI8_REF_ARITHMETIC);
  return FPI8_REF_ARITHMETIC;
}

/* Phases 6 and 7, rows [row, row + n) of a key or value matrix: each row
 * goes straight into the cache after the 32-bit fit check ("The attention
 * cache"; the planner's charge is per row stored).  Returns 0 at the first
 * row that does not fit (the rows before it are stored). */
static int store_rows(const cfg_t *c, const mat_t *M, const int64_t *in, int64_t *tmp,
                      uint32_t row, uint32_t n, int32_t *cache, uint32_t cachepos, uint32_t l,
                      uint32_t pos) {
  fpi8_ref_rows(M->w + (uint64_t)row * M->cols, M->s + row, n, M->cols, in, 1, tmp);
  for (uint32_t k = 0; k < n; k++) {
    const uint32_t r = row + k;
    if (!fits32(tmp[k])) return 0;
    cache[cache_index(c, cachepos, l, r / c->head, pos, r % c->head)] = (int32_t)tmp[k];
  }
  return 1;
}

/* Runs the phase the state's cursor names ("The forward pass, in order"),
 * from wherever inside it the cursor stands, for at most *budget units of
 * work ("The resumable state": a row of a matrix, a position or an output
 * element of an attention stage, a vocabulary entry of a sampling pass, or
 * one whole vector operation), which it takes off *budget.  Every phase
 * reads only the state's buffers and writes its results back into them.
 * When the budget ends inside the phase the cursor records where (row,
 * attention stage and index, sampling pass, and the running maximum, sum,
 * choice and remainder) and *done stays 0.  Otherwise *done is set and the
 * cursor names the next phase; *ended is set when that ends the position:
 * the cursor then stands at the next position's embedding (phase 3), or at
 * phase 20 when the run is complete.  Returns 0, or the error that froze
 * the run. */
static int32_t run_phase(const model_t *m, const mat_t *mats, run_t *r, uint64_t *budget,
                         int *done, int *ended) {
  const cfg_t *c = &m->c;
  uint8_t *st = r->st;
  const uint32_t p = rd32(st + H_PHASE), l = rd32(st + H_LAYER);
  const uint32_t t = rd32(st + H_POSITION);
  const uint32_t n_ids = rd32(st + H_NIDS), cachepos = rd32(st + H_CACHEPOS);
  const uint32_t half = c->head / 2;
  const uint32_t group = c->heads / c->kv_heads;
  const mat_t *Lm = &mats[1 + 7 * l];
  uint32_t np = p + 1, nl = l;
  *done = 0;
  *ended = 0;
  if (*budget == 0) return 0;
  /* the matrix of a row phase, its input and its output */
  const mat_t *M = NULL;
  const int64_t *in = r->w1;
  int64_t *out = NULL;
  switch (p) {
    case 5: M = &Lm[K_Q - 1]; out = r->w2; break;
    case 6: M = &Lm[K_K - 1]; break;
    case 7: M = &Lm[K_V - 1]; break;
    case 10: M = &Lm[K_O - 1]; in = r->w3; out = r->w1; break;
    case 12: M = &Lm[K_GATE - 1]; out = r->gate; break;
    case 13: M = &Lm[K_UP - 1]; out = r->up; break;
    case 15: M = &Lm[K_DOWN - 1]; in = r->gate; out = r->w1; break;
    case 18: M = &mats[1 + 7 * c->layers]; out = r->logits; break;
    default: break;
  }
  if (M) {
    /* Phases 5, 6, 7 (query, key, value), 10 (attention output matrix), 12
     * and 13 (gate, up), 15 (down), 18 (classifier): rows from the cursor's
     * row on, as many as the budget allows. */
    const uint32_t row = rd32(st + H_ROW);
    const uint64_t left = M->rows - row;
    const uint32_t n = (uint32_t)(left < *budget ? left : *budget);
    if (out) {
      fpi8_ref_rows(M->w + (uint64_t)row * M->cols, M->s + row, n, M->cols, in, 1, out + row);
    } else if (!store_rows(c, M, in, r->tmp, row, n, p == 6 ? r->keys : r->values, cachepos, l, t)) {
      return fail(r, p, l);
    }
    *budget -= n;
    if (row + n < M->rows) {
      wr32(st + H_ROW, row + n);
      return 0;
    }
    wr32(st + H_ROW, 0);
  } else if (p == 9) {
    /* Attention, head by head (the cursor's row is the head), stage by
     * stage, outputs into w3; head h reads key and value head
     * h / (heads / kv_heads). */
    uint32_t h = rd32(st + H_ROW);
    attn_cursor ac = {rd32(st + H_STAGE), rd32(st + H_INDEX), (int64_t)rd64(st + H_MAXSCORE),
                      rd64(st + H_SUM)};
    /* When the budget covers every remaining head whole, the heads may run
     * on several threads: each head's scores, exponentials, probabilities
     * and outputs are its own (the shared scores buffer is only scratch
     * between them), so every word is still computed whole, in the same
     * order.  Heads other than the last use a scratch buffer of their own;
     * the last one leaves its probabilities, largest score and sum in the
     * state, as the head-by-head walk does. */
    const uint64_t per_head = 3ull * (t + 1) + c->head;
    if (g_threads > 1 && ac.stage == 0 && ac.index == 0 && h + 1 < c->heads &&
        *budget >= (uint64_t)(c->heads - h) * per_head) {
      int64_t *scratch = (int64_t *)malloc(sizeof(int64_t) * (uint64_t)(t + 1) * (uint64_t)g_threads);
      if (scratch) {
        int64_t last_max = 0;
        uint64_t last_sum = 0;
        const uint32_t h0 = h;
#pragma omp parallel for schedule(dynamic, 1) num_threads(g_threads)
        for (uint32_t hh = h0; hh < c->heads; hh++) {
#ifdef _OPENMP
          const int tid = omp_get_thread_num();
#else
          const int tid = 0;
#endif
          const uint32_t kh = hh / group;
          int64_t *sc = hh + 1 == c->heads ? r->scores : scratch + (uint64_t)tid * (t + 1);
          attn_cursor hc = {0, 0, 0, 0};
          while (!attention_unit(&r->w2[hh * c->head], &r->keys[cache_index(c, cachepos, l, kh, 0, 0)],
                                 &r->values[cache_index(c, cachepos, l, kh, 0, 0)], t + 1, c->head,
                                 c->head, m->inv, m->exp_tab, sc, &r->w3[hh * c->head], &hc)) {
          }
          if (hh + 1 == c->heads) {
            last_max = hc.max;
            last_sum = hc.sum;
          }
        }
        free(scratch);
        *budget -= (uint64_t)(c->heads - h) * per_head;
        h = c->heads;
        ac.stage = 0;
        ac.index = 0;
        ac.max = last_max;
        ac.sum = last_sum;
      }
    }
    while (h < c->heads && *budget > 0) {
      const uint32_t kh = h / group;
      const int32_t *K = &r->keys[cache_index(c, cachepos, l, kh, 0, 0)];
      const int32_t *V = &r->values[cache_index(c, cachepos, l, kh, 0, 0)];
      const int last = attention_unit(&r->w2[h * c->head], K, V, t + 1, c->head, c->head, m->inv,
                                      m->exp_tab, r->scores, &r->w3[h * c->head], &ac);
      (*budget)--;
      if (last) {
        h++;
        ac.stage = 0;
        ac.index = 0;
      }
    }
    wr64(st + H_MAXSCORE, (uint64_t)ac.max);
    wr64(st + H_SUM, ac.sum);
    wr32(st + H_STAGE, ac.stage);
    wr32(st + H_INDEX, ac.index);
    if (h < c->heads) {
      wr32(st + H_ROW, h);
      return 0;
    }
    wr32(st + H_ROW, 0);
  } else if (p == 19) {
    /* Sampling, entry by entry; the token is appended, then phase 20
     * (token 1 or 2, or max tokens reached) or the next position. */
    sample_cursor sc = {rd32(st + H_PASS), rd32(st + H_ROW), rd32(st + H_CHOSEN),
                        (int64_t)rd64(st + H_MAXSCORE), rd64(st + H_SUM), rd64(st + H_REMAINDER)};
    uint64_t gen = rd64(st + H_GENERATOR);
    int chosen = 0;
    while (!chosen && *budget > 0) {
      chosen = sample_unit(r->logits, c->vocab, rd32(st + H_TEMP), m->exp_tab, &gen, &sc);
      (*budget)--;
    }
    wr64(st + H_GENERATOR, gen);
    wr32(st + H_CHOSEN, sc.chosen);
    wr64(st + H_MAXSCORE, (uint64_t)sc.max);
    wr64(st + H_SUM, sc.sum);
    wr64(st + H_REMAINDER, sc.rem);
    if (!chosen) {
      wr32(st + H_PASS, sc.pass);
      wr32(st + H_ROW, sc.row);
      return 0;
    }
    wr32(st + H_PASS, 0);
    wr32(st + H_ROW, 0);
    const uint32_t next = sc.chosen;
    uint32_t g = rd32(st + H_GENERATED);
    r->out[g] = next;
    g++;
    wr32(st + H_GENERATED, g);
    const int complete = next == 1 || next == 2 || g == rd32(st + H_MAX);
    wr32(st + H_TOKEN, next);
    wr32(st + H_POSITION, t + 1);
    np = complete ? 20 : 3;
    nl = 0;
    *ended = 1;
  } else {
    /* the phases that are one whole vector operation */
    (*budget)--;
    switch (p) {
      case 3: {
        /* Embedding, ((byte - 128) * scale) >> 8 with the token row's scale. */
        const uint32_t tok = rd32(st + H_TOKEN);
        const mat_t *E = &mats[0];
        const uint8_t *row = E->w + (uint64_t)tok * c->dim;
        uint32_t sc = rd32(E->s_bytes + 4ull * tok);
        for (uint32_t i = 0; i < c->dim; i++)
          r->x[i] = asr(wmul((int64_t)row[i] - 128, (int64_t)(uint64_t)sc), 8);
        nl = 0;
        break;
      }
      case 4: /* attention normalization into w1 */
        fpi8_ref_rmsnorm(r->x, m->norm + (uint64_t)(2 * l) * c->dim, c->dim, r->w1);
        break;
      case 8: {
        /* Rotary.  Reading: pairs are adjacent elements (2j, 2j+1) of each
         * head, turned by the position's entry j of the tables; the query
         * first, then this position's keys, each stored key checked. */
        const int32_t *cs = m->cos_tab + (uint64_t)t * half;
        const int32_t *sn = m->sin_tab + (uint64_t)t * half;
        for (uint32_t h = 0; h < c->heads; h++)
          for (uint32_t j = 0; j < half; j++)
            fpi8_ref_rotate(&r->w2[h * c->head + 2 * j], &r->w2[h * c->head + 2 * j + 1], cs[j], sn[j]);
        for (uint32_t kh = 0; kh < c->kv_heads; kh++)
          for (uint32_t j = 0; j < half; j++) {
            int32_t *k0 = &r->keys[cache_index(c, cachepos, l, kh, t, 2 * j)];
            int64_t a = k0[0], b = k0[1];
            fpi8_ref_rotate(&a, &b, cs[j], sn[j]);
            if (!fits32(a) || !fits32(b)) return fail(r, 8, l);
            k0[0] = (int32_t)a;
            k0[1] = (int32_t)b;
          }
        break;
      }
      case 11: /* residual, then the feed-forward normalization into w1 */
        for (uint32_t i = 0; i < c->dim; i++) r->x[i] = wadd(r->x[i], r->w1[i]);
        fpi8_ref_rmsnorm(r->x, m->norm + (uint64_t)(2 * l + 1) * c->dim, c->dim, r->w1);
        break;
      case 14: /* gate element through SiLU times the up element, >> 16, kept in gate */
        for (uint32_t i = 0; i < c->hidden; i++)
          r->gate[i] = asr(wmul(fpi8_ref_silu(r->gate[i], m->silu_tab), r->up[i]), 16);
        break;
      case 16: /* residual; then the next layer, the final phases, or the next
                * prompt position (phases 17-19 run only where a token is
                * generated: the last prompt position and every later one) */
        for (uint32_t i = 0; i < c->dim; i++) r->x[i] = wadd(r->x[i], r->w1[i]);
        if (l + 1 < c->layers) {
          np = 4;
          nl = l + 1;
        } else if (t + 1 >= n_ids) {
          np = 17;
          nl = 0;
        } else {
          wr32(st + H_TOKEN, r->ids[t + 1]);
          wr32(st + H_POSITION, t + 1);
          np = 3;
          nl = 0;
          *ended = 1;
        }
        break;
      case 17: /* final normalization into w1 */
        fpi8_ref_rmsnorm(r->x, m->norm + (uint64_t)(2 * c->layers) * c->dim, c->dim, r->w1);
        break;
      default:
        return FPI8_REF_INVALID_STATE;
    }
  }
  wr32(st + H_PHASE, np);
  wr32(st + H_LAYER, nl);
  *done = 1;
  return 0;
}

/* Rows of the matrix phase p works through, 0 for the other phases. */
static uint32_t phase_rows(const cfg_t *c, uint32_t p) {
  switch (p) {
    case 5: case 10: case 15: return c->dim;
    case 6: case 7: return c->kvd;
    case 12: case 13: return c->hidden;
    case 18: return c->vocab;
    default: return 0;
  }
}

/* State checks shared by turn: tag, alignment, size for the configuration,
 * and a cursor the pass can stand at ("Core errors", InvalidState): phase 3
 * (a position's start), 4 to 16 with a layer, or 17 to 19 at a position
 * that generates; inside a matrix phase a row below its rows, inside
 * attention a head, a stage 0 to 3 and an index below the stage's units
 * (with a sum of exponentials once stage 1 has ended), inside sampling a
 * pass 0 to 2 (1 and 2 above temperature zero) and an entry below the
 * vocabulary (in the draw pass a remainder below the sum).  Every other
 * sub-phase field is zero. */
static int32_t check_state(const cfg_t *c, uint8_t *st, uint64_t len, fpi8_ref_layout *L) {
  if (((uintptr_t)st) & 7 || len < HEADER || memcmp(st, STATE_TAG, 8))
    return FPI8_REF_INVALID_STATE;
  uint32_t n_ids = rd32(st + H_NIDS), mx = rd32(st + H_MAX);
  if (!layout_ids(c, n_ids, mx, L) || L->total != len) return FPI8_REF_INVALID_STATE;
  if (rd32(st + H_CACHEPOS) != L->cache_positions) return FPI8_REF_INVALID_STATE;
  const uint32_t phase = rd32(st + H_PHASE), layer = rd32(st + H_LAYER);
  if (rd32(st + H_ERROR) != 0 || phase < 3 || phase > 19) return FPI8_REF_INVALID_STATE;
  if ((phase >= 4 && phase <= 16) ? layer >= c->layers : layer != 0) return FPI8_REF_INVALID_STATE;
  uint32_t pos = rd32(st + H_POSITION), gen = rd32(st + H_GENERATED);
  if (phase >= 17 && pos + 1 < n_ids) return FPI8_REF_INVALID_STATE;
  if (pos >= L->cache_positions) return FPI8_REF_INVALID_STATE;
  if (gen != (pos + 1 > n_ids ? pos + 1 - n_ids : 0)) return FPI8_REF_INVALID_STATE;
  if (rd32(st + H_TOKEN) >= c->vocab || rd32(st + H_TEMP) > (16u << 16))
    return FPI8_REF_INVALID_STATE;
  const uint32_t row = rd32(st + H_ROW), stage = rd32(st + H_STAGE), index = rd32(st + H_INDEX);
  const uint32_t pass = rd32(st + H_PASS);
  if (phase == 9) {
    if (row >= c->heads || stage > 3 || index >= (stage < 3 ? pos + 1 : c->head) || pass != 0)
      return FPI8_REF_INVALID_STATE;
    if (stage >= 2 && rd64(st + H_SUM) == 0) return FPI8_REF_INVALID_STATE;
  } else if (phase == 19) {
    if (pass > 2 || (pass > 0 && rd32(st + H_TEMP) == 0) || row >= c->vocab || stage != 0 ||
        index != 0)
      return FPI8_REF_INVALID_STATE;
    if (pass == 2 && rd64(st + H_REMAINDER) >= rd64(st + H_SUM)) return FPI8_REF_INVALID_STATE;
  } else {
    if (row >= (phase_rows(c, phase) ? phase_rows(c, phase) : 1) || stage != 0 || index != 0 ||
        pass != 0)
      return FPI8_REF_INVALID_STATE;
  }
  return 0;
}

/* A turn from the cursor (mode 0: up to count positions, the first one
 * finished from wherever the cursor stands; 1: up to count phases, the
 * first one likewise; 2: up to count units of work). */
static int32_t turn(const uint8_t *blob, uint64_t blob_len, uint8_t *state, uint64_t state_len,
                    uint64_t count, int mode) {
  model_t m;
  mat_t *mats;
  uint32_t nm;
  {
    model_t probe;
    int32_t e = parse(blob, blob_len, &probe, NULL);
    if (e) return e;
    nm = 2 + 7 * probe.c.layers;
  }
  mats = (mat_t *)calloc(nm, sizeof(mat_t));
  if (!mats) return FPI8_REF_BUFFER_TOO_SMALL;
  parse(blob, blob_len, &m, mats);
  run_t r;
  int32_t e = check_state(&m.c, state, state_len, &r.L);
  if (e) { free(mats); return e; }
  r.tmp = (int64_t *)malloc(8ull * m.c.kvd);
  if (!r.tmp) { free(mats); return FPI8_REF_BUFFER_TOO_SMALL; }
  r.st = state;
  r.x = (int64_t *)(state + r.L.x);
  r.w1 = (int64_t *)(state + r.L.w1);
  r.w2 = (int64_t *)(state + r.L.w2);
  r.w3 = (int64_t *)(state + r.L.w3);
  r.gate = (int64_t *)(state + r.L.gate);
  r.up = (int64_t *)(state + r.L.up);
  r.logits = (int64_t *)(state + r.L.logits);
  r.scores = (int64_t *)(state + r.L.scores);
  r.keys = (int32_t *)(state + r.L.keys);
  r.values = (int32_t *)(state + r.L.values);
  r.ids = (uint32_t *)(state + r.L.ids);
  r.out = (uint32_t *)(state + r.L.out);
  wr64(state + H_TURNS, rd64(state + H_TURNS) + 1);
  uint64_t units = mode == 2 ? count : UINT64_MAX;
  uint64_t n = 0;
  while (mode == 2 ? units > 0 : n < count) {
    int done, ended;
    e = run_phase(&m, mats, &r, &units, &done, &ended);
    if (e || !done) break;
    if ((mode == 0 && ended) || mode == 1) n++;
    if (rd32(state + H_PHASE) == 20) break;
  }
  free(r.tmp);
  free(mats);
  return e;
}

int32_t fpi8_ref_turn(const uint8_t *blob, uint64_t blob_len, uint8_t *state,
                      uint64_t state_len, uint32_t max_positions) {
  return turn(blob, blob_len, state, state_len, max_positions, 0);
}

int32_t fpi8_ref_turn_phases(const uint8_t *blob, uint64_t blob_len, uint8_t *state,
                             uint64_t state_len, uint32_t max_phases) {
  return turn(blob, blob_len, state, state_len, max_phases, 1);
}

int32_t fpi8_ref_turn_units(const uint8_t *blob, uint64_t blob_len, uint8_t *state,
                            uint64_t state_len, uint64_t max_units) {
  return turn(blob, blob_len, state, state_len, max_units, 2);
}
