/*
 * fpi8_ref.h - the oracle of the fixed-point forward pass (plain C, CPU).
 *
 * TEST INFRASTRUCTURE.  This library is the slow, literal CPU reading of
 * the curta-core inference core ("The inference core" page) against which
 * the GPU library is checked bit for bit.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load or call it; the
 * GPU library shares no code, header, table or helper with it.
 *
 * Citations name the page's sections: "Fixed-point arithmetic", "A matrix
 * row", "RMS normalization", "The attention cache", "Lookup tables", "The
 * forward pass, in order", "Attention, stage by stage", "The resumable
 * state", "Sampling", "The Rust API", "WebAssembly exports", "Core errors".
 *
 * All 64-bit arithmetic wraps modulo 2^64; ">>" on signed values is an
 * arithmetic (flooring) shift; "/" on signed values truncates toward zero.
 */
#ifndef FPI8_REF_H
#define FPI8_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Core error numbers ("Core errors"). */
enum {
  FPI8_REF_OK = 0,
  FPI8_REF_INVALID_CONFIG = 1,
  FPI8_REF_INVALID_FORMAT = 2,
  FPI8_REF_INVALID_STATE = 3,
  FPI8_REF_BUFFER_TOO_SMALL = 4,
  FPI8_REF_MISSING_WEIGHTS = 5,
  FPI8_REF_INVALID_PROMPT = 6,
  FPI8_REF_CONTEXT_EXCEEDED = 7,
  FPI8_REF_ARITHMETIC = 8
};

typedef struct {
  uint32_t phase, layer, position, token;
  uint32_t n_ids, max_tokens, temperature_q16, generated;
  uint32_t cache_positions, error, complete, reserved;
  uint64_t generator, turns;
} fpi8_ref_info;

/* ---- primitives ------------------------------------------------------- */

/* Largest r with r*r <= n ("RMS normalization": integer square root). */
uint64_t fpi8_ref_isqrt(uint64_t n);

/* One matrix row ("A matrix row"): bytes are weight+128. */
int64_t fpi8_ref_row(const uint8_t *w, uint32_t scale, const int64_t *x, uint32_t n);

/* y[b*rows + r] = row r of W (row-major, rows x cols) times x[b*cols ...]. */
void fpi8_ref_rows(const uint8_t *W, const uint32_t *scales, uint32_t rows,
                   uint32_t cols, const int64_t *x, uint32_t batch, int64_t *y);

/* RMS normalization ("RMS normalization"), y may not alias x. */
void fpi8_ref_rmsnorm(const int64_t *x, const int32_t *w, uint32_t d, int64_t *y);

/* One rotary pair rotated by a cosine and sine at Q24 ("Phase 8"). */
void fpi8_ref_rotate(int64_t *a, int64_t *b, int32_t c, int32_t s);

/* Exponential-table index of a score difference ("Lookup tables"). */
uint32_t fpi8_ref_exp_index(uint64_t d);

/* SiLU through the table ("Lookup tables"). */
int64_t fpi8_ref_silu(int64_t x, const int32_t *tab);

/* Phase 9 for one head ("Attention, stage by stage").  K and V point at the
 * head's first cached position; consecutive positions are `stride` words
 * apart.  scores has npos entries and ends holding the probabilities. */
void fpi8_ref_attention_head(const int64_t *q, const int32_t *K, const int32_t *V,
                             uint32_t npos, uint32_t head, uint64_t stride,
                             uint32_t inv_sqrt_head, const uint32_t *exp_tab,
                             int64_t *scores, int64_t *out,
                             int64_t *max_out, uint64_t *sum_out);

/* xorshift64* ("Sampling"): advances *state, returns state * multiplier. */
uint64_t fpi8_ref_xorshift64s(uint64_t *state);

/* Phase 19 over a logit vector ("Sampling"); advances *generator at T > 0. */
uint32_t fpi8_ref_sample(const int64_t *logits, uint32_t vocab, uint32_t temperature_q16,
                         const uint32_t *exp_tab, uint64_t *generator);

/* ---- artifact, state and turn ---------------------------------------- */

/* Validates an artifact; 0, 1, 2 or 5.  cfg_out may be NULL. */
int32_t fpi8_ref_blob_check(const uint8_t *blob, uint64_t len, uint32_t cfg_out[7]);

/* Size of the ids-in state; UINT64_MAX for parameters out of range. */
uint64_t fpi8_ref_state_size(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens);

/* Size of the pages' own run account (prompt bytes in, 256-byte account
 * header included); UINT64_MAX out of range.  Used to pin the buffer table
 * against the four sizes the page prints. */
uint64_t fpi8_ref_pages_state_size(const uint32_t cfg[7], uint32_t prompt_bytes,
                                   uint32_t max_tokens);

int32_t fpi8_ref_init_state(const uint32_t cfg[7], uint8_t *state, uint64_t state_len,
                            const uint32_t *ids, uint32_t n_ids, uint32_t max_tokens,
                            uint32_t temperature_q16, uint64_t seed);

int32_t fpi8_ref_state_info(const uint8_t *state, uint64_t len, fpi8_ref_info *out);

/* Runs up to max_positions positions of one run; the first one is
 * finished from wherever the state's cursor stands. */
int32_t fpi8_ref_turn(const uint8_t *blob, uint64_t blob_len, uint8_t *state,
                      uint64_t state_len, uint32_t max_positions);

/* Runs up to max_phases phases of one run from the state's cursor (the
 * first one finished from wherever inside it the cursor stands), stopping
 * early at phase 20 or an error. */
int32_t fpi8_ref_turn_phases(const uint8_t *blob, uint64_t blob_len, uint8_t *state,
                             uint64_t state_len, uint32_t max_phases);

/* Runs up to max_units units of work of one run from the state's cursor: a
 * row of a matrix, a position or output element of an attention stage, a
 * vocabulary entry of a sampling pass, or a phase that is one whole vector
 * operation.  It may stop inside a phase; the cursor then records where. */
int32_t fpi8_ref_turn_units(const uint8_t *blob, uint64_t blob_len, uint8_t *state,
                            uint64_t state_len, uint64_t max_units);

/* Byte offsets of the state's buffers (for tests that read them). */
typedef struct {
  uint64_t ids, out, x, w1, w2, w3, gate, up, logits, scores, keys, values, total;
  uint32_t cache_positions;
} fpi8_ref_layout;
int32_t fpi8_ref_state_layout(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens,
                              fpi8_ref_layout *out);

/* Threads for the loops over matrix rows (OpenMP); returns the count used. */
int32_t fpi8_ref_set_threads(int32_t n);

#ifdef __cplusplus
}
#endif
#endif
