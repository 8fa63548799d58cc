// fpi8_charges.cpp - the compute units the turn planner of "The inference
// core" page charges for one position, on the host.
//
// "The turn planner": each chunk of work adds 160 units (reading the
// cursor, dispatching, writing it back).  "Compute costs": a matrix chunk
// costs 6n + 350 for summing its input and 37 floor(n/8) + 8 (n mod 8) + 34
// per row (42 for a key or value row stored in the cache); the vector
// operations cost 16d + 512 (embedding), 48d + 1,500 (the normalizations
// before attention and at the end), 48d + 512 (rotary), 56d + 1,500 (the
// residual with the feed-forward normalization), 24h + 512 (SiLU) and
// 8d + 128 (the residual); an attention stage costs its setup (100, 80, 60,
// 60) and per unit 53 floor(q/8) + 11 (q mod 8) + 25, 23 and 8 per position
// so far and 11 p + 32 per output element; a sampling pass costs 350, 11,
// 36 or 42 per vocabulary entry and 4,000 to finish.
//
// Readings: every chunk is whole (one per matrix of a layer, per stage of a
// head, per sampling pass, per vector operation); where a turn boundary
// splits a chunk the planner charges its setup and 160 again, and each turn
// adds 18,000, neither of which is counted here.  Above temperature zero
// there are three passes, each with its setup and finishing charge.
#include <stdint.h>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

using namespace fpi8;

namespace {

constexpr uint64_t kChunk = 160;

uint64_t matrix(uint64_t rows, uint64_t n, bool cache) {
  const uint64_t row = 37 * (n / 8) + 8 * (n % 8) + (cache ? 42 : 34);
  return 6 * n + 350 + rows * row + kChunk;
}

uint64_t attention_head(uint64_t q, uint64_t p) {
  const uint64_t scores = 100 + p * (53 * (q / 8) + 11 * (q % 8) + 25);
  const uint64_t exps = 80 + p * 23;
  const uint64_t norm = 60 + p * 8;
  const uint64_t values = 60 + q * (11 * p + 32);
  return scores + exps + norm + values + 4 * kChunk;
}

}  // namespace

extern "C" {

int32_t fpi8_position_charges(const uint32_t cfg[7], uint32_t position, int32_t generating,
                              uint32_t temperature_q16, uint64_t out[17]) {
  Cfg c;
  if (!cfg || !cfg_from_words(cfg, &c)) return FPI8_INVALID_CONFIG;
  if (position >= c.context || temperature_q16 > (16u << 16)) return FPI8_INVALID_PROMPT;
  if (!out) return FPI8_BUFFER_TOO_SMALL;
  const uint64_t d = c.dim, h = c.hidden, q = c.head, p = (uint64_t)position + 1;
  for (int i = 0; i < 17; i++) out[i] = 0;
  // out[phase - 3], phases 3 to 19
  out[0] = 16 * d + 512 + kChunk;
  for (uint32_t l = 0; l < c.layers; l++) {
    out[1] += 48 * d + 1500 + kChunk;                 // 4 attention normalization
    out[2] += matrix(d, d, false);                    // 5 query
    out[3] += matrix(c.kvd, d, true);                 // 6 key, into the cache
    out[4] += matrix(c.kvd, d, true);                 // 7 value, into the cache
    out[5] += 48 * d + 512 + kChunk;                  // 8 rotary
    out[6] += (uint64_t)c.heads * attention_head(q, p);  // 9 attention
    out[7] += matrix(d, d, false);                    // 10 attention output
    out[8] += 56 * d + 1500 + kChunk;                 // 11 residual, feed-forward normalization
    out[9] += matrix(h, d, false);                    // 12 gate
    out[10] += matrix(h, d, false);                   // 13 up
    out[11] += 24 * h + 512 + kChunk;                 // 14 SiLU
    out[12] += matrix(d, h, false);                   // 15 down
    out[13] += 8 * d + 128 + kChunk;                  // 16 residual
  }
  if (generating) {
    out[14] = 48 * d + 1500 + kChunk;                 // 17 final normalization
    out[15] = matrix(c.vocab, d, false);              // 18 classifier
    const uint64_t per[3] = {11, 36, 42};             // 19 sampling: max, sum, draw
    const int passes = temperature_q16 == 0 ? 1 : 3;
    for (int k = 0; k < passes; k++) out[16] += 350 + (uint64_t)c.vocab * per[k] + 4000 + kChunk;
  }
  return 0;
}

}  // extern "C"
