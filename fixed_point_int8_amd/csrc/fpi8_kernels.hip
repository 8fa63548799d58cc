// fpi8_kernels.hip - HIP kernels (gfx950) of the fixed-point forward pass of
// the curta-core inference core ("The inference core" page).
//
// Every value is an integer with a fixed count of fractional bits ("Fixed-
// point arithmetic"); 64-bit products and sums wrap, ">>" on signed values
// floors, "/" truncates.  The kernels advance a batch of independent runs by
// one position per launch sequence:
//
//   begin -> embedding -> per layer [norm -> Q/K/V rows (+ rotary, cache
//   store, fit checks) -> attention -> output rows (+ residual) -> norm ->
//   gate/up rows (+ SiLU) -> down rows (+ residual)] -> final norm ->
//   classifier rows -> sampling
//
// The matrix row ("A matrix row") runs on the int8 matrix cores.  Each i64
// input x is split into three signed base-256 digits, x = d0 + 256 d1 +
// 65536 d2 with every d in [-128, 127], which covers |x| up to about 2^23
// (128.0 at Q16).  The weight byte b becomes the signed weight b - 128 by
// flipping its top bit, and one 16x16x64 int8 MFMA per digit gives exact
// i32 partial sums (|sum| <= 2^14 * cols < 2^31).  Recombined they are the
// signed dot sum_c (b_c - 128) x_c exactly, which equals the page's
// acc - 128 * sum modulo 2^64.  A launch whose inputs hold any value outside
// the three-digit range takes an exact 64-bit path instead (a standalone call
// of one or two inputs decides wave by wave), so the result is the page's
// for every input.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"
#include "fpi8_device.h"

namespace fpi8 {





__device__ __forceinline__ void put_digits(int8_t *planes, uint32_t bp, uint32_t kp, uint32_t b,
                                           uint32_t k, int64_t x, uint32_t *oflag) {
  int8_t d0, d1, d2;
  if (!digits3(x, d0, d1, d2)) atomicOr(oflag, 1u);
  const uint64_t limb = (uint64_t)bp * kp, at = digit_at(b, k, kp);
  planes[at] = d0;
  planes[limb + at] = d1;
  planes[2 * limb + at] = d2;
}

__device__ __forceinline__ uint64_t isqrt64(uint64_t n) {
  uint64_t r = (uint64_t)sqrt((double)n);
  if (r > 0xFFFFFFFFull) r = 0xFFFFFFFFull;
  while (r * r > n) --r;
  while (r < 0xFFFFFFFFull && (r + 1) * (r + 1) <= n) ++r;
  return r;
}

// floor(2^64 / r) for 2 <= r < 2^32, by long division in base 2^32 with
// 32-bit quotient digits: the high digit floor(2^32 / r) from a 32-bit
// division, the low digit floor(rem * 2^32 / r) from a correctly rounded
// double quotient (rem * 2^32 is exact in a double; the rounded quotient is
// at most one above the true floor), checked with one exact product.  Two
// 64-bit integer divisions cost about 1.4 us of a normalization's chain.
__device__ __forceinline__ uint64_t recip64_32(uint32_t r) {
  uint32_t q1 = 0xFFFFFFFFu / r;
  if (0xFFFFFFFFu - q1 * r == r - 1) q1++;           // floor(2^32 / r)
  const uint32_t rem = 0u - q1 * r;                   // 2^32 - q1 * r, in [0, r)
  const uint64_t n = (uint64_t)rem << 32;
  uint64_t q0 = (uint64_t)((double)n / (double)r);
  if (q0 * r > n) q0--;                               // floor(rem * 2^32 / r)
  return ((uint64_t)q1 << 32) | q0;
}

// floor(2^64 / d) for any d >= 2: recip64_32 below 2^32; from 2^32 on the
// quotient is below 2^32, so a correctly rounded double quotient is the
// floor or one above it, settled by the exact 128-bit product.
__device__ __forceinline__ uint64_t recip64(uint64_t d) {
  if (d < (1ull << 32)) return recip64_32((uint32_t)d);
  uint64_t q = (uint64_t)(18446744073709551616.0 / (double)d);
  const uint64_t hi = __umul64hi(q, d);
  if (hi > 1 || (hi == 1 && q * d != 0)) q--;  // q * d > 2^64
  return q;
}

__device__ __forceinline__ uint8_t *run_base(uint8_t *states, const RunDesc &rd) {
  return states + rd.base;
}

// Block-wide sums and maxima (256 threads).
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t *scratch) {
  for (int o = 32; o > 0; o >>= 1) v += (uint64_t)__shfl_xor((long long)v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  uint64_t s = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); i++) s += scratch[i];
  return s;
}

__device__ __forceinline__ int64_t block_max_i64(int64_t v, int64_t *scratch) {
  for (int o = 32; o > 0; o >>= 1) {
    int64_t u = (int64_t)__shfl_xor((long long)v, o, 64);
    v = u > v ? u : v;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  int64_t m = scratch[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); i++) m = scratch[i] > m ? scratch[i] : m;
  return m;
}

// ---------------------------------------------------------------------------
// Turn and position bookkeeping

__global__ void k_turn_start(uint8_t *states, RunDesc *runs, uint32_t n_runs) {
  const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= n_runs || !runs[b].valid) return;
  uint64_t *turns = reinterpret_cast<uint64_t *>(run_base(states, runs[b]) + ST_TURNS);
  *turns += 1;
}

// First kernel of a position: which runs compute it, which generate, and
// for a run whose state stands between two phases, the step it starts at
// and the phase its fused launch picks up at (run_flags).  A phase whose
// inputs are still in the state and whose outputs nothing has read yet is
// run again rather than picked up: the normalizations (5 after 4, 12 after
// 11, 18 after 17) and attention (10 after 9) give the same words again.
// A turn of units of work ("The resumable state": a row of a matrix, a
// position or output element of an attention stage, a vocabulary entry of a
// sampling pass, or a phase that is one vector operation).  Units of phase p
// in a position of npos positions; sampling counts its maximum and sum
// passes here (the draw pass ends where the draw falls).
__device__ __forceinline__ uint64_t phase_units(const BeginArgs &a, uint32_t p, uint32_t npos,
                                                uint32_t temp) {
  switch (p) {
    case 5: case 10: case 15: return a.dim;
    case 6: case 7: return a.kvd;
    case 9: return (uint64_t)a.heads * (3ull * npos + a.head);
    case 12: case 13: return a.hidden;
    case 18: return a.vocab;
    case 19: return (uint64_t)a.vocab * (temp ? 2u : 1u);
    default: return 1;
  }
}

// The step of the launch that holds phase p of layer l.
__device__ __forceinline__ uint32_t phase_step(const BeginArgs &a, uint32_t p, uint32_t l) {
  const uint32_t l7 = 7 * l, f7 = 7 * a.layers;
  switch (p) {
    case 3: return 0;
    case 4: return 1 + l7;
    case 5: case 6: case 7: case 8: return 2 + l7;
    case 9: return 3 + l7;
    case 10: case 11: return 4 + l7;
    case 12: case 13: case 14: return 6 + l7;
    case 15: case 16: return 7 + l7;
    case 17: return 1 + f7;
    case 18: return 2 + f7;
    default: return 3 + f7;
  }
}

// Where a turn of units stops a run inside the position its cursor (p, l,
// and d units of phase p done) stands in: walks the phases in order,
// taking each one's units off the budget, and records the cursor where
// the budget ends (rd.stop_*), or leaves rd.stop_ph 0 when the position's
// phases fit (rd.budget then holds what is left, for the draw pass or the
// next position).  Returns the step the run stops before, ~0 if none.
__device__ uint32_t units_stop(const BeginArgs &a, RunDesc &rd, uint32_t p, uint32_t l, uint64_t d,
                               uint32_t pos) {
  const uint32_t npos = pos + 1, temp = rd.temp;
  const bool gen = pos + 1 >= rd.n_ids;
  uint64_t B = rd.budget;
  rd.stop_ph = 0;
  bool stop = false;
  for (;;) {
    if (p == 19 && temp != 0 && d >= 2ull * a.vocab) break;  // inside the draw pass
    const uint64_t u = phase_units(a, p, npos, temp);
    if (B < u - d) {
      d += B;
      B = 0;
      stop = true;
      break;
    }
    B -= u - d;
    d = 0;
    if (p == 19) break;  // the maximum (and sum) pass done; the draw is the sampler's
    if (p == 16) {
      if (l + 1 < a.layers) { p = 4; l++; }
      else if (gen) { p = 17; l = 0; }
      else break;  // the position's phases fit
    } else {
      p++;
    }
  }
  rd.budget = B;
  rd.stop_in = 0xFFFFFFFFu;
  if (!stop) return 0xFFFFFFFFu;
  // The budget ends inside phase p after d of its units.
  rd.stop_ph = p;
  rd.stop_layer = l;
  rd.stop_row = 0; rd.stop_stage = 0; rd.stop_index = 0; rd.stop_pass = 0;
  if (p == 9) {
    const uint64_t per = 3ull * npos + a.head, r = d % per;
    rd.stop_row = (uint32_t)(d / per);
    rd.stop_stage = r < 3ull * npos ? (uint32_t)(r / npos) : 3u;
    rd.stop_index = (uint32_t)(rd.stop_stage < 3 ? r % npos : r - 3ull * npos);
  } else if (p == 19) {
    rd.stop_pass = (uint32_t)(d / a.vocab);
    rd.stop_row = (uint32_t)(d % a.vocab);
  } else {
    rd.stop_row = (uint32_t)d;
  }
  // At the start of a launch's first phase the run stops before that
  // launch; anywhere else the launch runs for it in part.
  const uint32_t L = phase_step(a, p, l);
  const bool first = p == 3 || p == 4 || p == 5 || p == 9 || p == 10 || p == 12 || p == 15 ||
                     p == 17 || p == 18 || p == 19;
  if (d == 0 && first) return L;
  rd.stop_in = L;
  return L + 1;
}

__global__ void k_begin(BeginArgs a) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < a.n_oflags) a.oflags[i] = 0;
  if (i >= a.n_runs) return;
  RunDesc &rd = a.runs[i];
  uint32_t flags = 0, end = 0xFFFFFFFFu;
  if (rd.valid && rd.units && rd.halted) {
    // stopped by the budget in an earlier position of this turn
  } else if (rd.valid) {
    const uint8_t *st = run_base(a.states, rd);
    const uint32_t phase = *reinterpret_cast<const uint32_t *>(st + ST_PHASE);
    const uint32_t layer = *reinterpret_cast<const uint32_t *>(st + ST_LAYER);
    const uint32_t err = *reinterpret_cast<const uint32_t *>(st + ST_ERROR);
    const uint32_t pos = *reinterpret_cast<const uint32_t *>(st + ST_POSITION);
    if (pos == rd.stop_pos) end = rd.stop_step;
    if (phase >= 3 && phase <= 19 && err == 0 && end != 0) {
      rd.pos = pos;
      rd.token = *reinterpret_cast<const uint32_t *>(st + ST_TOKEN);
      const uint32_t l7 = 7 * layer, f7 = 7 * a.layers;
      uint32_t start = 0, pick = 0, after = 0;
      switch (phase) {
        case 4: case 5: start = 1 + l7; break;
        case 6: case 7: case 8: start = 1 + l7; pick = phase; after = 1; break;
        case 9: case 10: start = 3 + l7; break;
        case 11: start = 4 + l7; pick = 11; break;
        case 12: start = 5 + l7; break;
        case 13: case 14: case 15: start = 5 + l7; pick = phase; after = 1; break;
        case 16: start = 7 + l7; pick = 16; break;
        case 17: case 18: start = 1 + f7; break;
        case 19: start = 3 + f7; break;
        default: break;
      }
      flags = run_flags(RUN_ACTIVE | (pos + 1 >= rd.n_ids ? RUN_GEN : 0u), start, pick, after);
      if (rd.units) {
        if (rd.budget == 0) {
          flags = 0;  // nothing to do: the state stays as it is
          rd.halted = 1;
        } else {
          // units of the current phase already done, from the cursor
          const uint32_t row = *reinterpret_cast<const uint32_t *>(st + ST_ROW);
          const uint32_t npos = pos + 1;
          uint64_t d = row;
          if (phase == 9) {
            const uint32_t stage = *reinterpret_cast<const uint32_t *>(st + ST_STAGE);
            const uint32_t index = *reinterpret_cast<const uint32_t *>(st + ST_INDEX);
            d = (uint64_t)row * (3ull * npos + a.head) + (stage < 3 ? (uint64_t)stage * npos : 3ull * npos) + index;
          } else if (phase == 19) {
            d = (uint64_t)*reinterpret_cast<const uint32_t *>(st + ST_PASS) * a.vocab + row;
          }
          end = units_stop(a, rd, phase, layer, d, pos);
          if (rd.stop_ph != 0) rd.halted = 1;
        }
      }
    }
  }
  rd.flags = flags;
  rd.end = end;
  rd.errkey = 0xFFFFFFFFu;
}

// Whether a run takes part in the launch at `step` of its position: it is
// active, generates where `need` says so, does not start later and is not
// stopped before (flags is rd.flags, maybe read earlier).
__device__ __forceinline__ bool live_at(const RunDesc &rd, uint32_t flags, uint32_t need,
                                        uint32_t step, uint32_t partial) {
  return (flags & need) != 0 && (partial == 0 || ((flags >> 8) <= step && step < rd.end));
}

// The state's phase that the fused launch at `step` picks up at for this
// run, or 0 when it runs the launch's phases from the start.
__device__ __forceinline__ uint32_t pick_at(uint32_t flags, uint32_t step, uint32_t partial) {
  return partial != 0 && (flags >> 8) + ((flags >> 7) & 1u) == step ? (flags >> 2) & 31u : 0u;
}

// Phase 3: ((byte - 128) * scale) >> 8 with the token row's scale.
__global__ void k_embed(EmbedArgs a) {
  const uint32_t b = blockIdx.y;
  const RunDesc &rd = a.runs[b];
  if (!live_at(rd, rd.flags, RUN_ACTIVE, 0, a.partial)) return;
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.dim) return;
  const uint32_t tok = rd.token;
  if (tok >= a.vocab) return;  // an id the state should not hold; never read past the table
  const int64_t s = (int64_t)(uint64_t)a.S[tok];
  const int64_t w = (int64_t)a.E[(uint64_t)tok * a.dim + i] - 128;
  int64_t *x = reinterpret_cast<int64_t *>(run_base(a.states, rd) + rd.off_x);
  x[i] = wmul(w, s) >> 8;
}

// Phases 4, 11 (normalization part) and 17: RMS normalization of x into w1,
// rms = isqrt(sum(x*x) / dim + 42,950) at least 1, y = ((x * w) / rms) >> 8;
// also writes the digits of w1 for the next matrix.
__global__ __launch_bounds__(512) void k_norm(NormArgs a) {
  __shared__ uint64_t scratch[8];
  constexpr int U = 8;  // loads in flight per thread
  const uint32_t b = blockIdx.x, nt = blockDim.x;
  const bool whole = a.dim <= nt * U;
  // When every run keeps x at the same offset (a.x_first), the whole-vector
  // path reads x before the run's descriptor arrives, so the two round trips
  // overlap; a run that takes no part leaves after its sum.
  const int64_t *xu = whole && a.x_first ? reinterpret_cast<const int64_t *>(a.x_first + (uint64_t)b * a.x_stride)
                                         : nullptr;
  int64_t xv[U];
  int32_t wv[U];
  if (xu) {
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t i = threadIdx.x + u * nt;
      xv[u] = i < a.dim ? xu[i] : 0;
      wv[u] = i < a.dim ? a.w[i] : 0;
    }
  }
  // The descriptor fields this kernel reads, requested together.
  const RunDesc &rd = a.runs[b];
  const uint32_t flags = rd.flags, rend = rd.end, partial = a.partial, step = a.step;
  const uint64_t base = rd.base, off_x = rd.off_x, off_w1 = rd.off_w1;
  asm volatile("" ::"s"(flags), "s"(rend), "s"(partial), "s"(step), "s"(base), "s"(off_x), "s"(off_w1));
  const bool live = (flags & (a.final_norm ? RUN_GEN : RUN_ACTIVE)) != 0 &&
                    (partial == 0 || ((flags >> 8) <= step && step < rend));
  if (!xu && !live) return;
  uint8_t *st = a.states + base;
  const int64_t *x = reinterpret_cast<const int64_t *>(st + off_x);
  int64_t *y = reinterpret_cast<int64_t *>(st + off_w1);
  // y = ((x * w) / rms) >> 8 with a truncating division by rms, through
  // its 64-bit reciprocal m = floor(2^64 / rms): q = mulhi(|p|, m) is the
  // quotient or one less, and one remainder test fixes it (Granlund and
  // Montgomery, "Division by invariant integers using multiplication", 1994).
  auto finish = [&](uint32_t i, int64_t xi, int32_t wi, uint64_t r, uint64_t m) {
    const int64_t p = wmul(xi, (int64_t)wi);
    const uint64_t n = p < 0 ? 0ull - (uint64_t)p : (uint64_t)p;
    uint64_t q = n;
    if (r > 1) {
      q = __umul64hi(n, m);
      if (n - q * r >= r) q++;
    }
    const int64_t v = (p < 0 ? (int64_t)(0ull - q) : (int64_t)q) >> 8;
    y[i] = v;
    put_digits(a.planes, a.bp, a.kp, b, i, v, a.oflag);
  };
  auto rms_of = [&](uint64_t ss, uint64_t &m) {
    uint64_t r = isqrt64(ss / a.dim + 42950u);
    if (r < 1) r = 1;
    // floor(2^64 / r) (r < 2^32: an isqrt of a 64-bit word); unused for r = 1
    m = r > 1 ? recip64_32((uint32_t)r) : 0;
    return r;
  };
  if (whole) {
    // The whole vector fits in registers: x and the weights are read once,
    // together.  gridDim.y workgroups share a run: each sums all of x (a
    // few L2 reads) and finishes its own share of the registers, so the
    // stores spread over more compute units.
    uint64_t ss = 0;
    if (!xu) {
#pragma unroll
      for (int u = 0; u < U; u++) {
        const uint32_t i = threadIdx.x + u * nt;
        xv[u] = i < a.dim ? x[i] : 0;
        wv[u] = i < a.dim ? a.w[i] : 0;
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) ss += (uint64_t)wmul(xv[u], xv[u]);
    ss = block_sum_u64(ss, scratch);
    if (!live) return;
    uint64_t m;
    const uint64_t r = rms_of(ss, m);
    const uint32_t part = blockIdx.y, parts = gridDim.y;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t i = threadIdx.x + u * nt;
      if ((u * parts) / U == part && i < a.dim) finish(i, xv[u], wv[u], r, m);
    }
    return;
  }
  if (blockIdx.y != 0) return;
  uint64_t ss = 0;
  for (uint32_t base = threadIdx.x; base < a.dim; base += nt * U) {
    int64_t v[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t i = base + u * nt;
      v[u] = i < a.dim ? x[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; u++) ss += (uint64_t)wmul(v[u], v[u]);
  }
  ss = block_sum_u64(ss, scratch);
  uint64_t m;
  const uint64_t r = rms_of(ss, m);
  for (uint32_t base = threadIdx.x; base < a.dim; base += nt * U) {
    int64_t xv[U];
    int32_t wv[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t i = base + u * nt;
      xv[u] = i < a.dim ? x[i] : 0;
      wv[u] = i < a.dim ? a.w[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t i = base + u * nt;
      if (i < a.dim) finish(i, xv[u], wv[u], r, m);
    }
  }
}

// ---------------------------------------------------------------------------
// The matrix row on the int8 matrix cores.
//
// A workgroup owns 16*MT rows and 16*BT runs; its four waves split the
// contraction into four contiguous ranges of 64-column blocks.  Each wave
// streams the weight and digit fragments of its range straight into
// registers, P blocks ahead, and keeps exact i32 sums per digit in the
// matrix-core accumulators; at the end the four partial sums meet in LDS and
// wave 0 runs the epilogue.  No wave waits on another inside the loop, and a
// row tile of only 16 rows still spreads a small matrix over every compute
// unit.  MFMA 16x16x64 lanes: lane (i = lane % 16, g = lane / 16) supplies
// row i of the weight tile and run i of the digit tile, columns
// [16g, 16g + 16) of the block; it receives rows 4g..4g+3 of run i.

// 16 raw weight bytes (weight + 128) of one row; bytes outside the matrix
// read as 0x80, which is the weight 0.
__device__ __forceinline__ v4i load_weights_raw(const uint8_t *W, uint32_t row, uint32_t rows,
                                                uint32_t cols, uint32_t k0, bool vec) {
  v4i r = {(int)0x80808080u, (int)0x80808080u, (int)0x80808080u, (int)0x80808080u};
  if (row >= rows) return r;
  const uint8_t *p = W + (uint64_t)row * cols + k0;
  if (vec && k0 + 16 <= cols) return *reinterpret_cast<const v4i *>(p);
  uint32_t w[4] = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
  for (int t = 0; t < 16; t++) {
    const uint32_t k = k0 + t;
    if (k < cols) w[t >> 2] = (w[t >> 2] & ~(0xFFu << (8 * (t & 3)))) | ((uint32_t)p[t] << (8 * (t & 3)));
  }
  r.x = (int)w[0]; r.y = (int)w[1]; r.z = (int)w[2]; r.w = (int)w[3];
  return r;
}

// PART: the launch of a position where some run starts or stops between two
// phases (RowsArgs::partial); only the row kernel instantiated for it checks
// each run's steps and picks up finished phases.
template <int EPI, bool PART>
__device__ __forceinline__ bool row_run_ok(const RowsArgs &a, uint32_t b) {
  if (b >= a.n_runs) return false;
  if (EPI == EPI_RAW) return true;
  const RunDesc &rd = a.runs[b];
  return live_at(rd, rd.flags, EPI == EPI_CLS ? RUN_GEN : RUN_ACTIVE, a.step, PART ? 1u : 0u);
}

template <int EPI>
__device__ __forceinline__ const int64_t *row_input(const RowsArgs &a, uint32_t b) {
  if (EPI == EPI_RAW) return a.x_raw + (uint64_t)b * a.cols;
  const RunDesc &rd = a.runs[b];
  const uint8_t *st = a.states + rd.base;
  const uint64_t off = a.in_sel == IN_W1 ? rd.off_w1 : a.in_sel == IN_W3 ? rd.off_w3 : rd.off_gate;
  return reinterpret_cast<const int64_t *>(st + off);
}

__device__ __forceinline__ bool fits32(int64_t v) { return v >= INT32_MIN && v <= INT32_MAX; }

__device__ __forceinline__ void fail(RunDesc &rd, uint32_t layer, uint32_t phase) {
  atomicMin(&rd.errkey, (layer << 8) | phase);
}


// The rows one wave finishes: 16 * MT rows in MT tiles of 16, from the
// segment (matrix) that holds them; for the gate/up pair, HALF tiles of the
// gate matrix and the same rows of the up matrix.  unit numbers the 16*MT-row
// units of the launch over all its segments in order (segment i starts at
// unit seg[i].unit0), so one workgroup may finish rows of two matrices.
// ptile is the packed 16-row tile the wave streams: that of rbase, or the
// matrix's last one for rows past its end (their sums are never stored).
// A wave that runs the epilogue (scales = true) fetches the scales of the
// rows its lanes finish here, long before the epilogue needs them.
template <int MT>
struct RowTile {
  uint32_t si;
  const uint8_t *Wp[MT];
  const uint8_t *Pp[MT];
  uint32_t rbase[MT], rcount[MT], ptile[MT];
  bool vecw[MT];
  uint32_t sc[MT][4];
};

template <int EPI, int MT>
__device__ __forceinline__ void row_tile(const RowsArgs &a, uint32_t unit, int lg, bool scales,
                                         RowTile<MT> &t) {
  constexpr int HALF = MT >= 2 ? MT / 2 : 1;
  t.si = 0;
  if (EPI != EPI_GATEUP)
    while (t.si + 1 < a.nseg && unit >= a.seg[t.si + 1].unit0) ++t.si;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const Seg &sg = EPI == EPI_GATEUP ? a.seg[mt < HALF ? 0 : 1] : a.seg[t.si];
    t.Wp[mt] = sg.W;
    t.Pp[mt] = sg.P;
    t.rcount[mt] = sg.rows;
    t.vecw[mt] = sg.pad != 0;
    t.rbase[mt] = EPI == EPI_GATEUP ? unit * 16 * HALF + 16 * (mt % HALF)
                                    : (unit - sg.unit0) * 16 * MT + 16 * mt;
    const uint32_t last = (sg.rows - 1) / 16;
    t.ptile[mt] = t.rbase[mt] / 16 < last ? t.rbase[mt] / 16 : last;
    if (scales) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t row = t.rbase[mt] + 4 * lg + j;
        t.sc[mt][j] = sg.S[row < t.rcount[mt] ? row : t.rcount[mt] - 1];
      }
    }
  }
}

// Exact 64-bit path: sum_c (b_c - 128) * x_c over columns [c_lo, c_hi) with
// wrapping products, for the outputs this lane holds.
template <int EPI, int MT, int BT, bool PART>
__device__ __forceinline__ void rows_exact(const RowsArgs &a, const RowTile<MT> &t, uint32_t b0,
                                           uint32_t c_lo, uint32_t c_hi, int li, int lg,
                                           int64_t (&v)[MT][BT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int bt = 0; bt < BT; bt++) {
      const uint32_t b = b0 + bt * 16 + li;
      const bool ok = row_run_ok<EPI, PART>(a, b);
      const int64_t *x = ok ? row_input<EPI>(a, b) : nullptr;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t row = t.rbase[mt] + 4 * lg + j;
        int64_t s = 0;
        if (ok && row < t.rcount[mt]) {
          if (t.Wp[mt] != nullptr) {
            const uint8_t *w = t.Wp[mt] + (uint64_t)row * a.cols;
            for (uint32_t k = c_lo; k < c_hi; k++) s = wadd(s, wmul((int64_t)w[k] - 128, x[k]));
          } else {
            // only the packed tiles (standalone call): byte (row, k) of tile
            // (row / 16, k / 64), lane 16 ((k % 64) / 16) + row % 16
            const uint8_t *P = t.Pp[mt] + (uint64_t)(row / 16) * a.kblocks * 1024 + (row % 16) * 16;
            for (uint32_t k = c_lo; k < c_hi; k++) {
              const uint8_t wb = P[(uint64_t)(k / 64) * 1024 + ((k % 64) / 16) * 256 + k % 16];
              s = wadd(s, wmul((int64_t)wb - 128, x[k]));
            }
          }
        }
        v[mt][bt][j] = s;
      }
    }
}


// What a lane's epilogue needs besides its sums, fetched while the matrix
// streams so that the epilogue waits on nothing: the descriptor fields of
// its runs (issued first), then the state or table values the phase reads
// (issued after the first matrix loads).  Runs that do not exist read
// offsets 0 and clamped rows: valid addresses whose values are never used.
template <int EPI, int MT, int BT>
struct EpiIn {
  static constexpr int NX = (EPI == EPI_RESID || EPI == EPI_DOWN) ? MT : 1;
  static constexpr int NR = EPI == EPI_QKV ? MT : 1;
  uint32_t flags[BT], pos[BT], cache[BT];
  uint64_t base[BT], o1[BT], o2[BT], o3[BT];
  int64_t x[NX][BT][4];
  int32_t c[NR][BT][2], s[NR][BT][2];
};

template <int EPI, int MT, int BT>
__device__ __forceinline__ void epi_begin(const RowsArgs &a, uint32_t b0, int li,
                                          EpiIn<EPI, MT, BT> &in) {
#pragma unroll
  for (int bt = 0; bt < BT; bt++) {
    const uint32_t b = b0 + bt * 16 + li;
    in.flags[bt] = 0; in.pos[bt] = 0; in.cache[bt] = 0;
    in.base[bt] = 0; in.o1[bt] = 0; in.o2[bt] = 0; in.o3[bt] = 0;
    if (EPI == EPI_RAW) {
      in.flags[bt] = b < a.n_runs ? 1u : 0u;
      continue;
    }
    const RunDesc &rd = a.runs[b < a.n_runs ? b : 0];
    in.flags[bt] = b < a.n_runs ? rd.flags : 0u;
    in.base[bt] = rd.base;
    if (EPI == EPI_CLS) in.o1[bt] = rd.off_logits;
    if (EPI == EPI_RESID || EPI == EPI_DOWN) { in.o1[bt] = rd.off_x; in.o2[bt] = rd.off_w1; }
    if (EPI == EPI_GATEUP) { in.o1[bt] = rd.off_gate; in.o2[bt] = rd.off_up; }
    if (EPI == EPI_QKV) {
      in.pos[bt] = rd.pos;
      in.cache[bt] = rd.cachepos;
      in.o1[bt] = rd.off_w2; in.o2[bt] = rd.off_keys; in.o3[bt] = rd.off_values;
    }
  }
}

template <int EPI, bool PART>
__device__ __forceinline__ bool epi_live(const RowsArgs &a, uint32_t flags, uint32_t b) {
  if (EPI == EPI_RAW) return flags != 0;
  return live_at(a.runs[b < a.n_runs ? b : 0], flags, EPI == EPI_CLS ? RUN_GEN : RUN_ACTIVE, a.step,
                 PART ? 1u : 0u);
}

template <int EPI, int MT, int BT>
__device__ __forceinline__ void epi_fetch(const RowsArgs &a, const RowTile<MT> &t, int lg,
                                          EpiIn<EPI, MT, BT> &in) {
  if constexpr (EPI == EPI_RESID || EPI == EPI_DOWN) {
#pragma unroll
    for (int bt = 0; bt < BT; bt++) {
      const int64_t *x = reinterpret_cast<const int64_t *>(a.states + in.base[bt] + in.o1[bt]);
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const uint32_t row = t.rbase[mt] + 4 * lg + j;
          in.x[mt][bt][j] = x[row < t.rcount[mt] ? row : t.rcount[mt] - 1];
        }
    }
  }
  if constexpr (EPI == EPI_QKV) {
#pragma unroll
    for (int bt = 0; bt < BT; bt++) {
      const int32_t *cs = a.rope_cos + (uint64_t)in.pos[bt] * a.half;
      const int32_t *sn = a.rope_sin + (uint64_t)in.pos[bt] * a.half;
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int jp = 0; jp < 2; jp++) {
          const uint32_t row = t.rbase[mt] + 4 * lg + 2 * jp;
          const uint32_t p = ((row < t.rcount[mt] ? row : 0) % a.head) >> 1;
          in.c[mt][bt][jp] = cs[p];
          in.s[mt][bt][jp] = sn[p];
        }
    }
  }
}

// The first 4096 entries of the SiLU table (the only ones an index can
// reach) into LDS with direct global-to-LDS loads: 16 of 1 KB, shared out
// over the workgroup's waves.
__device__ __forceinline__ void silu_to_lds(const int32_t *silu, int32_t *lds, int wave, int nwaves,
                                            int lane) {
  for (int i = wave; i < 16; i += nwaves)
    __builtin_amdgcn_global_load_lds((const void *)(silu + i * 256 + lane * 4),
                                     (lds_void *)(lds + i * 256), 16, 0, 0);
}

// Epilogue of the outputs this lane holds: y = (v * scale) >> 24, then the
// phase's own work.
template <int EPI, int MT, int BT, bool PART>
__device__ __forceinline__ void rows_epilogue(const RowsArgs &a, const RowTile<MT> &t, uint32_t b0,
                                              const int64_t (&v)[MT][BT][4], int li, int lg,
                                              const EpiIn<EPI, MT, BT> &in, const int32_t *silu) {
  constexpr int HALF = MT >= 2 ? MT / 2 : 1;
  const uint32_t si = t.si;
  const auto &rbase = t.rbase;
  const auto &rcount = t.rcount;
  const auto &sc = t.sc;
#pragma unroll
  for (int bt = 0; bt < BT; bt++) {
    const uint32_t b = b0 + bt * 16 + li;
    if (!epi_live<EPI, PART>(a, in.flags[bt], b)) continue;
    int64_t y[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const uint32_t row = rbase[mt] + 4 * lg + j;
        y[mt][j] = row < rcount[mt] ? wmul(v[mt][bt][j], (int64_t)(uint64_t)sc[mt][j]) >> 24 : 0;
      }
    if (EPI == EPI_RAW) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const uint32_t row = rbase[mt] + 4 * lg + j;
          if (row < rcount[mt]) a.y_raw[(uint64_t)b * rcount[mt] + row] = y[mt][j];
        }
      continue;
    }
    RunDesc &rd = a.runs[b];  // only for recording a fit failure
    uint8_t *st = a.states + in.base[bt];
    // A run that stopped inside this launch's phases: the results of the
    // phases it finished come from its state instead of the sums.
    const uint32_t pick = PART ? pick_at(in.flags[bt], a.step, 1u) : 0u;
    // A turn of units that stops the run inside this launch: the phase and
    // row of the stop.  The launch writes what the phases before the stop
    // leave in the state (matrix rows below the row, nothing turned, no
    // residual or SiLU yet) and nothing after it.
    uint32_t sp = 0, sr = 0;
    if (PART) {
      const RunDesc &rs = a.runs[b];
      if (rs.stop_ph != 0 && a.step == rs.stop_in) { sp = rs.stop_ph; sr = rs.stop_row; }
    }
#pragma unroll
    for (int mt = 0; mt < (EPI == EPI_GATEUP ? HALF : MT); mt++) {
      const uint32_t r0 = rbase[mt] + 4 * lg;
      if (EPI == EPI_CLS) {
        int64_t *lg_out = reinterpret_cast<int64_t *>(st + in.o1[bt]);
#pragma unroll
        for (int j = 0; j < 4; j++)
          if (r0 + j < rcount[mt] && (sp == 0 || r0 + j < sr)) lg_out[r0 + j] = y[mt][j];
      } else if (EPI == EPI_RESID || EPI == EPI_DOWN) {
        int64_t *x = reinterpret_cast<int64_t *>(st + in.o1[bt]);
        int64_t *w1 = reinterpret_cast<int64_t *>(st + in.o2[bt]);
        // picked up at 11 or 16: the matrix's output is already in w1
        const bool held = pick == (EPI == EPI_RESID ? 11u : 16u);
        // stopped at 10 or 15 (a row of the matrix) or 11 or 16 (before the
        // residual): the rows so far in w1, x as it was
        const uint32_t lim = (sp == 10 || sp == 15) ? sr : rcount[mt];
#pragma unroll
        for (int j = 0; j < 4; j++)
          if (r0 + j < rcount[mt]) {
            const int64_t yv = held ? w1[r0 + j] : y[mt][j];
            if (sp != 0) {
              if (r0 + j < lim) w1[r0 + j] = yv;
              continue;
            }
            if (EPI == EPI_DOWN) w1[r0 + j] = yv;
            x[r0 + j] = wadd(in.x[EPI == EPI_RESID || EPI == EPI_DOWN ? mt : 0][bt][j], yv);
          }
      } else if (EPI == EPI_GATEUP) {
        // Phase 14: h = (SILU(gate) * up) >> 16, kept in the gate vector.
        int64_t *gate = reinterpret_cast<int64_t *>(st + in.o1[bt]);
        int64_t *up = reinterpret_cast<int64_t *>(st + in.o2[bt]);
        const int64_t lim = (int64_t)16 << 16;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const uint32_t row = r0 + j;
          if (row >= a.hidden) continue;
          // picked up at 13: the gate is in the state; at 14 the up rows
          // too; at 15 the product is already in the gate vector
          const int64_t g = pick >= 13 ? gate[row] : y[mt][j];
          const int64_t u = pick >= 14 ? up[row] : y[mt + HALF][j];
          if (sp != 0) {
            // stopped at 12 or 13 (a row of the gate or up rows) or 14
            // (before SiLU): the rows so far, as they come from the matrices
            if (sp > 12 || row < sr) gate[row] = g;
            if (sp == 14 || (sp == 13 && row < sr)) up[row] = u;
            continue;
          }
          const int64_t sg = g >= lim ? g : g <= -lim ? 0 : (int64_t)silu[(g + lim) >> 9];
          const int64_t h = pick == 15 ? g : wmul(sg, u) >> 16;
          gate[row] = h;
          up[row] = u;
          put_digits(a.planes_out, a.bp, a.kp_out, b, row, h, a.oflag_out);
        }
      } else if (EPI == EPI_QKV) {
        const uint32_t role = a.seg[si].role;
        const uint32_t pos = in.pos[bt];
        if (role == ROLE_V) {
          // Phase 7: the value rows into the cache, each checked to fit 32 bits.
          int32_t *V = reinterpret_cast<int32_t *>(st + in.o3[bt]);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const uint32_t row = r0 + j;
            if (row >= rcount[mt]) continue;
            const uint32_t kvh = row / a.head, e = row % a.head;
            int32_t *dst = V + (((uint64_t)a.layer * a.kv_heads + kvh) * in.cache[bt] + pos) * a.head + e;
            const int64_t yv = pick >= 8 ? (int64_t)*dst : y[mt][j];  // stored before the cut
            if (sp != 0 && (sp < 7 || (sp == 7 && row >= sr))) continue;  // not reached by the stop
            if (!fits32(yv)) { fail(rd, a.layer, 7); continue; }
            *dst = (int32_t)yv;
          }
        } else {
          // Phase 8 on the query (kept in w2) and on the key after its
          // phase-6 store check: pairs (2p, 2p+1) of each head turned by
          // position pos's cosine and sine p.
          int64_t *q = reinterpret_cast<int64_t *>(st + in.o1[bt]);
          int32_t *K = reinterpret_cast<int32_t *>(st + in.o2[bt]);
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const uint32_t row = r0 + j;
            if (row >= rcount[mt]) continue;
            int32_t *dst = nullptr;  // the key's cache words
            if (role == ROLE_K)
              dst = K + (((uint64_t)a.layer * a.kv_heads + row / a.head) * in.cache[bt] + pos) * a.head + row % a.head;
            // picked up at 6 or later: the query (unturned) is in w2; at 7
            // or later the key (unturned) is in the cache
            int64_t A0 = y[mt][j], B0 = y[mt][j + 1];
            if (role == ROLE_Q && pick >= 6) { A0 = q[row]; B0 = q[row + 1]; }
            if (role == ROLE_K && pick >= 7) { A0 = dst[0]; B0 = dst[1]; }
            if (sp != 0) {
              // stopped at 5 (a query row), 6 (a key row), 7 or 8 (before
              // rotary): the rows so far, unturned
              const uint32_t lim = role == ROLE_Q ? (sp == 5 ? sr : rcount[mt])
                                                  : (sp < 6 ? 0u : sp == 6 ? sr : rcount[mt]);
              for (int e = 0; e < 2; e++) {
                if (row + e >= lim) continue;
                const int64_t val = e ? B0 : A0;
                if (role == ROLE_Q) {
                  q[row + e] = val;
                } else if (!fits32(val)) {
                  fail(rd, a.layer, 6);
                } else {
                  dst[e] = (int32_t)val;
                }
              }
              continue;
            }
            if (role == ROLE_K && (!fits32(A0) || !fits32(B0))) { fail(rd, a.layer, 6); continue; }
            const int64_t c = in.c[EPI == EPI_QKV ? mt : 0][bt][j >> 1];
            const int64_t s = in.s[EPI == EPI_QKV ? mt : 0][bt][j >> 1];
            const int64_t ra = wsub(wmul(A0, c), wmul(B0, s)) >> 24;
            const int64_t rb = wadd(wmul(A0, s), wmul(B0, c)) >> 24;
            if (role == ROLE_Q) {
              q[row] = ra;
              q[row + 1] = rb;
            } else {
              if (!fits32(ra) || !fits32(rb)) { fail(rd, a.layer, 8); continue; }
              dst[0] = (int32_t)ra;
              dst[1] = (int32_t)rb;
            }
          }
        }
      }
    }
  }
}



// Blocks in flight per wave: the fragments of a block take 4 * (MT + 3 BT)
// VGPRs (4 * MT when the digits come from LDS), and about 190 of them hold
// the prefetch ring.
template <int MT, int BT, bool XR = false>
struct RowsGeom {
  static constexpr int FRAG = MT + (XR ? 0 : 3 * BT);
  static constexpr int P0 = 48 / FRAG;
  static constexpr int P = P0 < 2 ? 2 : P0 > 12 ? 12 : P0;
};

// XR (standalone calls of one or two inputs): no digit planes;
// each wave reads its own columns of the raw inputs, splits them into
// digits in LDS (kRawInputLds bytes a wave: 3 limbs x inputs x its column
// span), and takes the exact path by itself when one of its words needs more.
constexpr uint32_t XR_CAP = kRawInputLds;

template <int EPI, int MT, int BT, bool XR = false, bool PART = false>
__global__ __launch_bounds__(256) void k_rows(RowsArgs a) {
  static_assert(!XR || (EPI == EPI_RAW && BT == 1), "raw-input rows are standalone calls of one or two inputs");
  constexpr int P = RowsGeom<MT, BT, XR>::P;
  __shared__ int64_t red[3][MT * BT * 4 * 64];
  __shared__ int32_t silu_lds[EPI == EPI_GATEUP ? 4096 : 1];
  __shared__ __align__(16) int8_t xdig[XR ? 4 * XR_CAP : 16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 15, lg = lane >> 4;

  // Workgroup -> (row tile, batch chunk).  The batch chunks of one row tile
  // get workgroup ids 8 apart, which the dispatcher places on one XCD, so
  // the tile's weight rows come from HBM once and from that XCD's L2 after.
  const uint32_t nchunk = a.chunks;
  const uint32_t grp = blockIdx.x / (8 * nchunk), rem = blockIdx.x % (8 * nchunk);
  const uint32_t chunk = rem / 8, tile = grp * 8 + rem % 8;
  if (tile >= a.ntiles) return;
  const uint32_t b0 = chunk * BT * 16;

  // Whether this batch chunk has a run in this phase (the classifier skips
  // prompt positions and finished runs); read first, tested after the first
  // loads are on their way.
  const bool busy = EPI == EPI_RAW || row_run_ok<EPI, PART>(a, b0 + (tid & (16 * BT - 1)));

  RowTile<MT> t;
  row_tile<EPI, MT>(a, tile, lg, wave == 0, t);
  EpiIn<EPI, MT, BT> in;
  if (wave == 0) epi_begin<EPI, MT, BT>(a, b0, li, in);  // only wave 0 runs the epilogue
  if constexpr (EPI == EPI_GATEUP) silu_to_lds(a.silu, silu_lds, wave, 4, lane);

  // This wave's blocks [k_lo, k_lo + n).
  const uint32_t nkb = a.kblocks, per = (nkb + 3) / 4;
  const uint32_t k_lo = wave * per < nkb ? wave * per : nkb;
  const uint32_t n = (k_lo + per < nkb ? k_lo + per : nkb) - k_lo;

  v4i acc[MT][3][BT];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int l = 0; l < 3; l++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++) acc[mt][l][bt] = v4i{0, 0, 0, 0};

  // Digit fragments (l, bt, kb) are 1 KB apart per block in the
  // fragment-major planes.  Lanes of runs that do not exist load run 0's
  // bytes (the same address as a live lane, so no extra traffic), and rows
  // past the end of a segment re-read its last row: both only fill
  // product entries that are never stored.  Every load is unconditional,
  // which keeps the prefetch ring free of branches.
  const uint32_t live = a.n_runs > b0 ? a.n_runs - b0 : 0;
  const uint32_t kbp = a.kp / 64, nbt = a.bp / 16;
  const int8_t *dsrc[3][BT];
  const uint32_t dstride = a.compact ? 64 : 1024;  // bytes from one 64-column block to the next
#pragma unroll
  for (int bt = 0; bt < BT; bt++) {
    const uint32_t ie = bt * 16 + li < live ? li : 0;
#pragma unroll
    for (int l = 0; l < 3; l++)
      dsrc[l][bt] = a.compact
          ? a.planes + ((uint64_t)l * a.bp + b0 + bt * 16 + ie) * a.kp + (uint64_t)k_lo * 64 + lg * 16
          : a.planes + ((((uint64_t)l * nbt + (b0 >> 4) + bt) * kbp + k_lo) * 64 + lg * 16 + ie) * 16;
  }
  // Weights: the packed 1 KB tiles (whole cache lines per load), or the
  // rows themselves (rows past the end of a segment re-read its last row).
  const uint8_t *wsrc[MT];
  const uint32_t wstride = a.packed ? 1024 : 64;  // bytes from one 64-column block to the next
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const uint32_t row = t.rbase[mt] + li < t.rcount[mt] ? t.rbase[mt] + li : t.rcount[mt] - 1;
    wsrc[mt] = a.packed
        ? t.Pp[mt] + ((uint64_t)t.ptile[mt] * a.kblocks + k_lo) * 1024 + lane * 16
        : t.Wp[mt] + (uint64_t)row * a.cols + (uint64_t)k_lo * 64 + lg * 16;
  }

  // XR: this wave's digits, [limb][input][column of its span], in LDS.
  const uint32_t span = per * 64;
  int8_t *xd = xdig + (XR ? wave * XR_CAP : 0);
  bool x_exact = false;
  const uint32_t xrun = li < a.n_runs ? li : 0;  // XR: the input this lane's product column takes

  v4i Wr[P][MT], Dr[XR ? 1 : P][3][BT];
  auto load_digits = [&](int s, uint32_t i) {
    if constexpr (!XR) {
#pragma unroll
      for (int l = 0; l < 3; l++)
#pragma unroll
        for (int bt = 0; bt < BT; bt++)
          Dr[s][l][bt] = *reinterpret_cast<const v4i *>(dsrc[l][bt] + (uint64_t)i * dstride);
    }
  };
  // Block k_lo + i into ring slot s: whole 16-byte pieces of aligned rows.
  // The scheduling fences keep each slot's loads together and in ring
  // order, so the oldest slot is always the next one computed.
  auto load = [&](int s, uint32_t i) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0; mt < MT; mt++) Wr[s][mt] = *reinterpret_cast<const v4i *>(wsrc[mt] + (uint64_t)i * wstride);
    load_digits(s, i);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The same with every byte checked against the matrix (bytes outside
  // it read as the weight 0).
  auto load_checked = [&](int s, uint32_t i) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
      Wr[s][mt] = load_weights_raw(t.Wp[mt], t.rbase[mt] + li, t.rcount[mt], a.cols, (k_lo + i) * 64 + lg * 16, t.vecw[mt]);
    load_digits(s, i);
  };
  // Ring slot s, which holds block k_lo + i.
  auto compute = [&](int s, uint32_t i) {
    const int flip = (int)0x80808080u;
    v4i w[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      w[mt] = Wr[s][mt];
      w[mt].x ^= flip; w[mt].y ^= flip; w[mt].z ^= flip; w[mt].w ^= flip;
    }
#pragma unroll
    for (int l = 0; l < 3; l++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++) {
        v4i d;
        if constexpr (XR)
          d = *reinterpret_cast<const v4i *>(xd + ((uint64_t)l * a.n_runs + xrun) * span + i * 64 + lg * 16);
        else
          d = Dr[s][l][bt];
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
          acc[mt][l][bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[mt], d, acc[mt][l][bt], 0, 0, 0);
      }
  };

  // Whole 64-column blocks of this wave, then (for the wave that owns it)
  // the partial block at the end of the rows.
  const uint32_t nfull = a.packed ? nkb : a.cols / 64;
  const uint32_t n_main = k_lo >= nfull ? 0 : (k_lo + n < nfull ? n : nfull - k_lo);
  bool fast = true;
#pragma unroll
  for (int mt = 0; mt < MT; mt++) fast = fast && t.vecw[mt];
  fast = fast || a.packed != 0;
  // XR: split this wave's columns of the inputs into digits in LDS (16
  // columns a lane, both inputs' words requested before any is used).  It
  // goes before the weight tiles: a wait for the inputs would otherwise
  // wait for every tile requested before them.
  if constexpr (XR) {
    bool fits = true;
    for (uint32_t c = 16 * lane; c < n * 64; c += 1024) {
      // columns of the row left from here; none in the padding blocks past its end
      const int64_t room = (int64_t)a.cols - (int64_t)(k_lo * 64 + c);
      int64_t xv[2][16];
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const int64_t *xr = a.x_raw + (uint64_t)b * a.cols + (uint64_t)k_lo * 64 + c;
#pragma unroll
        for (int e = 0; e < 16; e++) xv[b][e] = (uint32_t)b < a.n_runs && e < room ? xr[e] : 0;
      }
#pragma unroll
      for (int b = 0; b < 2; b++) {
        if ((uint32_t)b >= a.n_runs) break;
        uint32_t w[3][4] = {};
#pragma unroll
        for (int e = 0; e < 16; e++) {
          int8_t d0, d1, d2;
          fits = digits3(xv[b][e], d0, d1, d2) && fits;
          const int sh = 8 * (e & 3);
          w[0][e >> 2] |= (uint32_t)(uint8_t)d0 << sh;
          w[1][e >> 2] |= (uint32_t)(uint8_t)d1 << sh;
          w[2][e >> 2] |= (uint32_t)(uint8_t)d2 << sh;
        }
#pragma unroll
        for (int l = 0; l < 3; l++)
          *reinterpret_cast<v4i *>(xd + ((uint64_t)l * a.n_runs + b) * span + c) =
              v4i{(int)w[l][0], (int)w[l][1], (int)w[l][2], (int)w[l][3]};
      }
    }
    x_exact = __any(fits ? 0 : 1) != 0;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's own digit stores, before its reads
  }
  // The ring's first P blocks go out before anything waits.
  const uint32_t last = n_main ? n_main - 1 : 0;
  if (fast && n_main > 0) {
#pragma unroll
    for (int s = 0; s < P; s++) load(s, (uint32_t)s < n_main ? (uint32_t)s : last);
  }
  if (wave == 0) epi_fetch<EPI, MT, BT>(a, t, lg, in);

  // The input needs more than three digits somewhere: exact path (a scalar
  // read, so it does not wait behind the loads above).
  const bool exact = input_needs_exact(a);
  if (EPI != EPI_RAW && !__any(busy ? 1 : 0)) {  // every wave sees all runs of the chunk
    wait_vm<0>();  // no table load may still be landing in LDS
    return;
  }

  int64_t v[MT][BT][4];
  if (!exact && !x_exact) {
    if (fast && n_main > 0) {
      // P blocks in flight; the loop body has no branches, so the compiler
      // waits only for the slot about to be used.
      uint32_t i = 0;
      for (; i + 2 * P <= n_main; i += P) {
#pragma unroll
        for (int s = 0; s < P; s++) {
          compute(s, i + s);
          load(s, i + s + P);
        }
      }
#pragma unroll
      for (int s = 0; s < P; s++) {
        if (i + s < n_main) compute(s, i + s);
        const uint32_t nx = i + s + P;
        load(s, nx < n_main ? nx : last);
      }
      i += P;
#pragma unroll
      for (int s = 0; s < P; s++)
        if (i + s < n_main) compute(s, i + s);
    } else {
      for (uint32_t i = 0; i < n_main; i++) {
        load_checked(0, i);
        compute(0, i);
      }
    }
    if (nfull < nkb && k_lo <= nfull && nfull < k_lo + n) {
      load_checked(0, nfull - k_lo);
      compute(0, nfull - k_lo);
    }

#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          v[mt][bt][j] = (int64_t)acc[mt][0][bt][j] + ((int64_t)acc[mt][1][bt][j] << 8) +
                         ((int64_t)acc[mt][2][bt][j] << 16);
  } else {
    // Exact 64-bit path over this wave's columns.
    const uint32_t c_lo = k_lo * 64, c_hi = (k_lo + n) * 64 < a.cols ? (k_lo + n) * 64 : a.cols;
    rows_exact<EPI, MT, BT, PART>(a, t, b0, c_lo, c_hi, li, lg, v);
  }

  // The four waves' sums meet in wave 0 (wrapping adds).
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++)
#pragma unroll
        for (int j = 0; j < 4; j++) red[wave - 1][((mt * BT + bt) * 4 + j) * 64 + lane] = v[mt][bt][j];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; w++)
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++)
#pragma unroll
        for (int j = 0; j < 4; j++) v[mt][bt][j] = wadd(v[mt][bt][j], red[w][((mt * BT + bt) * 4 + j) * 64 + lane]);

  rows_epilogue<EPI, MT, BT, PART>(a, t, b0, v, li, lg, in, silu_lds);
}

// The matrix row with the digits shared through LDS.  A workgroup of W
// waves owns wave_rows * 16 * MT rows (wave_rows of its waves each own
// 16 * MT of them: 3 or 4 of four, or all W of 3, 6 or 12) and 16 * BT runs,
// over the whole contraction.  All W waves stage each run of CD 64-column
// blocks of digit fragments into an LDS ring with direct global-to-LDS
// loads (an equal share each), P stages ahead, and every row-owning wave
// streams its own weight rows into a register ring of the same depth; one
// barrier per stage.  The digits then cross L2 once per wave_rows * 16 * MT
// rows rather than once per 16 * MT.  More waves than the four SIMDs keep
// more weight loads in flight and let one wave's matrix-core work overlap
// another's waits.  For packed matrices (kblocks even), or rows that are
// 16-byte aligned with a column count that is a multiple of 64 * CD.
template <int BT, int CD, int W, int PP = 0>
struct SharedGeom {
  static constexpr int FR = 3 * BT * CD;       // digit fragments per stage
  static constexpr int FW = FR / W;            // fragments each wave stages
  // stages in flight: PP when given, else 3 (4 for two-block stages of up
  // to 32 runs)
  static constexpr int P = PP > 0 ? PP : CD == 1 ? 3 : BT >= 4 ? 3 : 4;
  static constexpr int NB = P + 1;             // stage buffers (LDS and registers)
  static_assert(FR % W == 0, "every wave stages the same number of fragments");
  static_assert(NB <= 8, "at most eight stage buffers");
};


// Stage buffer I of the LDS ring: one distinct LDS object per buffer, so the
// compiler can tell which staging loads a read of the buffer waits for.
template <int I, int N>
__device__ __forceinline__ v4i *ring_buf() {
  __shared__ v4i buf[N];
  return buf;
}

template <int EPI, int MT, int BT, int W = 4, int CD = 2, int PP = 0>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(W == 4 && BT <= 2 ? 2 : 1))) void k_rows_shared(RowsArgs a) {
  using G = SharedGeom<BT, CD, W, PP>;
  constexpr int FR = G::FR, FW = G::FW, P = G::P, NB = G::NB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: branches on it are scalar
  const int li = lane & 15, lg = lane >> 4;

  // Workgroup -> (row tile, batch chunk), chunks of a tile 8 ids apart.  A
  // row tile is wave_rows units of 16 * MT rows, one per wave that owns
  // rows; the other waves only stage digits (the same rows are then
  // covered by more workgroups, so more compute units stream weights).
  const uint32_t nchunk = a.chunks;
  const uint32_t grp = blockIdx.x / (8 * nchunk), rem = blockIdx.x % (8 * nchunk);
  const uint32_t chunk = rem / 8, tile = grp * 8 + rem % 8;
  if (tile >= a.ntiles) return;
  const uint32_t b0 = chunk * BT * 16;
  const uint32_t wr = a.wave_rows;
  const bool own = (uint32_t)wave < wr;
  // Whether this batch chunk has a run in this phase; read first, tested
  // after the first stages are on their way.
  const bool busy = EPI == EPI_RAW || row_run_ok<EPI, false>(a, b0 + (tid & (16 * BT - 1)));

  __shared__ int32_t silu_lds[EPI == EPI_GATEUP ? 4096 : 1];
  RowTile<MT> t;
  row_tile<EPI, MT>(a, tile * wr + (own ? wave : 0), lg, own, t);

  const uint32_t nch = a.kblocks / CD;
  const uint32_t kbp = a.kp / 64, nbt = a.bp / 16;
  const uint8_t *wsrc[MT];
  const uint32_t wstride = a.packed ? 1024 : 64;  // bytes from one 64-column block to the next
#pragma unroll
  for (int mt = 0; mt < MT; mt++) {
    const uint32_t row = t.rbase[mt] + li < t.rcount[mt] ? t.rbase[mt] + li : t.rcount[mt] - 1;
    wsrc[mt] = a.packed ? t.Pp[mt] + (uint64_t)t.ptile[mt] * a.kblocks * 1024 + lane * 16
                        : t.Wp[mt] + (uint64_t)row * a.cols + lg * 16;
  }
  // This wave stages fragments f = wave + Wq of every stage; fragment f
  // is (limb l, run tile bt, block c).  Runs past the batch bring
  // whatever their plane rows hold; those product columns are never stored.
  const int8_t *dsrc[FW];
#pragma unroll
  for (int q = 0; q < FW; q++) {
    const int f = wave + W * q;
    const int l = f / (BT * CD), bt = (f / CD) % BT, c = f % CD;
    dsrc[q] = a.planes + ((((uint64_t)l * nbt + (b0 >> 4) + bt) * kbp + c) * 64 + lane) * 16;
  }
  v4i *ring[NB];
  ring[0] = ring_buf<0, FR * 64>();
  ring[1] = ring_buf<1, FR * 64>();
  ring[2] = ring_buf<2, FR * 64>();
  ring[3] = ring_buf<3, FR * 64>();
  if constexpr (NB > 4) ring[4] = ring_buf<4, FR * 64>();
  if constexpr (NB > 5) ring[5] = ring_buf<5, FR * 64>();
  if constexpr (NB > 6) ring[6] = ring_buf<6, FR * 64>();
  if constexpr (NB > 7) ring[7] = ring_buf<7, FR * 64>();

  v4i Wr[NB][MT][CD];
  // Stage st into buffer s (weights into register slot s, digits into LDS
  // buffer s), by a wave that owns rows (OWN) or only stages digits.
  auto issue = [&](auto own_tag, int s, uint32_t st) {
    constexpr bool OWN = decltype(own_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (OWN) {
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int c = 0; c < CD; c++)
          Wr[s][mt][c] = *reinterpret_cast<const v4i *>(wsrc[mt] + ((uint64_t)st * CD + c) * wstride);
    }
#pragma unroll
    for (int q = 0; q < FW; q++)
      __builtin_amdgcn_global_load_lds((const void *)(dsrc[q] + (uint64_t)st * CD * 1024),
                                       (lds_void *)(ring[s] + (wave + W * q) * 64), 16, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The ring's first P stages go out before anything waits (the run flags,
  // the descriptors, the inputs' digit check); the exact path and a chunk
  // with no run in this phase only drain them.
  const uint32_t last = nch - 1;
  if (own) {
#pragma unroll
    for (int s = 0; s < P; s++) issue(std::true_type{}, s, (uint32_t)s < nch ? (uint32_t)s : last);
  } else {
#pragma unroll
    for (int s = 0; s < P; s++) issue(std::false_type{}, s, (uint32_t)s < nch ? (uint32_t)s : last);
  }

  EpiIn<EPI, MT, BT> in;
  if (own) epi_begin<EPI, MT, BT>(a, b0, li, in);  // waves that own rows run an epilogue
  if constexpr (EPI == EPI_GATEUP) silu_to_lds(a.silu, silu_lds, wave, W, lane);
  const bool exact = input_needs_exact(a);
  if (EPI != EPI_RAW && !__any(busy ? 1 : 0)) {  // every wave sees all runs of the chunk
    wait_vm<0>();  // no staging or table load may still be landing in LDS
    return;
  }

  int64_t v[MT][BT][4];
  if (exact) {
    wait_vm<0>();  // the staged stages are not used; none may still be landing in LDS
    if (own) {
      epi_fetch<EPI, MT, BT>(a, t, lg, in);
      rows_exact<EPI, MT, BT, false>(a, t, b0, 0, a.cols, li, lg, v);
    }
  } else {
    v4i acc[MT][3][BT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int l = 0; l < 3; l++)
#pragma unroll
        for (int bt = 0; bt < BT; bt++) acc[mt][l][bt] = v4i{0, 0, 0, 0};

    // The stage loop, after the first P stages.
    auto stream = [&](auto own_tag) {
      constexpr bool OWN = decltype(own_tag)::value;
      constexpr int NL = (OWN ? MT * CD : 0) + FW;  // loads per stage
      auto compute = [&](int s) {
        if constexpr (OWN) {
          const int flip = (int)0x80808080u;
          const v4i *buf = ring[s];
#pragma unroll
          for (int c = 0; c < CD; c++) {
            v4i w[MT];
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
              w[mt] = Wr[s][mt][c];
              w[mt].x ^= flip; w[mt].y ^= flip; w[mt].z ^= flip; w[mt].w ^= flip;
            }
#pragma unroll
            for (int l = 0; l < 3; l++)
#pragma unroll
              for (int bt = 0; bt < BT; bt++) {
                const v4i Bv = buf[((l * BT + bt) * CD + c) * 64 + lane];
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
                  acc[mt][l][bt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[mt], Bv, acc[mt][l][bt], 0, 0, 0);
              }
          }
        }
      };
      // Stage k lives in buffer k % NB.  Once stage k has landed and every
      // wave has passed the barrier (so all have finished stage k - 1), a
      // wave issues stage k + P (the last stage again when there is no
      // further one) into buffer (k + P) % NB, the one stage k - 1 used,
      // then computes stage k.  P - 1 younger stages are in flight at every
      // wait (and the loads issued after the first P stages, which only
      // make the first waits longer).
      if constexpr (OWN) epi_fetch<EPI, MT, BT>(a, t, lg, in);
      uint32_t ch = 0;
      for (; ch + NB <= nch; ch += NB) {
#pragma unroll
        for (int s = 0; s < NB; s++) {
          wait_vm<(P - 1) * NL>();
          lds_barrier();
          const uint32_t nx = ch + s + P;
          issue(own_tag, (s + P) % NB, nx < nch ? nx : last);
          compute(s);
        }
      }
#pragma unroll
      for (int s = 0; s < NB; s++) {
        if (ch + s < nch) {
          wait_vm<(P - 1) * NL>();
          lds_barrier();
          const uint32_t nx = ch + s + P;
          issue(own_tag, (s + P) % NB, nx < nch ? nx : last);
          compute(s);
        }
      }
      // No staging load may still be landing in LDS when the workgroup ends.
      wait_vm<0>();
    };
    if (own)
      stream(std::integral_constant<bool, true>{});
    else
      stream(std::integral_constant<bool, false>{});
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int bt = 0; bt < BT; bt++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          v[mt][bt][j] = (int64_t)acc[mt][0][bt][j] + ((int64_t)acc[mt][1][bt][j] << 8) +
                         ((int64_t)acc[mt][2][bt][j] << 16);
  }
  if constexpr (EPI == EPI_GATEUP) {
    wait_vm<0>();
    lds_barrier();  // every wave's share of the SiLU table has landed
  }
  if (own) rows_epilogue<EPI, MT, BT, false>(a, t, b0, v, li, lg, in, silu_lds);
}

// Packing of a weight matrix into MFMA operand tiles (see launch_pack): one
// thread per 16-byte piece of a tile.
__global__ __launch_bounds__(256) void k_pack(const uint8_t *W, uint32_t rows, uint32_t cols,
                                              uint32_t kbp, uint8_t *P, uint64_t pieces) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const uint32_t lane = (uint32_t)(i % 64);
  const uint64_t tile = i / 64;
  const uint32_t kb = (uint32_t)(tile % kbp), rt = (uint32_t)(tile / kbp);
  const uint32_t row = rt * 16 + lane % 16, c0 = kb * 64 + (lane / 16) * 16;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint32_t c = c0 + 4 * q + e;
      const uint32_t byte = row < rows && c < cols ? W[(uint64_t)row * cols + c] : 0x80u;
      v |= byte << (8 * e);
    }
    w[q] = v;
  }
  *reinterpret_cast<v4i *>(P + i * 16) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

// Digits of a plain i64 matrix [n_runs][cols] (standalone matrix rows).
__global__ __launch_bounds__(256) void k_digits_raw(const int64_t *x, uint32_t n_runs, uint32_t cols,
                                                    int8_t *planes, uint32_t kp, uint32_t bp,
                                                    uint32_t compact, uint32_t *oflag, uint32_t seq) {
  const uint32_t b = blockIdx.y, k = blockIdx.x * blockDim.x + threadIdx.x;
  bool over = false;
  if (b < n_runs && k < cols) {
    int8_t d0, d1, d2;
    over = !digits3(x[(uint64_t)b * cols + k], d0, d1, d2);
    const uint64_t limb = (uint64_t)bp * kp;
    const uint64_t at = compact ? (uint64_t)b * kp + k : digit_at(b, k, kp);
    planes[at] = d0;
    planes[limb + at] = d1;
    planes[2 * limb + at] = d2;
  }
  if (__syncthreads_or(over ? 1 : 0) && threadIdx.x == 0) atomicExch(oflag, seq);
}

// ---------------------------------------------------------------------------
// Phase 9, one workgroup per (run, head) ("Attention, stage by stage").
// Scores, exponentials and probabilities of the head's positions stay in
// LDS (one 64-bit slot per cached position); the exponential table is read
// from L2, where its 16 KB stay hot.

template <int HS>
__global__ __launch_bounds__(256) void k_attention(AttnArgs a) {
  __shared__ uint64_t scratch[8];
  __shared__ int64_t qs[256];
  extern __shared__ __align__(16) uint8_t lds[];
  int64_t *sc = reinterpret_cast<int64_t *>(lds);  // scores, then exponentials, then probabilities
  int64_t *red = sc + a.max_npos;

  const uint32_t h = blockIdx.x, b = blockIdx.y;
  const uint32_t hs = HS ? HS : a.head;
  const int tid = threadIdx.x, l16 = tid & 15, grp = tid >> 4;
  const uint32_t kvh = h / a.group;

  // Heads of a power-of-two size of at least 4 take the vector path: LPP
  // lanes hold one position's row, 16 bytes each, so one load instruction of
  // a wave reads 1 KB of consecutive rows; U positions per lane in flight.
  constexpr bool VEC = HS != 0 && HS % 4 == 0;
  constexpr int LPP = VEC ? HS / 4 : 1;  // lanes per position (<= 64)
  constexpr int GP = 256 / LPP;          // positions per workgroup step
  constexpr int U = 4;                   // positions per lane in one batch; two batches in flight
  const int lp = tid % LPP, pg = tid / LPP;

  // When every run has the same layout (a.u_first), the head's queries and
  // its first batch of keys are requested before the run's descriptor
  // arrives, so the two round trips overlap.  That batch's rows past the
  // cache read its last row (in bounds); like every row at or past the
  // position, they count for nothing.
  const bool pre = VEC && a.u_first != nullptr;
  int64_t qpre = 0;
  v4i A[U];
  if (pre) {
    const uint8_t *su = a.u_first + (uint64_t)b * a.u_stride;
    if (tid < (int)hs) qpre = reinterpret_cast<const int64_t *>(su + a.u_off_q)[(uint64_t)h * hs + tid];
    const int32_t *Ku = reinterpret_cast<const int32_t *>(su + a.u_off_keys) +
                        ((uint64_t)a.layer * a.kv_heads + kvh) * a.u_cachepos * hs;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint32_t j = pg + GP * u;
      A[u] = __builtin_nontemporal_load(
          reinterpret_cast<const v4i *>(Ku + (uint64_t)(j < a.u_cachepos ? j : a.u_cachepos - 1) * hs + 4 * lp));
    }
  }

  // The descriptor fields this kernel reads, requested together (one round
  // trip rather than one per test below).
  const RunDesc &rd = a.runs[b];
  const uint32_t flags = rd.flags, pos = rd.pos, rend = rd.end, cachepos = rd.cachepos;
  const uint32_t stop_ph = rd.stop_ph, stop_in = rd.stop_in, stop_row = rd.stop_row;
  const uint64_t base = rd.base, off_w2 = rd.off_w2, off_keys = rd.off_keys, off_values = rd.off_values;
  const uint32_t partial = a.partial, step = a.step;
  asm volatile("" ::"s"(flags), "s"(pos), "s"(rend), "s"(cachepos), "s"(stop_ph), "s"(stop_in), "s"(stop_row),
               "s"(base), "s"(off_w2), "s"(off_keys), "s"(off_values), "s"(partial), "s"(step));
  if ((flags & RUN_ACTIVE) == 0 || (partial != 0 && ((flags >> 8) > step || step >= rend))) return;
  // A turn of units that stops the run inside this phase: the heads before
  // the stop's head are whole, the rest is the tail's (k_attention_tail).
  uint32_t last = a.heads - 1;
  if (partial && stop_ph == 9 && step == stop_in) {
    if (h >= stop_row) return;
    last = stop_row - 1;
  }
  const uint32_t npos = pos + 1;
  uint8_t *st = a.states + base;
  const int64_t *q = reinterpret_cast<const int64_t *>(st + off_w2) + (uint64_t)h * hs;
  const uint64_t head_base = ((uint64_t)a.layer * a.kv_heads + kvh) * cachepos * hs;
  const int32_t *K = reinterpret_cast<const int32_t *>(st + off_keys) + head_base;
  const int32_t *V = reinterpret_cast<const int32_t *>(st + off_values) + head_base;

  if (pre) {
    if (tid < (int)hs) qs[tid] = qpre;
  } else {
    for (uint32_t i = tid; i < hs; i += blockDim.x) qs[i] = q[i];
  }
  __syncthreads();

  // Batch jb holds positions jb + pg + GP u.  Positions past the end load
  // the last row (a valid address whose line is already near) and count
  // for nothing, so every load is unconditional and the next batch is
  // always in flight while one is summed.
  auto row = [&](uint32_t jb, int u) {
    const uint32_t j = jb + pg + GP * u;
    return j < npos ? j : npos - 1;
  };

  // Stage 0, scores: s_j = (((q . K_j) >> 16) * inv) >> 24.
  int64_t lmax = INT64_MIN;
  const int64_t inv = (int64_t)(uint64_t)a.inv;
  if constexpr (VEC) {
    int64_t qr[4];
    bool fits = true;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      qr[u] = qs[4 * lp + u];
      fits = fits && qr[u] >= INT32_MIN && qr[u] <= INT32_MAX;
    }
    // Queries that fit 32 bits (the usual case) multiply as 32 x 32 -> 64.
    const bool q32 = __syncthreads_and(fits ? 1 : 0) != 0;
    auto scores = [&](auto narrow) {
      auto fetch = [&](v4i (&kv)[U], uint32_t jb) {
#pragma unroll
        for (int u = 0; u < U; u++)
          kv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(K + (uint64_t)row(jb, u) * HS + 4 * lp));
      };
      auto dots = [&](const v4i (&kv)[U], uint32_t jb) {
        int64_t d[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
          if constexpr (decltype(narrow)::value) {
            d[u] = (int64_t)(int32_t)qr[0] * kv[u].x;
            d[u] = wadd(d[u], (int64_t)(int32_t)qr[1] * kv[u].y);
            d[u] = wadd(d[u], (int64_t)(int32_t)qr[2] * kv[u].z);
            d[u] = wadd(d[u], (int64_t)(int32_t)qr[3] * kv[u].w);
          } else {
            d[u] = wmul(qr[0], kv[u].x);
            d[u] = wadd(d[u], wmul(qr[1], kv[u].y));
            d[u] = wadd(d[u], wmul(qr[2], kv[u].z));
            d[u] = wadd(d[u], wmul(qr[3], kv[u].w));
          }
        }
        if constexpr (LPP >= U) {
          // Sum the U partial dots over the LPP lanes of a position while
          // spreading them out: each halving step keeps half of the
          // positions (chosen by one lane bit) and adds the partner's copy,
          // so log2(U) steps leave one position per lane; the remaining
          // lane bits then sum as usual.  Lane lp ends with position
          // u = its bits (LPP/2, LPP/4, ...) read as a binary number.
          int np = U;
#pragma unroll
          for (int o = LPP / 2; np > 1; o >>= 1) {
            const int half = np / 2;
            const bool up = (lp & o) != 0;
#pragma unroll
            for (int i = 0; i < half; i++) {
              const int64_t mine = up ? d[half + i] : d[i];
              const int64_t other = up ? d[i] : d[half + i];
              d[i] = wadd(mine, (int64_t)__shfl_xor((long long)other, o, LPP));
            }
            np = half;
          }
          constexpr int REST = LPP / U;  // lanes still holding parts of one position
#pragma unroll
          for (int o = REST / 2; o > 0; o >>= 1) d[0] = wadd(d[0], (int64_t)__shfl_xor((long long)d[0], o, LPP));
          const uint32_t j = jb + pg + GP * (lp / REST);
          if (lp % REST == 0 && j < npos) {
            const int64_t sj = wmul(d[0] >> 16, inv) >> 24;
            sc[j] = sj;
            lmax = sj > lmax ? sj : lmax;
          }
        } else {
#pragma unroll
          for (int u = 0; u < U; u++) {
            int64_t dot = d[u];
#pragma unroll
            for (int o = LPP / 2; o > 0; o >>= 1) dot = wadd(dot, (int64_t)__shfl_xor((long long)dot, o, LPP));
            const uint32_t j = jb + pg + GP * u;
            if (lp == 0 && j < npos) {
              const int64_t sj = wmul(dot >> 16, inv) >> 24;
              sc[j] = sj;
              lmax = sj > lmax ? sj : lmax;
            }
          }
        }
      };
      // The scheduling fences keep each batch's loads in program order, so
      // summing one batch waits only for that batch.
      v4i B[U];
      if (!pre) fetch(A, 0);
      for (uint32_t jb = 0; jb < npos; jb += 2 * GP * U) {
        __builtin_amdgcn_sched_barrier(0);
        fetch(B, jb + GP * U);
        __builtin_amdgcn_sched_barrier(0);
        dots(A, jb);
        __builtin_amdgcn_sched_barrier(0);
        fetch(A, jb + 2 * GP * U);
        __builtin_amdgcn_sched_barrier(0);
        dots(B, jb + GP * U);
      }
    };
    if (q32) scores(std::true_type{});
    else scores(std::false_type{});
  } else {
    for (uint32_t j = grp; j < npos; j += 16) {
      const int32_t *kr = K + (uint64_t)j * hs;
      int64_t dot = 0;
      for (uint32_t e = l16; e < hs; e += 16) dot = wadd(dot, wmul(qs[e], kr[e]));
      for (int o = 8; o > 0; o >>= 1) dot = wadd(dot, (int64_t)__shfl_xor((long long)dot, o, 16));
      if (l16 == 0) {
        const int64_t s = wmul(dot >> 16, inv) >> 24;
        sc[j] = s;
        lmax = s > lmax ? s : lmax;
      }
    }
  }
  const int64_t m = block_max_i64(lmax, reinterpret_cast<int64_t *>(scratch));

  // Stage 1, exponentials: EXP[min((m - s) >> 8, 4096)], and their sum.
  uint64_t lsum = 0;
  for (uint32_t j = tid; j < npos; j += blockDim.x) {
    const uint64_t d = (uint64_t)m - (uint64_t)sc[j];
    const uint64_t idx = d >> 8;
    const uint32_t e = a.exp_tab[idx > 4096 ? 4096 : idx];  // 16 KB table, hot in L2
    sc[j] = e;
    lsum += e;
  }
  const uint64_t S = block_sum_u64(lsum, scratch);

  // Stage 2, normalization: (e << 24) / S, at most 2^24.  The state keeps
  // the last head's probabilities, largest score and sum.
  int64_t *scores_out = h == last ? reinterpret_cast<int64_t *>(st + rd.off_scores) : nullptr;
  if (scores_out && tid == 0) {
    *reinterpret_cast<int64_t *>(st + ST_MAXSCORE) = m;
    *reinterpret_cast<uint64_t *>(st + ST_SUM) = S;
  }
  // The division by S through its reciprocal floor(2^64 / S): the high half
  // of n times it is the quotient or one less, and one remainder test fixes
  // it (Granlund and Montgomery, 1994).
  const uint64_t Sm = S > 1 ? recip64(S) : 0;
  for (uint32_t j = tid; j < npos; j += blockDim.x) {
    const uint64_t n = (uint64_t)sc[j] << 24;
    uint64_t q = n;
    if (S > 1) {
      q = __umul64hi(n, Sm);
      if (n - q * S >= S) q++;
    }
    const int64_t p = (int64_t)q;
    sc[j] = p;
    if (scores_out) scores_out[j] = p;
  }
  __syncthreads();

  // Stage 3, weighted values: o_i = (sum_j p_j * V_j,i) >> 24.
  int64_t *w3 = reinterpret_cast<int64_t *>(st + rd.off_w3) + (uint64_t)h * hs;
  if constexpr (VEC) {
    int64_t acc[4] = {0, 0, 0, 0};
    auto fetch = [&](v4i (&vv)[U], uint32_t jb) {
#pragma unroll
      for (int u = 0; u < U; u++)
        vv[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(V + (uint64_t)row(jb, u) * HS + 4 * lp));
    };
    auto weigh = [&](const v4i (&vv)[U], uint32_t jb) {
#pragma unroll
      for (int u = 0; u < U; u++) {
        // a position past the end weighs nothing (read without a branch)
        const int32_t p = (int32_t)sc[row(jb, u)] & -(int32_t)(jb + pg + GP * u < npos);
        acc[0] = wadd(acc[0], (int64_t)p * vv[u].x);
        acc[1] = wadd(acc[1], (int64_t)p * vv[u].y);
        acc[2] = wadd(acc[2], (int64_t)p * vv[u].z);
        acc[3] = wadd(acc[3], (int64_t)p * vv[u].w);
      }
    };
    v4i A[U], B[U];
    fetch(A, 0);
    for (uint32_t jb = 0; jb < npos; jb += 2 * GP * U) {
      __builtin_amdgcn_sched_barrier(0);
      fetch(B, jb + GP * U);
      __builtin_amdgcn_sched_barrier(0);
      weigh(A, jb);
      __builtin_amdgcn_sched_barrier(0);
      fetch(A, jb + 2 * GP * U);
      __builtin_amdgcn_sched_barrier(0);
      weigh(B, jb + GP * U);
    }
#pragma unroll
    for (int u = 0; u < 4; u++) red[pg * HS + 4 * lp + u] = acc[u];
    __syncthreads();
    for (uint32_t e = tid; e < HS; e += blockDim.x) {
      int64_t o = 0;
      for (int g = 0; g < GP; g++) o = wadd(o, red[g * HS + e]);
      o >>= 24;
      w3[e] = o;
      put_digits(a.planes, a.bp, a.kp, b, h * HS + e, o, a.oflag);
    }
  } else {
    const uint32_t groups = blockDim.x / hs;  // hs <= 256
    const uint32_t g = tid / hs, e = tid % hs;
    int64_t acc = 0;
    if (g < groups)
      for (uint32_t j = g; j < npos; j += groups) acc = wadd(acc, (int64_t)(int32_t)sc[j] * V[(uint64_t)j * hs + e]);
    if (g < groups) red[g * hs + e] = acc;
    __syncthreads();
    if (tid < (int)hs) {
      int64_t o = 0;
      for (uint32_t gg = 0; gg < groups; gg++) o = wadd(o, red[gg * hs + tid]);
      o >>= 24;
      w3[tid] = o;
      put_digits(a.planes, a.bp, a.kp, b, h * hs + tid, o, a.oflag);
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 19 and the end of a position ("Sampling").

__device__ __forceinline__ uint32_t temp_index(uint64_t d, uint32_t t) {
  // floor(d * 2^16 / t) >> 8, capped at 4,096: at or above the cap exactly
  // when d >= 16 t; below it d < 2^24 and the quotient fits 64 bits.
  if (d >= 16ull * t) return 4096u;
  const uint64_t i = ((d << 16) / t) >> 8;
  return i > 4096 ? 4096u : (uint32_t)i;
}

// The head a turn of units stops inside ("Attention, stage by stage", unit
// by unit as "The resumable state" counts them): its stages up to the
// stop's stage and index, in the state's scores buffer, with the largest
// score and the sum of exponentials in the header as far as the stages
// reached.  One workgroup of 256 per run; runs without such a stop leave.
__global__ __launch_bounds__(256) void k_attention_tail(AttnTailArgs a) {
  __shared__ uint64_t scratch[8];
  const RunDesc &rd = a.runs[blockIdx.x];
  if (!(rd.flags & RUN_ACTIVE) || rd.stop_ph != 9 || a.step != rd.stop_in) return;
  const uint32_t h = rd.stop_row, S = rd.stop_stage, I = rd.stop_index;
  const uint32_t npos = rd.pos + 1, hs = a.head, tid = threadIdx.x;
  uint8_t *st = a.states + rd.base;
  const int64_t *q = reinterpret_cast<const int64_t *>(st + rd.off_w2) + (uint64_t)h * hs;
  const uint64_t head_base = ((uint64_t)a.layer * a.kv_heads + h / a.group) * rd.cachepos * hs;
  const int32_t *K = reinterpret_cast<const int32_t *>(st + rd.off_keys) + head_base;
  const int32_t *V = reinterpret_cast<const int32_t *>(st + rd.off_values) + head_base;
  int64_t *sc = reinterpret_cast<int64_t *>(st + rd.off_scores);
  int64_t *out = reinterpret_cast<int64_t *>(st + rd.off_w3) + (uint64_t)h * hs;
  const int64_t inv = (int64_t)(uint64_t)a.inv;
  // stage 0: scores of the positions reached, and their maximum
  const uint32_t n0 = S == 0 ? I : npos;
  int64_t lmax = INT64_MIN;
  for (uint32_t j = tid; j < n0; j += 256) {
    int64_t dot = 0;
    for (uint32_t i = 0; i < hs; i++) dot = wadd(dot, wmul(q[i], (int64_t)K[(uint64_t)j * hs + i]));
    const int64_t s = wmul(dot >> 16, inv) >> 24;
    sc[j] = s;
    lmax = s > lmax ? s : lmax;
  }
  const int64_t m = block_max_i64(lmax, reinterpret_cast<int64_t *>(scratch));
  if (n0 > 0 && tid == 0) *reinterpret_cast<int64_t *>(st + ST_MAXSCORE) = m;
  if (S == 0) return;
  __threadfence_block();
  __syncthreads();
  // stage 1: exponentials and their sum (started from zero by its first unit)
  const uint32_t n1 = S == 1 ? I : npos;
  uint64_t lsum = 0;
  for (uint32_t j = tid; j < n1; j += 256) {
    const uint64_t d = (uint64_t)m - (uint64_t)sc[j];
    const uint64_t idx = d >> 8;
    const uint32_t e = a.exp_tab[idx > 4096 ? 4096 : idx];
    sc[j] = e;
    lsum += e;
  }
  const uint64_t sum = block_sum_u64(lsum, scratch);
  if (n1 > 0 && tid == 0) *reinterpret_cast<uint64_t *>(st + ST_SUM) = sum;
  if (S == 1) return;
  __threadfence_block();
  __syncthreads();
  // stage 2: normalization
  const uint32_t n2 = S == 2 ? I : npos;
  for (uint32_t j = tid; j < n2; j += 256) sc[j] = (int64_t)(((uint64_t)sc[j] << 24) / sum);
  if (S == 2) return;
  __threadfence_block();
  __syncthreads();
  // stage 3: the output elements reached
  for (uint32_t e = tid; e < I; e += 256) {
    int64_t acc = 0;
    for (uint32_t j = 0; j < npos; j++) acc = wadd(acc, wmul(sc[j], (int64_t)V[(uint64_t)j * hs + e]));
    out[e] = acc >> 24;
  }
}

// A cursor between two phases: no row, attention stage or index, or
// sampling pass of its own.
__device__ __forceinline__ void clear_sub_phase(uint8_t *st) {
  *reinterpret_cast<uint32_t *>(st + ST_ROW) = 0u;
  *reinterpret_cast<uint32_t *>(st + ST_PASS) = 0u;
  *reinterpret_cast<uint32_t *>(st + ST_STAGE) = 0u;
  *reinterpret_cast<uint32_t *>(st + ST_INDEX) = 0u;
}

__global__ __launch_bounds__(256) void k_sample(SampleArgs a) {
  __shared__ int64_t best_v[256];
  __shared__ uint32_t best_i[256];
  __shared__ uint64_t part[256];
  __shared__ uint64_t bcast[4];
  const uint32_t b = blockIdx.x;
  RunDesc &rd = a.runs[b];
  if (!(rd.flags & RUN_ACTIVE)) return;
  uint8_t *st = a.states + rd.base;
  const int tid = threadIdx.x;
  if (rd.errkey != 0xFFFFFFFFu) {
    // The run froze in this position: error 8 at the failing phase and layer.
    if (tid == 0) {
      *reinterpret_cast<uint32_t *>(st + ST_ERROR) = FPI8_ARITHMETIC;
      *reinterpret_cast<uint32_t *>(st + ST_PHASE) = rd.errkey & 0xFFu;
      *reinterpret_cast<uint32_t *>(st + ST_LAYER) = rd.errkey >> 8;
      a.run_err[b] = FPI8_ARITHMETIC;
    }
    return;
  }
  // The cursor's sampling pass and entry as the position started (a turn
  // may resume inside sampling).
  const uint32_t pass_start = *reinterpret_cast<const uint32_t *>(st + ST_PASS);
  const uint32_t row_start = *reinterpret_cast<const uint32_t *>(st + ST_ROW);
  const uint64_t budget = rd.budget;  // read once: thread 0 updates it below
  // A turn of units that stops the run in this position (rd.stop_*).
  const bool ustop = a.partial && rd.stop_ph != 0;
  auto write_stop = [&]() {
    *reinterpret_cast<uint32_t *>(st + ST_PHASE) = rd.stop_ph;
    *reinterpret_cast<uint32_t *>(st + ST_LAYER) = rd.stop_layer;
    *reinterpret_cast<uint32_t *>(st + ST_ROW) = rd.stop_row;
    *reinterpret_cast<uint32_t *>(st + ST_STAGE) = rd.stop_stage;
    *reinterpret_cast<uint32_t *>(st + ST_INDEX) = rd.stop_index;
    *reinterpret_cast<uint32_t *>(st + ST_PASS) = rd.stop_pass;
  };
  if (ustop && rd.stop_ph != 19) {
    __syncthreads();  // every thread has read the cursor above
    if (tid == 0) write_stop();
    return;
  }
  if (!ustop && a.partial && rd.end <= a.step) {
    // The turn stops the run before step rd.end: its cursor names the
    // phase that step starts (a boundary between two phases).
    if (tid == 0) {
      const uint32_t f = 1 + 7 * a.layers, end = rd.end;
      uint32_t phase = 4, layer = 0;
      if (end >= f) {
        phase = 17 + (end - f);
      } else if (end > 1) {
        // after the first normalization, q/k/v, attention, (the output rows
        // stop nowhere), the second normalization, gate/up, down
        const uint32_t r = (end - 2) % 7;
        layer = (end - 2) / 7;
        phase = r == 0 ? 5 : r == 1 ? 9 : r == 2 ? 10 : r == 4 ? 12 : r == 5 ? 15 : 4;
        if (r == 6) layer++;
      }
      *reinterpret_cast<uint32_t *>(st + ST_PHASE) = phase;
      *reinterpret_cast<uint32_t *>(st + ST_LAYER) = layer;
      clear_sub_phase(st);
    }
    return;
  }
  const uint32_t pos = rd.pos;
  uint32_t token = 0;
  bool complete = false;
  if (rd.flags & RUN_GEN) {
    const int64_t *lgt = reinterpret_cast<const int64_t *>(st + rd.off_logits);
    const uint32_t V = a.vocab;
    const uint32_t chunk = (V + blockDim.x - 1) / blockDim.x;
    const uint32_t c0 = tid * chunk, c1 = min(V, c0 + chunk);
    // a stop inside the maximum pass: the entries before its row
    const uint32_t lim0 = (ustop && rd.stop_pass == 0) ? rd.stop_row : V;
    // Maximum pass: the largest logit, the lowest index on a tie.  Each
    // thread strides over the entries (a wave reads 64 consecutive words),
    // U loads in flight; a thread meets its entries in increasing order, so
    // its first maximum is its lowest-index one, and the reduction below
    // keeps the lowest index among equal maxima.
    constexpr int U = 8;
    const uint32_t lim = min(V, lim0);
    int64_t bv = INT64_MIN;
    uint32_t bi = 0xFFFFFFFFu;
    for (uint32_t i0 = tid; i0 < lim; i0 += U * 256) {
      int64_t x[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const uint32_t i = i0 + u * 256;
        x[u] = i < lim ? lgt[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; u++) {
        const uint32_t i = i0 + u * 256;
        if (i < lim && (bi == 0xFFFFFFFFu || x[u] > bv)) { bv = x[u]; bi = i; }
      }
    }
    best_v[tid] = bv;
    best_i[tid] = bi;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) {
        const int64_t ov = best_v[tid + s];
        const uint32_t oi = best_i[tid + s];
        if (oi != 0xFFFFFFFFu &&
            (best_i[tid] == 0xFFFFFFFFu || ov > best_v[tid] || (ov == best_v[tid] && oi < best_i[tid]))) {
          best_v[tid] = ov;
          best_i[tid] = oi;
        }
      }
      __syncthreads();
    }
    const int64_t m = best_v[0];
    token = best_i[0];
    const uint32_t T = rd.temp;
    if (ustop && rd.stop_pass == 0) {
      // stopped inside the maximum pass
      if (tid == 0) {
        if (lim0 > 0) {
          *reinterpret_cast<int64_t *>(st + ST_MAXSCORE) = m;
          *reinterpret_cast<uint32_t *>(st + ST_CHOSEN) = token;
        }
        write_stop();
      }
      return;
    }
    if (T != 0) {
      // Sum pass over each thread's slice, then the draw and the walk.
      const uint32_t lim1 = ustop ? rd.stop_row : V;  // a stop inside the sum pass
      // Each thread sums its own contiguous slice (the walk below needs the
      // slices' sums in index order), U loads in flight.
      const uint32_t e1 = min(c1, lim1);
      uint64_t s = 0;
      for (uint32_t i0 = c0; i0 < e1; i0 += U) {
        int64_t x[U];
#pragma unroll
        for (int u = 0; u < U; u++) x[u] = i0 + u < e1 ? lgt[i0 + u] : 0;
#pragma unroll
        for (int u = 0; u < U; u++)
          if (i0 + u < e1) s += a.exp_tab[temp_index((uint64_t)m - (uint64_t)x[u], T)];
      }
      part[tid] = s;
      __syncthreads();
      if (ustop) {
        // stopped inside the sum pass (the generator has not advanced)
        if (tid == 0) {
          uint64_t total = 0;
          for (int i = 0; i < 256; i++) total += part[i];
          *reinterpret_cast<int64_t *>(st + ST_MAXSCORE) = m;
          *reinterpret_cast<uint32_t *>(st + ST_CHOSEN) = token;
          if (lim1 > 0) *reinterpret_cast<uint64_t *>(st + ST_SUM) = total;
          write_stop();
        }
        return;
      }
      if (tid == 0) {
        uint64_t total = 0;
        for (int i = 0; i < 256; i++) total += part[i];
        // The generator advances when the sum pass ends; a state stopped in
        // the draw pass has advanced it already.
        uint64_t *gen = reinterpret_cast<uint64_t *>(st + ST_GENERATOR);
        uint64_t x = *gen;
        if (pass_start != 2) {
          x ^= x >> 12;
          x ^= x << 25;
          x ^= x >> 27;
          *gen = x;
        }
        uint64_t r = (x * 0x2545F4914F6CDD1Dull) % total;
        bcast[1] = r;  // the draw, for a stop inside the walk
        uint32_t c = 0;
        while (c < 255 && r >= part[c]) { r -= part[c]; c++; }
        bcast[0] = c;
        bcast[2] = r;
        *reinterpret_cast<uint64_t *>(st + ST_SUM) = total;
      }
      __syncthreads();
      if ((uint64_t)tid == bcast[0]) {
        uint64_t r = bcast[2];
        for (uint32_t i = c0; i < c1; i++) {
          const uint64_t e = a.exp_tab[temp_index((uint64_t)m - (uint64_t)lgt[i], T)];
          if (r < e) { best_i[0] = i; bcast[3] = r; break; }
          r -= e;
        }
      }
      __syncthreads();
      const uint32_t drawn = best_i[0];
      // A turn of units walks at most rd.budget entries of the draw pass
      // from where this position's walk started.
      const uint32_t walk0 = pass_start == 2 ? row_start : 0u;
      if (a.partial && rd.units && (uint64_t)(drawn + 1 - walk0) > budget) {
        const uint32_t R = walk0 + (uint32_t)budget;  // entries walked by the stop
        uint64_t w = 0;
        for (uint32_t i = c0; i < min(c1, R); i++) w += a.exp_tab[temp_index((uint64_t)m - (uint64_t)lgt[i], T)];
        __syncthreads();
        part[tid] = w;
        __syncthreads();
        if (tid == 0) {
          uint64_t walked = 0;
          for (int i = 0; i < 256; i++) walked += part[i];
          *reinterpret_cast<int64_t *>(st + ST_MAXSCORE) = m;
          *reinterpret_cast<uint32_t *>(st + ST_CHOSEN) = token;
          *reinterpret_cast<uint64_t *>(st + ST_REMAINDER) = bcast[1] - walked;
          *reinterpret_cast<uint32_t *>(st + ST_PHASE) = 19u;
          *reinterpret_cast<uint32_t *>(st + ST_LAYER) = 0u;
          *reinterpret_cast<uint32_t *>(st + ST_ROW) = R;
          *reinterpret_cast<uint32_t *>(st + ST_STAGE) = 0u;
          *reinterpret_cast<uint32_t *>(st + ST_INDEX) = 0u;
          *reinterpret_cast<uint32_t *>(st + ST_PASS) = 2u;
          rd.halted = 1;
        }
        return;
      }
      if (tid == 0 && a.partial && rd.units) rd.budget = budget - (drawn + 1 - walk0);
      token = drawn;
      if (tid == 0) *reinterpret_cast<uint64_t *>(st + ST_REMAINDER) = bcast[3];
    }
    if (tid == 0) {
      // what the passes leave in the header: the largest logit, the chosen
      // entry (and above, the sum and what was left of the draw)
      *reinterpret_cast<int64_t *>(st + ST_MAXSCORE) = m;
      *reinterpret_cast<uint32_t *>(st + ST_CHOSEN) = token;
    }
    if (tid == 0) {
      uint32_t *gen_count = reinterpret_cast<uint32_t *>(st + ST_GENERATED);
      uint32_t *out = reinterpret_cast<uint32_t *>(st + rd.off_out);
      const uint32_t g = *gen_count;
      out[g] = token;
      *gen_count = g + 1;
      complete = token == 1 || token == 2 || g + 1 == rd.max_tokens;
    }
  } else if (tid == 0) {
    token = reinterpret_cast<const uint32_t *>(st + rd.off_ids)[pos + 1];
  }
  if (tid == 0) {
    *reinterpret_cast<uint32_t *>(st + ST_TOKEN) = token;
    *reinterpret_cast<uint32_t *>(st + ST_POSITION) = pos + 1;
    *reinterpret_cast<uint32_t *>(st + ST_PHASE) = complete ? 20u : 3u;
    *reinterpret_cast<uint32_t *>(st + ST_LAYER) = 0u;
    clear_sub_phase(st);
  }
}

// ---------------------------------------------------------------------------
// Launchers

static inline int ok(hipError_t e) { return e == hipSuccess ? 0 : FPI8_ERR_HIP; }

int launch_turn_start(uint8_t *states, RunDesc *runs, uint32_t n_runs, void *stream) {
  if (!n_runs) return 0;
  hipLaunchKernelGGL(k_turn_start, dim3((n_runs + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                     states, runs, n_runs);
  return ok(hipGetLastError());
}

int launch_begin(const BeginArgs &a, void *stream) {
  const uint32_t n = a.n_runs > a.n_oflags ? a.n_runs : a.n_oflags;
  hipLaunchKernelGGL(k_begin, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, a);
  return ok(hipGetLastError());
}

int launch_embed(const EmbedArgs &a, void *stream) {
  hipLaunchKernelGGL(k_embed, dim3((a.dim + 255) / 256, a.n_runs), dim3(256), 0,
                     (hipStream_t)stream, a);
  return ok(hipGetLastError());
}

int launch_norm(const NormArgs &a, void *stream) {
  // Several workgroups per run share the stores when the vector fits one
  // workgroup's registers (8 of them per thread): eight of 256 threads up
  // to 2048 elements, four of 512 up to 4096 (measured: eight of 512 were
  // slower there); otherwise one workgroup.
  const uint32_t threads = a.dim <= 256 * 8 ? 256 : 512;
  const uint32_t parts = a.dim <= 256 * 8 ? 8 : a.dim <= 512 * 8 ? 4 : 1;
  hipLaunchKernelGGL(k_norm, dim3(a.n_runs, parts), dim3(threads), 0, (hipStream_t)stream, a);
  return ok(hipGetLastError());
}

// The launch shapes the planner may pick: 16 * MT rows and 16 * BT runs per
// workgroup of four waves.
template <int EPI, int MT, int BT>
static int rows_launch(const RowsArgs &a, hipStream_t s) {
  const uint32_t groups = (a.ntiles + 7) / 8;
  const dim3 grid(groups * 8 * a.chunks), block(256);
  hipLaunchKernelGGL((k_rows<EPI, MT, BT>), grid, block, 0, s, a);
  return ok(hipGetLastError());
}

template <int EPI, int MT, int BT, int W = 4, int CD = 2, int PP = 0>
static int rows_launch_shared(const RowsArgs &a, hipStream_t s) {
  const uint32_t groups = (a.ntiles + 7) / 8;
  const dim3 grid(groups * 8 * a.chunks), block(64 * W);
  hipLaunchKernelGGL((k_rows_shared<EPI, MT, BT, W, CD, PP>), grid, block, 0, s, a);
  return ok(hipGetLastError());
}

// Kinds 2 and 3: every wave owns rows, one block of digits per stage, and
// the waves per workgroup follow the runs: 3 for 16 runs, 6 for 32, 12 for
// 64 (one digit fragment per wave and stage); P = 3 stages in flight (kind
// 2) or 7 (kind 3).
template <int EPI, int MT, int BT, int P>
static int rows_launch_waves(const RowsArgs &a, hipStream_t s) {
  constexpr int W = 3 * BT;
  if (a.wave_rows != (uint32_t)W) return FPI8_ERR_ARGUMENT;
  return rows_launch_shared<EPI, MT, BT, W, 1, P>(a, s);
}

template <int EPI>
static int rows_shape(int kind, int mt, int bt, const RowsArgs &a, hipStream_t s) {
  const int key = kind * 100 + mt * 10 + bt;
  if constexpr (EPI != EPI_GATEUP) {
    switch (key) {
      case 11: return rows_launch<EPI, 1, 1>(a, s);
      case 12: return rows_launch<EPI, 1, 2>(a, s);
      case 14: return rows_launch<EPI, 1, 4>(a, s);
      case 22: return rows_launch<EPI, 2, 2>(a, s);
      case 24: return rows_launch<EPI, 2, 4>(a, s);
      case 41: return rows_launch<EPI, 4, 1>(a, s);
      case 42: return rows_launch<EPI, 4, 2>(a, s);
      case 112: return rows_launch_shared<EPI, 1, 2>(a, s);
      case 114: return rows_launch_shared<EPI, 1, 4>(a, s);
      case 122: return rows_launch_shared<EPI, 2, 2>(a, s);
      case 124: return rows_launch_shared<EPI, 2, 4>(a, s);
      case 211: return rows_launch_waves<EPI, 1, 1, 3>(a, s);
      case 221: return rows_launch_waves<EPI, 2, 1, 3>(a, s);
      case 241: return rows_launch_waves<EPI, 4, 1, 3>(a, s);
      case 212: return rows_launch_waves<EPI, 1, 2, 3>(a, s);
      case 222: return rows_launch_waves<EPI, 2, 2, 3>(a, s);
      case 214: return rows_launch_waves<EPI, 1, 4, 3>(a, s);
      case 311: return rows_launch_waves<EPI, 1, 1, 7>(a, s);
      case 312: return rows_launch_waves<EPI, 1, 2, 7>(a, s);
    }
  } else {
    switch (key) {
      case 22: return rows_launch<EPI, 2, 2>(a, s);
      case 24: return rows_launch<EPI, 2, 4>(a, s);
      case 42: return rows_launch<EPI, 4, 2>(a, s);
      case 122: return rows_launch_shared<EPI, 2, 2>(a, s);
      case 124: return rows_launch_shared<EPI, 2, 4>(a, s);
      case 221: return rows_launch_waves<EPI, 2, 1, 3>(a, s);
      case 241: return rows_launch_waves<EPI, 4, 1, 3>(a, s);
      case 222: return rows_launch_waves<EPI, 2, 2, 3>(a, s);
      case 321: return rows_launch_waves<EPI, 2, 1, 7>(a, s);
    }
  }
  return FPI8_ERR_ARGUMENT;
}

int launch_rows_raw(int mt, const RowsArgs &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.ntiles == 0 || a.chunks == 0) return 0;
  if (a.chunks != 1 || a.n_runs > 2) return FPI8_ERR_ARGUMENT;
  const uint32_t per = (a.kblocks + 3) / 4;
  if ((uint64_t)3 * a.n_runs * per * 64 > XR_CAP) return FPI8_ERR_ARGUMENT;
  const dim3 grid((a.ntiles + 7) / 8 * 8), block(256);
  switch (mt) {
    case 1: hipLaunchKernelGGL((k_rows<EPI_RAW, 1, 1, true>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_rows<EPI_RAW, 4, 1, true>), grid, block, 0, s, a); break;
    default: return FPI8_ERR_ARGUMENT;
  }
  return ok(hipGetLastError());
}

// The one shape of a position where some run starts or stops between two
// phases (kind 0, 32 rows, 32 runs).
template <int EPI>
static int rows_launch_partial(const RowsArgs &a, hipStream_t s) {
  const uint32_t groups = (a.ntiles + 7) / 8;
  const dim3 grid(groups * 8 * a.chunks), block(256);
  hipLaunchKernelGGL((k_rows<EPI, 2, 2, false, true>), grid, block, 0, s, a);
  return ok(hipGetLastError());
}

int launch_rows(int epi, int kind, int mt, int bt, const RowsArgs &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  if (a.ntiles == 0 || a.chunks == 0) return 0;
  if (a.partial) {
    if (kind != 0 || mt != 2 || bt != 2) return FPI8_ERR_ARGUMENT;
    switch (epi) {
      case EPI_QKV: return rows_launch_partial<EPI_QKV>(a, s);
      case EPI_RESID: return rows_launch_partial<EPI_RESID>(a, s);
      case EPI_DOWN: return rows_launch_partial<EPI_DOWN>(a, s);
      case EPI_CLS: return rows_launch_partial<EPI_CLS>(a, s);
      case EPI_GATEUP: return rows_launch_partial<EPI_GATEUP>(a, s);
    }
    return FPI8_ERR_ARGUMENT;
  }
  switch (epi) {
    case EPI_RAW: return rows_shape<EPI_RAW>(kind, mt, bt, a, s);
    case EPI_QKV: return rows_shape<EPI_QKV>(kind, mt, bt, a, s);
    case EPI_RESID: return rows_shape<EPI_RESID>(kind, mt, bt, a, s);
    case EPI_DOWN: return rows_shape<EPI_DOWN>(kind, mt, bt, a, s);
    case EPI_CLS: return rows_shape<EPI_CLS>(kind, mt, bt, a, s);
    case EPI_GATEUP: return rows_shape<EPI_GATEUP>(kind, mt, bt, a, s);
  }
  return FPI8_ERR_ARGUMENT;
}

size_t attention_lds_bytes(uint32_t max_npos, uint32_t head) {
  // partial sums of stage 3: (256 / (head / 4)) position groups x head
  const size_t red = (head % 4 == 0 && (head & (head - 1)) == 0) ? 1024ull : 256ull;
  return 8ull * max_npos + 8ull * red;
}

static bool pow2_head(uint32_t h) { return h >= 4 && h <= 256 && (h & (h - 1)) == 0; }

int kernels_init(uint32_t max_npos, uint32_t head) {
  const int bytes = (int)attention_lds_bytes(max_npos, head);
  hipError_t e = hipSuccess;
  switch (pow2_head(head) ? head : 0) {
    case 4: e = hipFuncSetAttribute((const void *)k_attention<4>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    case 8: e = hipFuncSetAttribute((const void *)k_attention<8>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    case 16: e = hipFuncSetAttribute((const void *)k_attention<16>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    case 32: e = hipFuncSetAttribute((const void *)k_attention<32>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    case 64: e = hipFuncSetAttribute((const void *)k_attention<64>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    case 128: e = hipFuncSetAttribute((const void *)k_attention<128>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    case 256: e = hipFuncSetAttribute((const void *)k_attention<256>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
    default: e = hipFuncSetAttribute((const void *)k_attention<0>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes); break;
  }
  return ok(e);
}

uint64_t packed_bytes(uint32_t rows, uint32_t cols) {
  const uint64_t kbp = ((cols + 63) / 64 + 1) / 2 * 2;
  return (uint64_t)((rows + 15) / 16) * kbp * 1024;
}

int launch_pack(const uint8_t *W, uint32_t rows, uint32_t cols, uint8_t *P, void *stream) {
  const uint32_t kbp = (uint32_t)(((cols + 63) / 64 + 1) / 2 * 2);
  const uint64_t pieces = packed_bytes(rows, cols) / 16;
  hipLaunchKernelGGL(k_pack, dim3((uint32_t)((pieces + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     W, rows, cols, kbp, P, pieces);
  return ok(hipGetLastError());
}

int launch_attention_tail(const AttnTailArgs &a, void *stream) {
  if (!a.n_runs) return 0;
  hipLaunchKernelGGL(k_attention_tail, dim3(a.n_runs), dim3(256), 0, (hipStream_t)stream, a);
  return ok(hipGetLastError());
}

int launch_attention(const AttnArgs &a, void *stream) {
  const dim3 grid(a.heads, a.n_runs), block(256);
  const size_t lds = attention_lds_bytes(a.max_npos, a.head);
  hipStream_t s = (hipStream_t)stream;
  switch (pow2_head(a.head) ? a.head : 0) {
    case 4: hipLaunchKernelGGL(k_attention<4>, grid, block, lds, s, a); break;
    case 8: hipLaunchKernelGGL(k_attention<8>, grid, block, lds, s, a); break;
    case 16: hipLaunchKernelGGL(k_attention<16>, grid, block, lds, s, a); break;
    case 32: hipLaunchKernelGGL(k_attention<32>, grid, block, lds, s, a); break;
    case 64: hipLaunchKernelGGL(k_attention<64>, grid, block, lds, s, a); break;
    case 128: hipLaunchKernelGGL(k_attention<128>, grid, block, lds, s, a); break;
    case 256: hipLaunchKernelGGL(k_attention<256>, grid, block, lds, s, a); break;
    default: hipLaunchKernelGGL(k_attention<0>, grid, block, lds, s, a); break;
  }
  return ok(hipGetLastError());
}

int launch_sample(const SampleArgs &a, void *stream) {
  hipLaunchKernelGGL(k_sample, dim3(a.n_runs), dim3(256), 0, (hipStream_t)stream, a);
  return ok(hipGetLastError());
}


int launch_digits_raw(const int64_t *x, uint32_t n_runs, uint32_t cols, int8_t *planes,
                      uint32_t kp, uint32_t bp, uint32_t compact, uint32_t *oflag, uint32_t seq,
                      void *stream) {
  hipLaunchKernelGGL(k_digits_raw, dim3((cols + 255) / 256, n_runs), dim3(256), 0, (hipStream_t)stream,
                     x, n_runs, cols, planes, kp, bp, compact, oflag, seq);
  return ok(hipGetLastError());
}

}  // namespace fpi8
