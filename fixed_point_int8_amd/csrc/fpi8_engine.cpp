// fpi8_engine.cpp - the GPU engine of libfpi8: binds an artifact in device
// memory, owns the workspace, and runs turns by launching the kernels of
// fpi8_kernels.hip one position at a time for a whole batch of runs.
#include <hip/hip_runtime.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <vector>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

using namespace fpi8;

namespace {

constexpr int kTimingClasses = 5;
enum { T_ROWS = 0, T_ATTN = 1, T_NORM = 2, T_SAMPLE = 3, T_EMBED = 4 };

struct Mat {
  const uint8_t *W = nullptr;
  const uint8_t *P = nullptr;  // packed tiles (engine workspace), all but the embedding
  const uint32_t *S = nullptr;
  uint32_t rows = 0, cols = 0;
  bool vec = false;
};

struct Timer {
  bool on = false;
  std::vector<hipEvent_t> starts, stops;
  size_t used = 0;
};

inline uint32_t round_up(uint32_t v, uint32_t m) { return (v + m - 1) / m * m; }

}  // namespace

struct fpi8_engine {
  Model model;
  Cfg c;
  const uint8_t *d_blob = nullptr;
  uint64_t blob_len = 0;
  uint32_t max_runs = 0, bp = 0, kp = 0, max_npos = 0;
  const uint32_t *exp_tab = nullptr;
  const int32_t *silu = nullptr, *cos_t = nullptr, *sin_t = nullptr, *norm = nullptr;
  std::vector<Mat> mats;  // [0] embedding, [1 + 7l + kind - 1], [1 + 7L] classifier
  // device workspace
  RunDesc *d_runs = nullptr;
  uint8_t *d_packed = nullptr;  // every matrix but the embedding, in MFMA operand tiles
  int8_t *d_planes0 = nullptr, *d_planes1 = nullptr;  // per run group: [2][3][bp][kp]
  uint32_t *d_oflags = nullptr;                        // per run group: [2][n_oflags]
  uint32_t n_oflags = 0;
  int32_t *d_run_err = nullptr;
  // pinned host buffers
  RunDesc *h_runs = nullptr;
  uint8_t *h_headers = nullptr;
  int32_t *h_err = nullptr;
  Timer timers[kTimingClasses];
  // One position's launches recorded as a graph on a stream of the
  // engine's own (capture runs nothing) and replayed on the caller's
  // stream; valid for one (state arena, run count).
  hipStream_t cap_stream = nullptr;
  hipGraphExec_t graph = nullptr;
  uint8_t *graph_states = nullptr;
  uint32_t graph_runs = 0;
  uint32_t graph_cap = 0;
  uint32_t score_cap = 0;  // attention's LDS score slots for the current turn
  int row_kind = 0;  // 0 planner's choice, 1 to 7 restrict it (fpi8_engine_set_row_kernel)
  // Runs split into two groups advanced on two streams, so one group's
  // row kernels overlap the other's attention (2); one stream (0, 1).
  // Measured on the 7B-shaped decode at 64 runs, two groups are slower:
  // the row kernels at 32 runs read every weight twice.
  int streams = 0;
  bool use_graph = true;  // replay a recorded position (fpi8_engine_set_graph)
  uint32_t graph_groups = 0;
  hipStream_t side_stream = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  // The arena bound for queued turns (fpi8_turn_bind / fpi8_turn_async):
  // its run descriptors are on the device; `left` bounds the positions any
  // run still has; `resume`: some run stood inside a position at the bind.
  uint8_t *bound_states = nullptr;
  uint32_t bound_runs = 0, bound_left = 0, bound_resume = 0;
  // The current turn's layout when every run of the batch is a valid state
  // with the same buffer offsets and cache length (uni.on): the
  // normalization and attention then read their inputs before the run
  // descriptors arrive.  Part of what a recorded graph is valid for.
  struct Uniform {
    bool on = false;
    uint64_t stride = 0, off_x = 0, off_w2 = 0, off_keys = 0, off_values = 0;
    uint32_t cachepos = 0;
    bool operator==(const Uniform &o) const {
      return on == o.on && stride == o.stride && off_x == o.off_x && off_w2 == o.off_w2 &&
             off_keys == o.off_keys && off_values == o.off_values && cachepos == o.cachepos;
    }
  } uni, graph_uni;

  const Mat &layer_mat(uint32_t l, uint32_t kind) const { return mats[1 + 7 * l + (kind - M_Q)]; }
};

namespace {

int hip_ok(hipError_t e) { return e == hipSuccess ? 0 : FPI8_ERR_HIP; }

// Brackets a launch with events when its class is being timed.
struct TimedLaunch {
  Timer &t;
  hipStream_t s;
  bool on;
  TimedLaunch(Timer &timer, hipStream_t st) : t(timer), s(st) {
    on = t.on;
    if (!on) return;
    if (t.used == t.starts.size()) {
      // Timing only: no system-scope fence when an event is recorded, so
      // the event pair neither writes back and invalidates the caches around
      // the timed launch nor adds that cost to its interval.
      hipEvent_t a, b;
      (void)hipEventCreateWithFlags(&a, hipEventDisableSystemFence);
      (void)hipEventCreateWithFlags(&b, hipEventDisableSystemFence);
      t.starts.push_back(a);
      t.stops.push_back(b);
    }
    (void)hipEventRecord(t.starts[t.used], s);
  }
  TimedLaunch(fpi8_engine *eng, int c, hipStream_t st) : TimedLaunch(eng->timers[c], st) {}
  ~TimedLaunch() {
    if (!on) return;
    (void)hipEventRecord(t.stops[t.used], s);
    t.used++;
  }
};

int timer_sum(Timer &t, double *total_ms, uint64_t *launches) {
  double sum = 0;
  for (size_t i = 0; i < t.used; i++) {
    if (hipEventSynchronize(t.stops[i]) != hipSuccess) return FPI8_ERR_HIP;
    float ms = 0;
    if (hipEventElapsedTime(&ms, t.starts[i], t.stops[i]) != hipSuccess) return FPI8_ERR_HIP;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = t.used;
  return 0;
}

// Timing of the standalone row's row-kernel launches (measurement only).
Timer g_rows_timer;

// Which arithmetic the standalone streaming row uses: 0 automatic (the
// matrix cores), 1 the matrix cores, 2 the vector ALU where it applies.
std::atomic<int> g_rows_path{0};

// Launch shape of one row-kernel call.  kind 0: 16 * mt rows and 16 * bt
// runs per workgroup of four waves, which split the contraction; kind 1:
// wr * 16 * mt rows (16 * mt for each of wr waves) and 16 * bt runs per
// workgroup of four waves that share their runs' digits through LDS.
struct RowPlan {
  int kind, mt, bt, wr;
  uint32_t chunks, tiles;
};

// Picks the shape with the least estimated time.  Every workgroup streams
// its weight rows and its runs' digits (3 bytes per run and column) through
// L2; the weights come from HBM once, at about 20 GB/s per compute unit, so
// a launch wants a workgroup on each of the 256 compute units.  The rate at
// which one compute unit draws a workgroup's bytes depends on the shape
// (registers left for loads in flight, sums per wave, one workgroup's digits
// serving three or four waves' rows); the figures come from sweeps of every
// shape over the 7B-, 1.1B- and long-context-shaped matrices on MI355X.
// shared_ok: the shared-digit kernel can run (columns a multiple of 128,
// aligned rows); force 1 or 2 restricts the choice to kind 0 or kind 1,
// force 3 to kind 1 with three row-owning waves.
RowPlan plan_rows(uint32_t rows, uint32_t cols, uint32_t n_runs, bool gateup, bool shared_ok,
                  int force) {
  // rate: GB/s one compute unit draws for the shape; occ: workgroups of the
  // shape that fit on one compute unit (registers, LDS).
  // Kind 2 (3 * bt waves, all owning rows, one block per stage): rates from
  // sweeps of the 7B-shaped matrices at 64 runs, taken a little below the
  // slowest matrix's so that the kind wins only where it clearly does.
  struct Cand { int kind, mt, bt, wr; double gbs; int occ; };
  static const Cand plain[] = {{0, 1, 1, 1, 26, 1}, {0, 1, 2, 1, 44, 2}, {0, 1, 4, 1, 46, 1},
                               {0, 2, 2, 1, 37, 1}, {0, 2, 4, 1, 42, 1}, {0, 4, 1, 1, 34, 1},
                               {0, 4, 2, 1, 28, 1},
                               {1, 1, 2, 4, 36, 2}, {1, 1, 4, 4, 30, 1}, {1, 2, 2, 4, 34, 2},
                               {1, 2, 4, 4, 26, 1}, {1, 2, 2, 3, 33, 2}, {1, 2, 4, 3, 24, 1},
                               {2, 1, 1, 3, 42, 1}, {2, 2, 1, 3, 38, 1}, {2, 4, 1, 3, 40, 1},
                               {2, 1, 2, 6, 36, 1}, {2, 2, 2, 6, 40, 1}, {2, 1, 4, 12, 38, 1}};
  static const Cand pairs[] = {{0, 2, 2, 1, 37, 1}, {0, 2, 4, 1, 42, 1}, {0, 4, 2, 1, 28, 1},
                               {1, 2, 2, 4, 34, 2}, {1, 2, 4, 4, 26, 1}, {1, 2, 2, 3, 33, 2},
                               {1, 2, 4, 3, 24, 1},
                               {2, 2, 1, 3, 38, 1}, {2, 4, 1, 3, 40, 1}, {2, 2, 2, 6, 40, 1}};
  const Cand *cand = gateup ? pairs : plain;
  const int n = gateup ? 10 : 19;
  const double cus = 256, hbm_cu = 20e9;
  RowPlan best{0, 1, 1, 1, 1, 1};
  double best_t = 1e30;
  for (int i = 0; i < n; i++) {
    const int kind = cand[i].kind;
    if (kind >= 1 && !shared_ok) continue;
    // Kind 2 is chosen by launch (multi_wave_plan) unless forced.
    if (kind == 2 && force < 4) continue;
    if ((force == 1 && kind != 0) || ((force == 2 || force == 3) && shared_ok && kind != 1) ||
        (force == 3 && shared_ok && cand[i].wr != 3) ||
        (force >= 4 && shared_ok && (kind != 2 || cand[i].bt != 1 << (force - 4))))
      continue;
    RowPlan p{kind, cand[i].mt, cand[i].bt, cand[i].wr, 0, 0};
    const uint32_t bc = 16 * p.bt;
    p.chunks = (n_runs + bc - 1) / bc;
    // 64 rows by 16 runs trades digit loads for weight tiles re-read from
    // L2; measured to pay only when four or more batch chunks share them.
    if (kind == 0 && p.mt == 4 && p.bt == 1 && p.chunks < 4) continue;
    const uint32_t per_tile = 16 * (gateup ? p.mt / 2 : p.mt) * p.wr;
    p.tiles = (rows + per_tile - 1) / per_tile;
    const double wgs = (double)p.tiles * p.chunks;
    const double act = wgs < cus ? wgs : cus;
    // Each 64-column block costs a workgroup one 1 KB load per weight tile
    // and per digit tile, whether or not all its runs exist.  Workgroups run
    // in rounds of 256 * occ; a compute unit holding k of them shares its
    // rate among them.
    const double per_wg = 1024.0 * (p.wr * p.mt + 3 * p.bt) * ((cols + 63) / 64);
    const double rounds = std::ceil(wgs / (cus * cand[i].occ));
    const double per_cu = std::min((double)cand[i].occ, std::ceil(wgs / cus));
    const double t_hbm = (double)rows * cols * (gateup ? 2 : 1) / (act * hbm_cu);
    const double t_l2 = rounds * per_cu * per_wg / (cand[i].gbs * 1e9);
    const double t = std::max(t_hbm, t_l2);
    if (t < best_t * 0.999) { best_t = t; best = p; }
  }
  // A restriction no candidate meets (the gate/up pair has no 12-wave
  // shape): the planner's own choice.
  if (best_t == 1e30 && force) return plan_rows(rows, cols, n_runs, gateup, shared_ok, 0);
  return best;
}

// The shape of the multi-wave shared-digit kernel (kinds 2 and 3: 3, 6 or
// 12 waves, every one owning rows, one block of digits per stage) for the
// launches it was measured to win, else kind -1.  Measured on MI355X over
// the decode matrices of the 7B-shaped (64 runs, 4096 columns), 1.1B-shaped
// (32 runs, 2048) and long-context (16 runs, 2048) models against the
// planner's shapes: query/key/value and gate/up at every one of them (3
// waves and seven stages in flight from 2048 columns, 6 waves from 4096),
// the classifier at 64 runs over 4096 columns (12 waves); the output and
// down matrices stay with the kernel whose waves split the contraction.
RowPlan multi_wave_plan(int epi, uint32_t rows, uint32_t cols, uint32_t n_runs, bool any_width) {
  RowPlan p{-1, 1, 1, 1, 0, 0};
  const bool wide = cols >= 4096;
  if ((cols < 2048 && !any_width) || cols % 128 != 0) return p;
  if (epi == EPI_QKV)
    p = wide ? RowPlan{3, 1, 2, 6, 0, 0} : RowPlan{3, 1, 1, 3, 0, 0};
  else if (epi == EPI_GATEUP)
    p = wide ? RowPlan{2, 2, 2, 6, 0, 0} : RowPlan{3, 2, 1, 3, 0, 0};
  else if (epi == EPI_CLS && ((wide && n_runs >= 48) || any_width))
    p = RowPlan{2, 1, 4, 12, 0, 0};
  else
    return p;
  p.chunks = (n_runs + 16 * p.bt - 1) / (16 * p.bt);
  const uint32_t per_tile = 16 * (epi == EPI_GATEUP ? p.mt / 2 : p.mt) * p.wr;
  p.tiles = (rows + per_tile - 1) / per_tile;
  return p;
}

// The runs [r0, r0 + n) of a batch with their own digit planes and flags:
// every kernel of a position sees them as a batch of n runs.
struct Group {
  uint32_t n;
  RunDesc *runs;
  int8_t *planes0, *planes1;
  uint32_t *oflags;
  int32_t *run_err;
};

Group group(fpi8_engine *e, int g, uint32_t r0, uint32_t n) {
  const size_t planes = 3ull * e->bp * e->kp;
  return Group{n, e->d_runs + r0, e->d_planes0 + g * planes, e->d_planes1 + g * planes,
               e->d_oflags + g * e->n_oflags, e->d_run_err + r0};
}

RowsArgs rows_base(fpi8_engine *e, const Group &G, uint8_t *states, uint32_t cols,
                   const int8_t *planes, const uint32_t *oflag, uint32_t in_sel, uint32_t layer,
                   uint32_t step, uint32_t partial) {
  const uint32_t n_runs = G.n;
  RowsArgs a;
  memset(&a, 0, sizeof a);
  a.cols = cols;
  a.kblocks = ((cols + 63) / 64 + 1) / 2 * 2;  // the packed tiles' blocks per row tile
  a.packed = 1;
  a.planes = planes;
  a.kp = e->kp;
  a.bp = e->bp;
  a.n_runs = n_runs;
  a.in_sel = in_sel;
  a.oflag = oflag;
  a.states = states;
  a.runs = G.runs;
  a.layer = layer;
  a.rope_cos = e->cos_t;
  a.rope_sin = e->sin_t;
  a.silu = e->silu;
  a.head = e->c.head;
  a.half = e->c.head / 2;
  a.kv_heads = e->c.kv_heads;
  a.hidden = e->c.hidden;
  a.step = step;
  a.partial = partial;
  return a;
}

void add_seg(RowsArgs &a, const Mat &m, uint32_t role) {
  Seg &s = a.seg[a.nseg++];
  s.W = m.W;
  s.S = m.S;
  s.rows = m.rows;
  s.role = role;
  s.pad = m.vec ? 1u : 0u;
  s.P = m.P;
}

// Plans the launch over the segments added so far and runs it.
int run_rows(fpi8_engine *e, int epi, RowsArgs &a, uint32_t n_runs, hipStream_t s) {
  const bool gateup = epi == EPI_GATEUP;
  uint32_t rows = 0;
  for (uint32_t i = 0; i < a.nseg; i++) rows += a.seg[i].rows;
  bool shared_ok = a.cols % 128 == 0;
  for (uint32_t i = 0; i < a.nseg; i++) shared_ok = shared_ok && a.seg[i].pad != 0;
  shared_ok = shared_ok || a.packed != 0;
  // A position where some run starts or stops between two phases uses the
  // one shape built for it (32 rows, 32 runs, kind 0).
  RowPlan p = a.partial ? RowPlan{0, 2, 2, 1, (n_runs + 31) / 32, 0}
                        : plan_rows(gateup ? a.seg[0].rows : rows, a.cols, n_runs, gateup,
                                    shared_ok, e->row_kind);
  if (!a.partial && (e->row_kind == 0 || e->row_kind == 7) && shared_ok) {
    const RowPlan m = multi_wave_plan(epi, gateup ? a.seg[0].rows : rows, a.cols, n_runs, e->row_kind == 7);
    if (m.kind >= 0) p = m;
  }
  // Units of 16 * mt rows (of each matrix of the gate/up pair: 16 * mt / 2)
  // over the segments in order; a workgroup finishes one (kind 0) or wr.
  const uint32_t unit_rows = 16 * (gateup ? p.mt / 2 : p.mt);
  uint32_t units = 0;
  for (uint32_t i = 0; i < a.nseg; i++) {
    a.seg[i].unit0 = gateup ? 0 : units;
    if (!gateup || i == 0) units += (a.seg[i].rows + unit_rows - 1) / unit_rows;
  }
  const uint32_t per = p.kind ? (uint32_t)p.wr : 1u;  // kinds 1-3: wr row-owning waves
  a.ntiles = (units + per - 1) / per;
  a.wave_rows = per;
  a.chunks = p.chunks;
  TimedLaunch t(e, T_ROWS, s);
  return launch_rows(epi, p.kind, p.mt, p.bt, a, s);
}

// Where the group's runs keep x, when every run of the turn keeps it at
// the same offset.
void uniform_x(const fpi8_engine *e, const Group &G, uint8_t *states, NormArgs &na) {
  if (!e->uni.on) return;
  na.x_first = states + (uint64_t)(G.runs - e->d_runs) * e->uni.stride + e->uni.off_x;
  na.x_stride = e->uni.stride;
}

// One position of every active run of a group.  `partial`: some run starts
// this position between two phases or stops before its end, so each launch
// checks the steps each run runs (run_flags, RunDesc::end); every launch
// below is one step, in order.
int step_group(fpi8_engine *e, const Group &G, uint8_t *states, hipStream_t s, uint32_t partial) {
  const Cfg &c = e->c;
  const uint32_t n_runs = G.n;
  int r;
  {
    BeginArgs a{states, G.runs, n_runs, G.oflags, e->n_oflags, c.layers,
                c.dim, c.hidden, c.kvd, c.heads, c.head, c.vocab};
    if ((r = launch_begin(a, s))) return r;
  }
  {
    EmbedArgs a{states, G.runs, n_runs, c.dim, c.vocab, e->mats[0].W, e->mats[0].S, partial};
    TimedLaunch t(e, T_EMBED, s);
    if ((r = launch_embed(a, s))) return r;
  }
  for (uint32_t l = 0; l < c.layers; l++) {
    uint32_t *fl = G.oflags + 4 * l;
    const uint32_t s0 = 1 + 7 * l;
    NormArgs na{states, G.runs, n_runs, c.dim, e->norm + (uint64_t)(2 * l) * c.dim,
                G.planes0, e->kp, e->bp, fl + 0, 0, s0, partial};
    uniform_x(e, G, states, na);
    {
      TimedLaunch t(e, T_NORM, s);
      if ((r = launch_norm(na, s))) return r;
    }
    {
      RowsArgs a = rows_base(e, G, states, c.dim, G.planes0, fl + 0, IN_W1, l, s0 + 1, partial);
      add_seg(a, e->layer_mat(l, M_Q), ROLE_Q);
      add_seg(a, e->layer_mat(l, M_K), ROLE_K);
      add_seg(a, e->layer_mat(l, M_V), ROLE_V);
      if ((r = run_rows(e, EPI_QKV, a, n_runs, s))) return r;
    }
    {
      AttnArgs a{states, G.runs, n_runs, l, c.heads, c.kv_heads, c.head,
                 c.heads / c.kv_heads, e->model.inv, e->exp_tab, G.planes0, e->kp, e->bp,
                 fl + 1, e->score_cap, s0 + 2, partial};
      if (e->uni.on) {
        a.u_first = states + (uint64_t)(G.runs - e->d_runs) * e->uni.stride;
        a.u_stride = e->uni.stride;
        a.u_off_q = e->uni.off_w2;
        a.u_off_keys = e->uni.off_keys;
        a.u_cachepos = e->uni.cachepos;
      }
      TimedLaunch t(e, T_ATTN, s);
      if ((r = launch_attention(a, s))) return r;
    }
    if (partial) {
      // the head a turn of units stops inside, for the runs it stops
      AttnTailArgs ta{states, G.runs, n_runs, l, c.kv_heads, c.head, c.heads / c.kv_heads, s0 + 2,
                      e->model.inv, e->exp_tab};
      if ((r = launch_attention_tail(ta, s))) return r;
    }
    {
      RowsArgs a = rows_base(e, G, states, c.dim, G.planes0, fl + 1, IN_W3, l, s0 + 3, partial);
      add_seg(a, e->layer_mat(l, M_O), ROLE_PLAIN);
      if ((r = run_rows(e, EPI_RESID, a, n_runs, s))) return r;
    }
    na.w = e->norm + (uint64_t)(2 * l + 1) * c.dim;
    na.oflag = fl + 2;
    na.step = s0 + 4;
    {
      TimedLaunch t(e, T_NORM, s);
      if ((r = launch_norm(na, s))) return r;
    }
    {
      RowsArgs a = rows_base(e, G, states, c.dim, G.planes0, fl + 2, IN_W1, l, s0 + 5, partial);
      add_seg(a, e->layer_mat(l, M_GATE), ROLE_PLAIN);
      add_seg(a, e->layer_mat(l, M_UP), ROLE_PLAIN);  // shares the gate's row tiles
      a.planes_out = G.planes1;
      a.kp_out = e->kp;
      a.oflag_out = fl + 3;
      if ((r = run_rows(e, EPI_GATEUP, a, n_runs, s))) return r;
    }
    {
      RowsArgs a = rows_base(e, G, states, c.hidden, G.planes1, fl + 3, IN_GATE, l, s0 + 6, partial);
      add_seg(a, e->layer_mat(l, M_DOWN), ROLE_PLAIN);
      if ((r = run_rows(e, EPI_DOWN, a, n_runs, s))) return r;
    }
  }
  uint32_t *ff = G.oflags + 4 * c.layers;
  {
    NormArgs na{states, G.runs, n_runs, c.dim, e->norm + (uint64_t)(2 * c.layers) * c.dim,
                G.planes0, e->kp, e->bp, ff, 1, 1 + 7 * c.layers, partial};
    uniform_x(e, G, states, na);
    TimedLaunch t(e, T_NORM, s);
    if ((r = launch_norm(na, s))) return r;
  }
  {
    RowsArgs a = rows_base(e, G, states, c.dim, G.planes0, ff, IN_W1, 0, 2 + 7 * c.layers, partial);
    add_seg(a, e->mats[1 + 7 * c.layers], ROLE_PLAIN);
    if ((r = run_rows(e, EPI_CLS, a, n_runs, s))) return r;
  }
  {
    SampleArgs a{states, G.runs, n_runs, c.vocab, e->exp_tab, G.run_err, 3 + 7 * c.layers,
                 partial, c.layers};
    TimedLaunch t(e, T_SAMPLE, s);
    if ((r = launch_sample(a, s))) return r;
  }
  return 0;
}

// How many run groups a turn of n_runs uses.
uint32_t n_groups(const fpi8_engine *e, uint32_t n_runs) {
  if (n_runs < 2) return 1;
  return e->streams == 2 ? 2 : 1;
}

// One position of every active run: one group on stream s, or two, the
// second on the engine's side stream, forked from and joined back to s.
int step(fpi8_engine *e, uint8_t *states, uint32_t n_runs, hipStream_t s, uint32_t partial) {
  if (n_groups(e, n_runs) == 1) return step_group(e, group(e, 0, 0, n_runs), states, s, partial);
  int r;
  const uint32_t h = (n_runs / 2 + 15) / 16 * 16 < n_runs ? (n_runs / 2 + 15) / 16 * 16 : n_runs / 2;
  if ((r = hip_ok(hipEventRecord(e->ev_fork, s))) ||
      (r = hip_ok(hipStreamWaitEvent(e->side_stream, e->ev_fork, 0))))
    return r;
  if ((r = step_group(e, group(e, 0, 0, h), states, s, partial))) return r;
  if ((r = step_group(e, group(e, 1, h, n_runs - h), states, e->side_stream, partial))) return r;
  if ((r = hip_ok(hipEventRecord(e->ev_join, e->side_stream))) ||
      (r = hip_ok(hipStreamWaitEvent(s, e->ev_join, 0))))
    return r;
  return 0;
}

// Records one position of the launch sequence as a graph (once per state
// arena and run count).  Every launch of a position reads the run
// descriptors on the device, so the same graph serves every position.
int step_graph(fpi8_engine *e, uint8_t *states, uint32_t n_runs) {
  if (e->graph && e->graph_states == states && e->graph_runs == n_runs && e->graph_cap == e->score_cap &&
      e->graph_groups == n_groups(e, n_runs) && e->graph_uni == e->uni)
    return 0;
  if (e->graph) {
    (void)hipGraphExecDestroy(e->graph);
    e->graph = nullptr;
  }
  int r;
  if (!e->cap_stream && (r = hip_ok(hipStreamCreateWithFlags(&e->cap_stream, hipStreamNonBlocking))))
    return r;
  if ((r = hip_ok(hipStreamBeginCapture(e->cap_stream, hipStreamCaptureModeThreadLocal)))) return r;
  const int rs = step(e, states, n_runs, e->cap_stream, 0);
  hipGraph_t g = nullptr;
  const hipError_t ec = hipStreamEndCapture(e->cap_stream, &g);
  if (rs) {
    if (g) (void)hipGraphDestroy(g);
    return rs;
  }
  if ((r = hip_ok(ec))) return r;
  const hipError_t ei = hipGraphInstantiate(&e->graph, g, nullptr, nullptr, 0);
  (void)hipGraphDestroy(g);
  if ((r = hip_ok(ei))) {
    e->graph = nullptr;
    return r;
  }
  e->graph_states = states;
  e->graph_runs = n_runs;
  e->graph_cap = e->score_cap;
  e->graph_groups = n_groups(e, n_runs);
  e->graph_uni = e->uni;
  return 0;
}

void release(fpi8_engine *e) {
  if (!e) return;
  if (e->graph) (void)hipGraphExecDestroy(e->graph);
  if (e->cap_stream) (void)hipStreamDestroy(e->cap_stream);
  if (e->side_stream) (void)hipStreamDestroy(e->side_stream);
  if (e->ev_fork) (void)hipEventDestroy(e->ev_fork);
  if (e->ev_join) (void)hipEventDestroy(e->ev_join);
  (void)hipFree(e->d_runs);
  (void)hipFree(e->d_packed);
  (void)hipFree(e->d_planes0);
  (void)hipFree(e->d_planes1);
  (void)hipFree(e->d_oflags);
  (void)hipFree(e->d_run_err);
  (void)hipHostFree(e->h_runs);
  (void)hipHostFree(e->h_headers);
  (void)hipHostFree(e->h_err);
  for (Timer &t : e->timers) {
    for (hipEvent_t ev : t.starts) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : t.stops) (void)hipEventDestroy(ev);
  }
  delete e;
}

}  // namespace

extern "C" {

int32_t fpi8_engine_create(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *d_blob,
                           uint64_t blob_len, uint32_t max_runs, fpi8_engine **out) {
  if (!out || !h_section0 || !d_blob || max_runs == 0 || max_runs > 65536) return FPI8_ERR_ARGUMENT;
  *out = nullptr;
  fpi8_engine *e = new fpi8_engine();
  int r = parse_section0(h_section0, section0_len, blob_len, &e->model);
  if (r) { delete e; return r; }
  e->c = e->model.cfg;
  const Cfg &c = e->c;
  if (c.head > 256) { delete e; return FPI8_ERR_UNSUPPORTED; }
  e->d_blob = d_blob;
  e->blob_len = blob_len;
  e->max_runs = max_runs;
  e->max_npos = c.context;
  // scores and partial sums, plus the kernel's own 4 KB, within 160 KB of LDS
  if (attention_lds_bytes(e->max_npos, c.head) + 4096 > 160 * 1024) { delete e; return FPI8_ERR_UNSUPPORTED; }
  e->exp_tab = reinterpret_cast<const uint32_t *>(d_blob + e->model.off_exp);
  e->silu = reinterpret_cast<const int32_t *>(d_blob + e->model.off_silu);
  e->cos_t = reinterpret_cast<const int32_t *>(d_blob + e->model.off_cos);
  e->sin_t = reinterpret_cast<const int32_t *>(d_blob + e->model.off_sin);
  e->norm = reinterpret_cast<const int32_t *>(d_blob + e->model.off_norm);
  e->mats.resize(e->model.mats.size());
  for (size_t i = 0; i < e->mats.size(); i++) {
    const MatLoc &ml = e->model.mats[i];
    Mat &m = e->mats[i];
    m.W = d_blob + ml.w;
    m.S = reinterpret_cast<const uint32_t *>(d_blob + ml.s);
    m.rows = ml.rows;
    m.cols = ml.cols;
    m.vec = (ml.cols % 16 == 0) && ((reinterpret_cast<uintptr_t>(m.W) & 15) == 0);
  }
  // Workspace: digit planes [3][bp][kp] twice, run descriptors, flags.
  e->bp = round_up(max_runs, 64);
  e->kp = round_up(std::max(c.dim, c.hidden), 128);
  e->n_oflags = 4 * c.layers + 1;
  const size_t planes = 3ull * e->bp * e->kp;
  if ((r = hip_ok(hipMalloc(&e->d_runs, sizeof(RunDesc) * max_runs))) ||
      (r = hip_ok(hipMalloc(&e->d_planes0, 2 * planes))) ||
      (r = hip_ok(hipMalloc(&e->d_planes1, 2 * planes))) ||
      (r = hip_ok(hipMalloc(&e->d_oflags, 2 * 4ull * e->n_oflags))) ||
      (r = hip_ok(hipMalloc(&e->d_run_err, 4ull * max_runs))) ||
      (r = hip_ok(hipHostMalloc(&e->h_runs, sizeof(RunDesc) * max_runs))) ||
      (r = hip_ok(hipHostMalloc(&e->h_headers, 128ull * max_runs))) ||
      (r = hip_ok(hipHostMalloc(&e->h_err, 4ull * max_runs))) ||
      (r = hip_ok(hipMemset(e->d_planes0, 0, 2 * planes))) ||
      (r = hip_ok(hipMemset(e->d_planes1, 0, 2 * planes))) ||
      (r = hip_ok(hipMemset(e->d_oflags, 0, 2 * 4ull * e->n_oflags))) ||
      (r = hip_ok(hipStreamCreateWithFlags(&e->side_stream, hipStreamNonBlocking))) ||
      (r = hip_ok(hipEventCreateWithFlags(&e->ev_fork, hipEventDisableTiming))) ||
      (r = hip_ok(hipEventCreateWithFlags(&e->ev_join, hipEventDisableTiming))) ||
      (r = kernels_init(e->max_npos, c.head))) {
    release(e);
    return r;
  }
  // The matrices (all but the embedding, which is read one row at a time)
  // packed once into the tiles the row kernels load whole.
  uint64_t total = 0;
  for (size_t i = 1; i < e->mats.size(); i++) total += packed_bytes(e->mats[i].rows, e->mats[i].cols);
  if ((r = hip_ok(hipMalloc(&e->d_packed, total)))) {
    release(e);
    return r;
  }
  uint64_t at = 0;
  for (size_t i = 1; i < e->mats.size(); i++) {
    Mat &m = e->mats[i];
    m.P = e->d_packed + at;
    if ((r = launch_pack(m.W, m.rows, m.cols, e->d_packed + at, nullptr))) {
      release(e);
      return r;
    }
    at += packed_bytes(m.rows, m.cols);
  }
  if ((r = hip_ok(hipDeviceSynchronize()))) {
    release(e);
    return r;
  }
  *out = e;
  return 0;
}

void fpi8_engine_destroy(fpi8_engine *e) { release(e); }

}  // extern "C"

namespace {

// Phases a position has done when the cursor stands at (phase, layer): 0 at
// its start (phase 3), then one per phase in the order of the pass.
uint32_t phases_done(const Cfg &c, uint32_t phase, uint32_t layer) {
  if (phase <= 3) return 0;
  if (phase <= 16) return 1 + 13 * layer + (phase - 4);
  return 1 + 13 * c.layers + (phase - 17);
}

// Where a turn of at most max_phases phases stops a run whose cursor is
// (pos, phase, layer): the position and the step (run_flags) before which it
// stops there, at the last launch boundary the phases reach.  A launch
// boundary is a cursor between two phases, except inside phase 11 (the
// output rows carry its residual, the second normalization its rest).  No
// stop when the run reaches the end of its cache positions first.
void stop_of(const Cfg &c, uint32_t n_ids, uint32_t cachepos, uint32_t pos, uint32_t phase,
             uint32_t layer, uint32_t max_phases, RunDesc &rd) {
  rd.stop_pos = 0xFFFFFFFFu;
  rd.stop_step = 0xFFFFFFFFu;
  uint64_t k = max_phases;
  uint32_t d = phases_done(c, phase, layer);
  for (uint32_t t = pos; t < cachepos; t++, d = 0) {
    const bool gen = t + 1 >= n_ids;
    const uint64_t total = 1 + 13ull * c.layers + (gen ? 3 : 0);
    if (k >= total - d) {
      k -= total - d;
      continue;
    }
    const uint64_t target = d + k;
    uint32_t best = 0;
    auto at = [&](uint64_t end, uint64_t done) {
      if (done > d && done <= target && done < total) best = (uint32_t)end;
    };
    at(1, 1);
    for (uint64_t l = 0; l < c.layers; l++) {
      at(2 + 7 * l, 2 + 13 * l);   // after the first normalization: phase 5
      at(3 + 7 * l, 6 + 13 * l);   // after q/k/v with rotary: phase 9
      at(4 + 7 * l, 7 + 13 * l);   // after attention: phase 10
      at(6 + 7 * l, 9 + 13 * l);   // after the second normalization: phase 12
      at(7 + 7 * l, 12 + 13 * l);  // after gate/up with SiLU: phase 15
      at(8 + 7 * l, 14 + 13 * l);  // after down: phase 4 of the next layer, or 17
    }
    if (gen) {
      at(2 + 7ull * c.layers, 2 + 13ull * c.layers);  // after the final normalization: 18
      at(3 + 7ull * c.layers, 3 + 13ull * c.layers);  // after the classifier: 19
    }
    rd.stop_pos = t;
    rd.stop_step = best;
    return;
  }
}

// A turn over a batch: up to max_positions positions, and, when max_phases
// is not ~0, up to max_phases phases of each run, or, when max_units is not
// ~0, up to max_units units of work of each run (counted on the device,
// where the draw pass shows its length).
int32_t turn(fpi8_engine *e, uint8_t *d_states, uint64_t stride, uint32_t n_runs,
             uint32_t max_positions, uint32_t max_phases, uint64_t max_units, void *stream,
             int32_t *h_run_errors, bool bind_only = false) {
  if (!e || !d_states || n_runs == 0 || n_runs > e->max_runs) return FPI8_ERR_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  e->bound_states = nullptr;  // this turn replaces the device run descriptors
  if ((reinterpret_cast<uintptr_t>(d_states) & 7) != 0 || (stride & 7) != 0 || stride < 128) {
    if (h_run_errors)
      for (uint32_t b = 0; b < n_runs; b++) h_run_errors[b] = FPI8_INVALID_STATE;
    return FPI8_INVALID_STATE;
  }
  int r;
  // Read every header, check it, fill the static run descriptors.
  if ((r = hip_ok(hipMemcpy2DAsync(e->h_headers, 128, d_states, stride, 128, n_runs,
                                   hipMemcpyDeviceToHost, s))) ||
      (r = hip_ok(hipStreamSynchronize(s))))
    return r;
  // Positions each run computes in this turn (its first one maybe only in
  // part), and which positions of the turn have a run that starts or stops
  // between two phases.
  std::vector<uint32_t> first(n_runs, 0), count(n_runs, 0);
  uint32_t steps = 0, resume = 0;
  for (uint32_t b = 0; b < n_runs; b++) {
    RunDesc &rd = e->h_runs[b];
    memset(&rd, 0, sizeof rd);
    rd.stop_pos = 0xFFFFFFFFu;
    rd.stop_step = 0xFFFFFFFFu;
    const uint8_t *h = e->h_headers + 128ull * b;
    StateLayout L;
    const int chk = check_header(e->c, h, stride, &L);
    e->h_err[b] = chk > 0 ? chk : 0;
    if (chk != 0) continue;
    uint32_t v, pos, phase, layer;
    memcpy(&v, h + ST_NIDS, 4); rd.n_ids = v;
    memcpy(&v, h + ST_MAX, 4); rd.max_tokens = v;
    memcpy(&v, h + ST_TEMP, 4); rd.temp = v;
    memcpy(&pos, h + ST_POSITION, 4);
    memcpy(&phase, h + ST_PHASE, 4);
    memcpy(&layer, h + ST_LAYER, 4);
    rd.cachepos = L.cachepos;
    rd.valid = 1;
    rd.base = stride * b;
    rd.off_x = L.x; rd.off_w1 = L.w1; rd.off_w2 = L.w2; rd.off_w3 = L.w3;
    rd.off_gate = L.gate; rd.off_up = L.up; rd.off_logits = L.logits; rd.off_scores = L.scores;
    rd.off_keys = L.keys; rd.off_values = L.values; rd.off_ids = L.ids; rd.off_out = L.out;
    if (max_phases != 0xFFFFFFFFu)
      stop_of(e->c, rd.n_ids, L.cachepos, pos, phase, layer, max_phases, rd);
    first[b] = pos;
    count[b] = rd.stop_pos == 0xFFFFFFFFu ? L.cachepos - pos
                                           : rd.stop_pos - pos + (rd.stop_step != 0 ? 1 : 0);
    if (max_units != ~0ull) {
      // Every position has at least the units of a prompt position at its
      // first place: a bound on the positions the budget reaches.
      const Cfg &c = e->c;
      const uint64_t per_layer = 5 + 3ull * c.dim + 2ull * c.kvd + 2ull * c.hidden +
                                 (uint64_t)c.heads * (3 + c.head);
      const uint64_t least = 1 + per_layer * c.layers;
      rd.units = 1;
      rd.budget = max_units;
      count[b] = (uint32_t)std::min<uint64_t>(count[b], max_units / least + 2);
    }
    steps = std::max(steps, count[b]);
    if (phase != 3) resume = 1;
  }
  steps = std::min(steps, max_positions);
  // Attention keeps one score per cached position in LDS: size it for the
  // longest cache of the batch (in steps of 256, so a graph recorded for one
  // turn serves the next).
  uint32_t cap = 256;
  for (uint32_t b = 0; b < n_runs; b++)
    if (e->h_runs[b].valid) cap = std::max(cap, (e->h_runs[b].cachepos + 255) / 256 * 256);
  // One layout for the whole batch, all of whose states are valid (so that
  // every run's state holds the bytes read at those offsets).
  {
    const RunDesc &r0 = e->h_runs[0];
    fpi8_engine::Uniform u;
    u.on = r0.valid != 0;
    u.stride = stride;
    u.off_x = r0.off_x; u.off_w2 = r0.off_w2; u.off_keys = r0.off_keys; u.off_values = r0.off_values;
    u.cachepos = r0.cachepos;
    for (uint32_t b = 1; b < n_runs && u.on; b++) {
      const RunDesc &rd = e->h_runs[b];
      u.on = rd.valid && rd.off_x == u.off_x && rd.off_w2 == u.off_w2 && rd.off_keys == u.off_keys &&
             rd.off_values == u.off_values && rd.cachepos == u.cachepos;
    }
    if (!u.on) u = fpi8_engine::Uniform{};
    e->uni = u;
  }
  e->score_cap = std::min(cap, e->max_npos);
  if ((r = hip_ok(hipMemcpyAsync(e->d_runs, e->h_runs, sizeof(RunDesc) * n_runs,
                                 hipMemcpyHostToDevice, s))) ||
      (r = hip_ok(hipMemcpyAsync(e->d_run_err, e->h_err, 4ull * n_runs, hipMemcpyHostToDevice, s))))
    return r;
  if (bind_only) {
    // Queued turns advance whole positions: bound the positions any run has left.
    uint32_t left = 0;
    for (uint32_t b = 0; b < n_runs; b++)
      if (e->h_runs[b].valid) left = std::max(left, count[b]);
    if ((r = hip_ok(hipStreamSynchronize(s)))) return r;  // the pinned descriptors are copied
    e->bound_states = d_states;
    e->bound_runs = n_runs;
    e->bound_left = left;
    e->bound_resume = resume;
    int32_t first_err = 0;
    for (uint32_t b = 0; b < n_runs; b++) {
      if (h_run_errors) h_run_errors[b] = e->h_err[b];
      if (!first_err && e->h_err[b]) first_err = e->h_err[b];
    }
    return first_err;
  }
  if ((r = launch_turn_start(d_states, e->d_runs, n_runs, s))) return r;
  bool timing = false;
  for (const Timer &t : e->timers) timing = timing || t.on;
  // A position where some run starts or stops between two phases runs in
  // launches that check each run's steps; the recorded position serves the
  // others.
  for (uint32_t k = 0; k < steps; k++) {
    uint32_t partial = k == 0 ? resume : 0;
    if (max_units != ~0ull) partial = 1;
    for (uint32_t b = 0; b < n_runs && !partial; b++) {
      const RunDesc &rd = e->h_runs[b];
      if (rd.valid && rd.stop_pos == first[b] + k && rd.stop_step != 0) partial = 1;
    }
    if (!partial && !timing && e->use_graph) {
      if ((r = step_graph(e, d_states, n_runs))) return r;
      if ((r = hip_ok(hipGraphLaunch(e->graph, s)))) return r;
    } else if ((r = step(e, d_states, n_runs, s, partial))) {
      return r;
    }
  }
  if ((r = hip_ok(hipMemcpyAsync(e->h_err, e->d_run_err, 4ull * n_runs, hipMemcpyDeviceToHost, s))) ||
      (r = hip_ok(hipStreamSynchronize(s))))
    return r;
  int32_t first_err = 0;
  for (uint32_t b = 0; b < n_runs; b++) {
    if (h_run_errors) h_run_errors[b] = e->h_err[b];
    if (!first_err && e->h_err[b]) first_err = e->h_err[b];
  }
  return first_err;
}

}  // namespace

extern "C" {

int32_t fpi8_turn(fpi8_engine *e, uint8_t *d_states, uint64_t stride, uint32_t n_runs,
                  uint32_t max_positions, void *stream, int32_t *h_run_errors) {
  return turn(e, d_states, stride, n_runs, max_positions, 0xFFFFFFFFu, ~0ull, stream, h_run_errors);
}

int32_t fpi8_turn_bind(fpi8_engine *e, uint8_t *d_states, uint64_t stride, uint32_t n_runs, void *stream,
                       int32_t *h_run_errors) {
  return turn(e, d_states, stride, n_runs, 0xFFFFFFFFu, 0xFFFFFFFFu, ~0ull, stream, h_run_errors, true);
}

int32_t fpi8_turn_async(fpi8_engine *e, uint32_t max_positions, void *stream, int32_t *d_run_errors) {
  if (!e || !e->bound_states) return FPI8_ERR_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  uint8_t *states = e->bound_states;
  const uint32_t n_runs = e->bound_runs;
  const uint32_t steps = std::min(max_positions, e->bound_left);
  e->bound_left -= steps;
  int r;
  if ((r = launch_turn_start(states, e->d_runs, n_runs, s))) return r;
  bool timing = false;
  for (const Timer &t : e->timers) timing = timing || t.on;
  for (uint32_t k = 0; k < steps; k++) {
    const uint32_t partial = k == 0 ? e->bound_resume : 0;
    if (!partial && !timing && e->use_graph) {
      if ((r = step_graph(e, states, n_runs))) return r;
      if ((r = hip_ok(hipGraphLaunch(e->graph, s)))) return r;
    } else if ((r = step(e, states, n_runs, s, partial))) {
      return r;
    }
    e->bound_resume = 0;
  }
  if (d_run_errors &&
      (r = hip_ok(hipMemcpyAsync(d_run_errors, e->d_run_err, 4ull * n_runs, hipMemcpyDeviceToDevice, s))))
    return r;
  return 0;
}

int32_t fpi8_turn_phases(fpi8_engine *e, uint8_t *d_states, uint64_t stride, uint32_t n_runs,
                         uint32_t max_phases, void *stream, int32_t *h_run_errors) {
  if (max_phases == 0xFFFFFFFFu) max_phases--;
  return turn(e, d_states, stride, n_runs, 0xFFFFFFFFu, max_phases, ~0ull, stream, h_run_errors);
}

int32_t fpi8_turn_units(fpi8_engine *e, uint8_t *d_states, uint64_t stride, uint32_t n_runs,
                        uint64_t max_units, void *stream, int32_t *h_run_errors) {
  if (max_units == ~0ull) max_units--;
  return turn(e, d_states, stride, n_runs, 0xFFFFFFFFu, 0xFFFFFFFFu, max_units, stream,
              h_run_errors);
}

int32_t fpi8_engine_set_row_kernel(fpi8_engine *e, int32_t kind) {
  if (!e || kind < 0 || kind > 7) return FPI8_ERR_ARGUMENT;
  if (e->row_kind != kind) {
    e->row_kind = kind;
    e->graph_states = nullptr;  // record the position again with the new shapes
    e->graph_runs = 0;
  }
  return 0;
}

int32_t fpi8_engine_set_graph(fpi8_engine *e, int32_t enable) {
  if (!e) return FPI8_ERR_ARGUMENT;
  e->use_graph = enable != 0;
  return 0;
}

int32_t fpi8_engine_set_streams(fpi8_engine *e, int32_t streams) {
  if (!e || streams < 0 || streams > 2) return FPI8_ERR_ARGUMENT;
  e->streams = streams;
  return 0;
}

int32_t fpi8_engine_set_timing(fpi8_engine *e, int32_t kernel, int32_t enable) {
  if (!e || kernel < 0 || kernel >= kTimingClasses) return FPI8_ERR_ARGUMENT;
  Timer &t = e->timers[kernel];
  t.on = enable != 0;
  t.used = 0;
  return 0;
}

int32_t fpi8_engine_timing(fpi8_engine *e, int32_t kernel, double *total_ms, uint64_t *launches) {
  if (!e || kernel < 0 || kernel >= kTimingClasses) return FPI8_ERR_ARGUMENT;
  return timer_sum(e->timers[kernel], total_ms, launches);
}

int32_t fpi8_matrix_rows_set_timing(int32_t enable) {
  g_rows_timer.on = enable != 0;
  g_rows_timer.used = 0;
  return 0;
}

int32_t fpi8_matrix_rows_timing(double *total_ms, uint64_t *launches) {
  return timer_sum(g_rows_timer, total_ms, launches);
}

int32_t fpi8_matrix_rows_set_path(int32_t path) {
  if (path < 0 || path > 2) return FPI8_ERR_ARGUMENT;
  g_rows_path.store(path);
  return 0;
}

// Workspace of the standalone row: the overflow word (256 bytes kept), then the digits.
uint64_t fpi8_matrix_rows_workspace_size(uint32_t rows, uint32_t cols, uint32_t batch) {
  (void)rows;
  const uint64_t kp = round_up(cols, 128), bp = round_up(batch, 64);
  return 256 + 3 * bp * kp;
}

uint64_t fpi8_matrix_packed_size(uint32_t rows, uint32_t cols) {
  if (rows == 0 || cols == 0 || cols > 65536) return UINT64_MAX;
  return packed_bytes(rows, cols);
}

int32_t fpi8_matrix_pack(const uint8_t *d_W, uint32_t rows, uint32_t cols, uint8_t *d_P,
                         uint64_t p_len, void *stream) {
  if (!d_W || !d_P || rows == 0 || cols == 0 || cols > 65536 || p_len < packed_bytes(rows, cols))
    return FPI8_ERR_ARGUMENT;
  return launch_pack(d_W, rows, cols, d_P, stream);
}

}  // extern "C"

namespace fpi8 {

// The standalone row over row-major weights (d_W) or packed tiles (d_P).
int matrix_rows(const uint8_t *d_W, const uint8_t *d_P, const uint32_t *d_scale, uint32_t rows,
                uint32_t cols, const int64_t *d_x, uint32_t batch, int64_t *d_y, void *d_work,
                uint64_t work_len, void *stream, bool timed) {
  Timer untimed;  // no events: an empty timer that is off
  Timer &tm = timed ? g_rows_timer : untimed;
  if ((!d_W && !d_P) || !d_scale || !d_x || !d_y || !d_work || rows == 0 || cols == 0 ||
      batch == 0 || cols > 65536 || batch > 65536)
    return FPI8_ERR_ARGUMENT;
  if (work_len < fpi8_matrix_rows_workspace_size(rows, cols, batch) ||
      (reinterpret_cast<uintptr_t>(d_work) & 255) != 0 || (reinterpret_cast<uintptr_t>(d_P) & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(d_x) & 7) != 0 || (reinterpret_cast<uintptr_t>(d_y) & 7) != 0)
    return FPI8_ERR_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  const uint32_t kp = round_up(cols, 128), bp = round_up(batch, 64);
  uint8_t *base = reinterpret_cast<uint8_t *>(d_work);
  uint32_t *flag = reinterpret_cast<uint32_t *>(base);
  int8_t *planes = reinterpret_cast<int8_t *>(base + 256);
  const bool packed = d_P != nullptr;
  const bool aligned = cols % 16 == 0 && (reinterpret_cast<uintptr_t>(d_W) & 15) == 0;
  const bool shared_ok = packed || (aligned && cols % 128 == 0);
  const uint32_t kblocks = packed ? ((cols + 63) / 64 + 1) / 2 * 2 : (cols + 63) / 64;
  RowsArgs a;
  memset(&a, 0, sizeof a);
  a.cols = cols;
  a.kblocks = kblocks;
  a.packed = packed ? 1u : 0u;
  a.kp = kp;
  a.bp = bp;
  a.n_runs = batch;
  a.in_sel = IN_RAW;
  a.x_raw = d_x;
  a.y_raw = d_y;
  Seg &sg = a.seg[0];
  sg.W = packed ? nullptr : d_W;
  sg.P = d_P;
  sg.S = d_scale;
  sg.rows = rows;
  sg.unit0 = 0;
  sg.role = ROLE_PLAIN;
  sg.pad = packed || aligned ? 1u : 0u;
  a.nseg = 1;

  static std::atomic<uint32_t> calls{0};

  // Many rows of a packed matrix: the persistent streaming kernel over
  // fragment-major digit planes (one launch for the digits, one for the rows).
  // On request, up to four inputs take the vector-ALU variant instead (one
  // launch: its workgroups split the inputs into digits in LDS).
  if (packed && batch <= 128 && kblocks % kStreamBlockMultiple == 0 && rows >= stream_min_rows()) {
    if (g_rows_path.load() == 2 && stream_valu_fits(kblocks, batch)) {
      TimedLaunch t(tm, s);
      return launch_rows_stream_valu(a, s);
    }
    uint32_t seq = ++calls;
    if (seq == 0) seq = ++calls;
    int r = launch_digits_raw(d_x, batch, cols, planes, kp, bp, 0, flag, seq, s);
    if (r) return r;
    a.planes = planes;
    a.oflag = flag;
    a.oflag_seq = seq;
    a.compact = 0;
    a.chunks = 1;
    TimedLaunch t(tm, s);
    return launch_rows_stream(a, s);
  }

  // One or two inputs whose digits fit a wave's LDS share: one launch, the
  // kernel's waves split the inputs into digits themselves.
  const uint32_t per = (kblocks + 3) / 4;
  if (batch <= 2 && (uint64_t)3 * batch * per * 64 <= kRawInputLds) {
    const RowPlan p = plan_rows(rows, cols, batch, false, shared_ok, 1);
    if (p.kind == 0 && p.bt == 1 && (p.mt == 1 || p.mt == 4)) {
      a.ntiles = p.tiles;
      a.wave_rows = 1;
      a.chunks = p.chunks;
      TimedLaunch t(tm, s);
      return launch_rows_raw(p.mt, a, s);
    }
  }

  // Otherwise the digits first.  Each call marks an overflow with its own
  // number, so the flag word never needs clearing; a stale word that happens
  // to match only sends the call down the exact path, which gives the same
  // result.
  uint32_t seq = ++calls;
  if (seq == 0) seq = ++calls;
  // One or two inputs: plain digit rows, so the four lanes of a run read one
  // whole 64-byte piece per block (the kernel whose waves split the
  // contraction reads them); more: the fragment-major layout both kernels
  // read, where the runs of a lane group share 16-byte pieces of one line.
  const uint32_t compact = batch <= 2 ? 1u : 0u;
  int r = launch_digits_raw(d_x, batch, cols, planes, kp, bp, compact, flag, seq, s);
  if (r) return r;
  const RowPlan p = plan_rows(rows, cols, batch, false, shared_ok, compact ? 1 : 0);
  a.planes = planes;
  a.oflag = flag;
  a.oflag_seq = seq;
  a.compact = compact;
  a.ntiles = p.tiles;
  a.wave_rows = p.kind ? (uint32_t)p.wr : 1u;
  a.chunks = p.chunks;
  TimedLaunch t(tm, s);
  return launch_rows(EPI_RAW, p.kind, p.mt, p.bt, a, s);
}

}  // namespace fpi8

extern "C" {

int32_t fpi8_matrix_rows(const uint8_t *d_W, const uint32_t *d_scale, uint32_t rows,
                         uint32_t cols, const int64_t *d_x, uint32_t batch, int64_t *d_y,
                         void *d_work, uint64_t work_len, void *stream) {
  if (!d_W) return FPI8_ERR_ARGUMENT;
  return fpi8::matrix_rows(d_W, nullptr, d_scale, rows, cols, d_x, batch, d_y, d_work, work_len, stream,
                           true);
}

int32_t fpi8_matrix_rows_packed(const uint8_t *d_P, const uint32_t *d_scale, uint32_t rows,
                                uint32_t cols, const int64_t *d_x, uint32_t batch, int64_t *d_y,
                                void *d_work, uint64_t work_len, void *stream) {
  if (!d_P) return FPI8_ERR_ARGUMENT;
  return fpi8::matrix_rows(nullptr, d_P, d_scale, rows, cols, d_x, batch, d_y, d_work, work_len, stream,
                           true);
}

}  // extern "C"
