// fpi8_internal.h - types shared by the host side and the HIP kernels of
// libfpi8 (the MI355X fixed-point inference core).  Not part of the C ABI.
#pragma once
#include <stdint.h>

#include <vector>

namespace fpi8 {

// Configuration: dim, hidden, layers, heads, kv_heads, vocab, context.
struct Cfg {
  uint32_t dim, hidden, layers, heads, kv_heads, vocab, context;
  uint32_t head, kvd;
};

bool cfg_from_words(const uint32_t w[7], Cfg *c);

// Where a matrix lies inside the artifact (byte offsets from its start).
struct MatLoc {
  uint64_t w = 0, s = 0;
  uint32_t rows = 0, cols = 0;
};

// Section zero, parsed: table offsets and the matrix table, [0] embedding,
// [1 + 7 * layer + kind - 1] layer matrices, [1 + 7 * layers] classifier.
struct Model {
  Cfg cfg;
  uint32_t inv;
  uint64_t off_exp, off_silu, off_cos, off_sin, off_norm;
  std::vector<MatLoc> mats;
};

int parse_section0(const uint8_t *s0, uint64_t s0_len, uint64_t blob_len, Model *m);

// The tokenizer block of section zero (layout in fpi8_tokenizer.cpp).
struct Vocab {
  uint32_t n = 0, longest = 0;
  const uint8_t *score = nullptr, *start = nullptr, *sorted = nullptr, *pool = nullptr;
  uint32_t at(const uint8_t *p, uint32_t i) const {
    uint32_t v;
    __builtin_memcpy(&v, p + 4ull * i, 4);
    return v;
  }
  const uint8_t *piece(uint32_t id) const { return pool + at(start, id); }
  uint32_t piece_len(uint32_t id) const { return at(start, id + 1) - at(start, id); }
};
bool vocab_parse(const uint8_t *blk, uint64_t len, uint32_t vocab, Vocab *v);
int64_t vocab_lookup(const Vocab &v, const uint8_t *s, uint32_t n);
int32_t vocab_of(const uint8_t *s0, uint64_t s0_len, Model *m, Vocab *v);

// Byte offsets of a run's buffers inside its state.
struct StateLayout {
  uint64_t ids, out, x, w1, w2, w3, gate, up, logits, scores, keys, values, total;
  uint32_t cachepos;
};
bool state_layout(const Cfg &c, uint32_t n_ids, uint32_t max_tokens, StateLayout *L);
int check_header(const Cfg &c, const uint8_t *h, uint64_t stride, StateLayout *L);

// The state's tag, FPI8ST01.
extern const char kStateTag[8];

// State header field offsets.
enum : uint32_t {
  ST_PHASE = 8, ST_LAYER = 12, ST_ROW = 16, ST_POSITION = 20, ST_TOKEN = 24, ST_ERROR = 28,
  ST_NIDS = 32, ST_MAX = 36, ST_TEMP = 40, ST_GENERATED = 44, ST_CACHEPOS = 48,
  ST_GENERATOR = 72, ST_TURNS = 80, ST_MAXSCORE = 88, ST_CHOSEN = 96, ST_PASS = 100, ST_SUM = 104,
  ST_REMAINDER = 112, ST_STAGE = 120, ST_INDEX = 124, ST_HEADER = 128
};

// Matrix kinds of the artifact.
enum : uint32_t { M_EMBED, M_Q, M_K, M_V, M_O, M_GATE, M_UP, M_DOWN, M_CLS, M_KINDS };

// What one launch needs to know about a run.  The static part is filled on
// the host at the start of a turn, the dynamic part by the first kernel of
// every position.
struct RunDesc {  // u32 fields (an even count), then 8-byte fields
  // dynamic
  uint32_t flags;     // RUN_ACTIVE, RUN_GEN, and where the position resumes (run_flags)
  uint32_t pos;       // position computed in this step
  uint32_t token;     // token embedded in this step
  uint32_t errkey;    // first failing (layer, phase) of this step, ~0 if none
  uint32_t end;       // the step this position stops before (~0: it runs to its end)
  // a turn of units that stops the run inside this position: the cursor it
  // stops at (phase, 0 for none; layer; row, stage, index and pass as the
  // state's header has them), and whether the run has stopped
  uint32_t stop_ph, stop_layer, stop_row, stop_stage, stop_index, stop_pass;
  uint32_t stop_in;   // the step of the launch the stop falls inside (~0: between launches)
  uint32_t halted;
  // static
  uint32_t n_ids, max_tokens, temp, cachepos;
  uint32_t valid;     // passed the host checks at the start of the turn
  uint32_t stop_pos;  // the turn stops this run in position stop_pos before step
  uint32_t stop_step; // stop_step (0: the position does not start); ~0: no stop
  uint32_t units;     // a turn of units of work: the budget below counts them
  uint32_t pad;
  uint64_t budget;    // units of work left (dynamic; a turn of units only)
  uint64_t base;      // byte offset of the run's state in the arena
  uint64_t off_x, off_w1, off_w2, off_w3, off_gate, off_up, off_logits, off_scores;
  uint64_t off_keys, off_values, off_ids, off_out;
};

enum : uint32_t { RUN_ACTIVE = 1u, RUN_GEN = 2u };

// A position runs as a fixed sequence of launches, numbered by step: 0 the
// embedding; for layer l, 1 + 7l the first normalization, 2 + 7l the query,
// key and value rows with rotary, 3 + 7l attention, 4 + 7l the output rows
// with the residual, 5 + 7l the second normalization, 6 + 7l gate/up with
// SiLU, 7 + 7l down with the residual; then 1 + 7L the final normalization,
// 2 + 7L the classifier and 3 + 7L sampling.  A run whose state stands
// between two phases of a position starts at a later step (`start`), and the
// fused launch that holds its phase takes the results of the phases already
// done from the state (`pick`, the state's phase; at step start + after).
// A turn may also stop a run before a later step (RunDesc::end).
// flags bits: 0-1 RUN_ACTIVE / RUN_GEN, 2-6 pick, 7 after, 8-31 start.
constexpr uint32_t run_flags(uint32_t active_gen, uint32_t start, uint32_t pick, uint32_t after) {
  return active_gen | (pick << 2) | (after << 7) | (start << 8);
}

// Rows of one matrix inside a row-kernel launch.
struct Seg {
  const uint8_t *W;      // rows x cols weight bytes (weight + 128), row-major
  const uint8_t *P;      // the same bytes packed in 16 x 64 tiles (see launch_pack), or nullptr
  const uint32_t *S;     // rows Q24 scales
  uint32_t rows;
  uint32_t unit0;        // first unit (16 * MT rows, or 16 * MT / 2 of the gate/up pair) of this matrix
  uint32_t role;         // epilogue role of the rows (ROLE_*)
  uint32_t pad;
};

enum : uint32_t { ROLE_Q, ROLE_K, ROLE_V, ROLE_PLAIN };

// Epilogues of the row kernel.
enum : int { EPI_RAW, EPI_QKV, EPI_RESID, EPI_GATEUP, EPI_DOWN, EPI_CLS };

// Which i64 input the exact (non-limb) path reads.
enum : uint32_t { IN_W1, IN_W3, IN_GATE, IN_RAW };

struct RowsArgs {
  Seg seg[3];
  uint32_t nseg;
  uint32_t ntiles;          // row tiles over all segments: one unit (kind 0) or wave_rows units (kind 1)
  uint32_t wave_rows;       // kind 1: waves of a workgroup (1..4) that own a unit of rows
  uint32_t cols;            // contraction length
  uint32_t kblocks;         // ceil(cols / 64)
  const int8_t *planes;     // [3][bp][kp] signed digits of the input, fragment-major
  uint32_t kp;              // plane pitch in bytes (multiple of 64, >= kblocks * 64)
  uint32_t bp;              // planes per limb (multiple of 16)
  uint32_t n_runs;
  uint32_t in_sel;          // IN_* for the exact path
  const uint32_t *oflag;    // some input needs more than three limbs: *oflag != 0, or
  uint32_t oflag_seq;       // when nonzero, *oflag == oflag_seq
  uint32_t compact;         // 1: planes [3][bp][kp] plain row-major (kp-byte rows), 0: fragment-major
  uint32_t packed;          // 1: the fast path reads every segment's packed tiles (kblocks even)
  // context
  uint8_t *states;          // state arena (turn) or nullptr (standalone)
  RunDesc *runs;
  uint32_t layer;
  const int32_t *rope_cos, *rope_sin;   // [context][head/2]
  const int32_t *silu;                  // [4097]
  uint32_t head, half, kv_heads, hidden;
  uint32_t step;            // this launch's step in the position (run_flags)
  uint32_t partial;         // some run starts this position after step 0 or stops before its end
  // gate/up epilogue: digits of the hidden vector for the down matrix
  int8_t *planes_out;
  uint32_t kp_out;
  uint32_t *oflag_out;
  // standalone matrix rows
  const int64_t *x_raw;     // [n_runs][cols]
  int64_t *y_raw;           // [n_runs][rows]
  uint32_t chunks;          // batch chunks of 16 * BT runs
};

struct NormArgs {
  uint8_t *states;
  RunDesc *runs;
  uint32_t n_runs, dim;
  const int32_t *w;         // norm weights
  int8_t *planes;
  uint32_t kp, bp;
  uint32_t *oflag;
  uint32_t final_norm;      // 1: only generating runs (phase 17)
  uint32_t step, partial;   // as in RowsArgs
  // Every run of the batch keeps x at the same offset of its state: run b's
  // x is at x_first + b * x_stride (nullptr: read each run's descriptor first)
  const uint8_t *x_first;
  uint64_t x_stride;
};

struct EmbedArgs {
  uint8_t *states;
  RunDesc *runs;
  uint32_t n_runs, dim, vocab;
  const uint8_t *E;
  const uint32_t *S;
  uint32_t partial;         // as in RowsArgs (the embedding is step 0)
};

struct AttnArgs {
  uint8_t *states;
  RunDesc *runs;
  uint32_t n_runs, layer, heads, kv_heads, head, group;
  uint32_t inv;
  const uint32_t *exp_tab;
  int8_t *planes;
  uint32_t kp, bp;
  uint32_t *oflag;
  uint32_t max_npos;        // LDS score slots: at least every run's cache positions
  uint32_t step, partial;   // as in RowsArgs
  // Every run of the batch has the same layout: run b's state is at
  // u_first + b * u_stride, its queries at u_off_q, its keys at u_off_keys
  // and u_cachepos cache positions (u_first nullptr: read each run's
  // descriptor first)
  const uint8_t *u_first;
  uint64_t u_stride, u_off_q, u_off_keys;
  uint32_t u_cachepos;
};

// The head of attention a turn of units stops inside: its stages up to the
// cursor (one workgroup per run).
struct AttnTailArgs {
  uint8_t *states;
  RunDesc *runs;
  uint32_t n_runs, layer, kv_heads, head, group, step;
  uint32_t inv;
  const uint32_t *exp_tab;
};

struct SampleArgs {
  uint8_t *states;
  RunDesc *runs;
  uint32_t n_runs, vocab;
  const uint32_t *exp_tab;
  int32_t *run_err;
  uint32_t step, partial, layers;  // step and partial as in RowsArgs
};

struct BeginArgs {
  uint8_t *states;
  RunDesc *runs;
  uint32_t n_runs;
  uint32_t *oflags;
  uint32_t n_oflags;
  uint32_t layers;
  // the sizes a turn of units counts its units by
  uint32_t dim, hidden, kvd, heads, head, vocab;
};

// Launchers (defined in the .hip file).
int launch_begin(const BeginArgs &a, void *stream);
int launch_turn_start(uint8_t *states, RunDesc *runs, uint32_t n_runs, void *stream);
int launch_embed(const EmbedArgs &a, void *stream);
int launch_norm(const NormArgs &a, void *stream);
// kind 0: the four waves of a workgroup split the contraction of 16 * mt
// rows; kind 1: they own 16 * mt rows each and share the digits through LDS
// (columns a multiple of 128, 16-byte aligned rows).
int launch_rows(int epi, int kind, int mt, int bt, const RowsArgs &a, void *stream);
// The standalone row of one or two inputs (x_raw) on the
// kernel whose waves split the contraction, without digit planes: each wave
// splits its own columns of the inputs into digits in kRawInputLds bytes of
// LDS, so 3 * n_runs * ceil(kblocks / 4) * 64 must fit that; mt 1 or 4.
constexpr uint32_t kRawInputLds = 24576;
int launch_rows_raw(int mt, const RowsArgs &a, void *stream);
// The standalone row over a packed matrix with many rows (one segment,
// fragment-major digit planes of at most 128 runs, kblocks a multiple of
// kStreamBlockMultiple): persistent workgroups, see fpi8_rows_stream.hip.
// Worth it from stream_min_rows() rows on (every wave gets a 64-row tile).
constexpr uint32_t kStreamBlockMultiple = 8;
uint32_t stream_min_rows();
// The vector-ALU streaming kernel (1 to 4 inputs, their digits in LDS).
constexpr uint32_t kStreamValuLds = 147456;
bool stream_valu_fits(uint32_t kblocks, uint32_t n_runs);
int launch_rows_stream_valu(const RowsArgs &a, void *stream);
int launch_rows_stream(const RowsArgs &a, void *stream);
// The standalone row (fpi8_matrix_rows / fpi8_matrix_rows_packed) over a
// caller's workspace; `timed` lets fpi8_matrix_rows_set_timing bracket its
// row-kernel launch with events.  Allocates nothing.
int matrix_rows(const uint8_t *d_W, const uint8_t *d_P, const uint32_t *d_scale, uint32_t rows,
                uint32_t cols, const int64_t *d_x, uint32_t batch, int64_t *d_y, void *d_work,
                uint64_t work_len, void *stream, bool timed);
int launch_attention(const AttnArgs &a, void *stream);
int launch_attention_tail(const AttnTailArgs &a, void *stream);
// Packs a rows x cols byte matrix into tiles of 16 rows x 64 columns, tile
// (rt, kb) at ((rt * kbp + kb) * 1024), inside it lane l = 16 g + i at
// 16 l holding row 16 rt + i, columns 64 kb + 16 g .. + 15 (the layout of
// one MFMA operand); kbp = ceil(cols / 64) rounded up to even.  Bytes
// outside the matrix are 0x80 (the weight 0).  P holds
// ceil(rows / 16) * kbp * 1024 bytes.
int launch_pack(const uint8_t *W, uint32_t rows, uint32_t cols, uint8_t *P, void *stream);
uint64_t packed_bytes(uint32_t rows, uint32_t cols);
int launch_sample(const SampleArgs &a, void *stream);
// Digits of x [n_runs][cols] into planes (compact or fragment-major); a
// workgroup that meets a word needing more than three digits stores seq in
// *oflag.  The word is never cleared: a call passes a seq of its own.
int launch_digits_raw(const int64_t *x, uint32_t n_runs, uint32_t cols, int8_t *planes,
                      uint32_t kp, uint32_t bp, uint32_t compact, uint32_t *oflag, uint32_t seq,
                      void *stream);
size_t attention_lds_bytes(uint32_t max_npos, uint32_t head);
int kernels_init(uint32_t max_npos, uint32_t head);

}  // namespace fpi8
