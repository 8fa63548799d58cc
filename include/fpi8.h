/*
 * fpi8.h - C ABI of libfpi8, the MI355X (gfx950) implementation of the
 * fixed-point transformer forward pass of the curta-core inference core
 * ("The inference core" page: sections "Fixed-point arithmetic", "A matrix
 * row", "RMS normalization", "The attention cache", "Lookup tables", "The
 * forward pass, in order", "Attention, stage by stage", "The resumable
 * state", "Sampling", "The Rust API", "WebAssembly exports", "Core errors").
 *
 * Conventions (after the page's WebAssembly exports): plain C functions,
 * pointers and 64-bit lengths, the configuration as seven u32 values in the
 * order dim, hidden, layers, heads, kv_heads, vocab, context.  Every
 * function returns 0 on success or one of the page's core error numbers
 * (1-8); numbers from 100 up are failures of the GPU runtime.  Pointers named
 * d_* are device memory, h_* and the rest host memory; the caller owns all
 * of it, and the library only borrows a pointer for the length of a call
 * (an engine keeps d_blob until it is destroyed).  A stream argument is a
 * hipStream_t passed as void* (NULL: the default stream).
 *
 * Token ids are fed in: the tokenizer phases 0-2 stay with the caller.
 */
#ifndef FPI8_H
#define FPI8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* "Core errors". */
enum {
  FPI8_OK = 0,
  FPI8_INVALID_CONFIG = 1,    /* a configuration value out of range */
  FPI8_INVALID_FORMAT = 2,    /* artifact tag, counts, offsets or descriptors */
  FPI8_INVALID_STATE = 3,     /* state tag, size, alignment, cursor, frozen */
  FPI8_BUFFER_TOO_SMALL = 4,  /* init_state given a length other than state_size */
  FPI8_MISSING_WEIGHTS = 5,   /* a matrix section absent or shorter than its matrix */
  FPI8_INVALID_PROMPT = 6,    /* no ids, an id >= vocab, max tokens 0 or > context,
                                 temperature above 16 (1,048,576 at Q16) */
  FPI8_CONTEXT_EXCEEDED = 7,  /* ids + max tokens - 1 above the context */
  FPI8_ARITHMETIC = 8,        /* a key or value that does not fit 32 bits */
  FPI8_ERR_HIP = 100,         /* a HIP runtime call failed */
  FPI8_ERR_UNSUPPORTED = 101, /* a shape the kernels cannot run (see engine_create) */
  FPI8_ERR_ARGUMENT = 102     /* a null pointer or a count beyond the engine's limits */
};

/* The cursor of a state ("The Rust API", StateInfo::read). */
typedef struct {
  uint32_t phase;           /* 3 at the start of a position, 20 when complete; on an
                               Arithmetic failure the phase that failed (6, 7 or 8) */
  uint32_t layer;           /* 0, or the failing layer */
  uint32_t position;        /* positions computed so far */
  uint32_t token;           /* the token the next position embeds */
  uint32_t n_ids, max_tokens, temperature_q16, generated;
  uint32_t cache_positions; /* n_ids + max_tokens - 1 */
  uint32_t error;           /* 0, or 8 once the run froze */
  uint32_t complete;        /* phase == 20 */
  uint32_t reserved;
  uint64_t generator;       /* xorshift64* state */
  uint64_t turns;           /* turns run on this state */
} fpi8_info;

/* ---- The artifact ----------------------------------------------------------
 * Little-endian, offsets from the artifact's start.  Section zero begins at
 * offset 0 and holds: tag "CURTAW01" (8 bytes); the configuration u32[7] at
 * 8; u32 section count at 36; u32 matrix count (2 + 7*layers) at 40; u32 one
 * over the square root of the head size (Q24) at 44; u64 offsets of the
 * exponential table u32[4097] Q30 (48), the SiLU table i32[4097] Q16 (56),
 * rotary cosines i32[context][head/2] Q24 (64), sines (72), normalization
 * weights i32 Q24 [layers][2][dim] then [dim] (80), the tokenizer block (88)
 * and its length (96), and the matrix descriptors (104); the section table
 * at 128, {u64 offset, u64 length} per section, entry 0 being {0, length of
 * section zero}.  A descriptor is 32 bytes: u32 kind, layer, rows, cols,
 * section, 0, then u64 offset inside the section of rows*cols weight bytes
 * (weight + 128, row-major), followed 8-aligned by rows u32 Q24 scales.
 * Kinds: 0 embedding [vocab][dim], 1 query, 2 key [kv_dim][dim], 3 value,
 * 4 attention output [dim][dim], 5 gate [hidden][dim], 6 up, 7 down
 * [dim][hidden], 8 classifier [vocab][dim].                                */

/* ---- The tokenizer (host) --------------------------------------------------
 * Section zero may hold a tokenizer block at the header's offset 88, of the
 * length at 96 (0: none): u32 n (the vocabulary size, at least 259), u32 the
 * longest token in bytes, u32 score[n] (the higher merges first), u32
 * start[n + 1] (token i is pool[start[i], start[i + 1]), 1 to 128 bytes),
 * u32 sorted_ids[n] (ids in increasing byte order of their strings, a prefix
 * first, no string twice), then the pool.  Ids 0, 1, 2 are the unknown,
 * opening and closing tokens and 3 + b the byte b, written <0xXX>.  A block
 * that breaks these rules makes the artifact invalid (error 2). */

/* Phases 0 to 2 ("The forward pass, in order"): the token ids of a prompt of
 * prompt_len bytes (UTF-8, no zero byte, at most 1,024): token 1, then the
 * token of a single space when the prompt has text; then each character (a
 * lead byte and up to three continuation bytes) looked up whole, else one
 * token per byte, id byte + 3; then, until no adjacent pair's joined string
 * is a token, the pair whose token scores highest (the leftmost among
 * equals) replaced by that token.  h_section0 is section zero of the
 * artifact in host memory (or the whole artifact).  Writes *n_ids (also
 * when ids is too small: error 4) and the ids.  Errors: 2 (no tokenizer or
 * an invalid artifact), 6 (the prompt or max_tokens out of range), 7 (the
 * ids and max_tokens do not fit the context), 4. */
int32_t fpi8_tokenize(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *prompt,
                      uint32_t prompt_len, uint32_t max_tokens, uint32_t *ids, uint32_t capacity,
                      uint32_t *n_ids);

/* The text a generated token adds after the token prev ("Sampling", last
 * paragraph): its bytes, a leading space dropped right after the opening
 * token, a byte token <0xXX> (two hexadecimal digits) written as that byte,
 * and nothing for tokens 1 and 2.  Writes *len (also when out is too small:
 * error 4).  Errors: 2, 6 (an id out of the vocabulary), 4. */
int32_t fpi8_token_text(const uint8_t *h_section0, uint64_t section0_len, uint32_t prev,
                        uint32_t token, uint8_t *out, uint32_t capacity, uint32_t *len);

/* The text of a state's generated tokens ("The Rust API", output_text): each
 * token's text as fpi8_token_text gives it, the first one after the
 * prompt's last id.  state is a host copy of a run's state.  Writes *len
 * (also when out is too small: error 4).  Errors: 2, 3 (not a state), 6, 4. */
int32_t fpi8_output_text(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *state,
                         uint64_t state_len, uint8_t *out, uint64_t capacity, uint64_t *len);

/* ---- The page's own state format (host) ------------------------------------
 * "The resumable state" lays a run's state out as a header tagged CURTAST2
 * and the buffers prompt bytes, prompt tokens (prompt bytes + 2), output
 * tokens, output text (max tokens x 128), x and three working vectors, gate
 * and up, logits, scores and the key and value caches, with cache positions
 * min(prompt bytes + max tokens + 1, context).  Readings: its caches are
 * [layer][position][kv head * head + element]; after tokenizing, its
 * tokenizer's next byte is the prompt's length and the other tokenizer
 * fields are zero. */

/* The size of a state in the page's format (UINT64_MAX out of range; the
 * page's run account adds a 256-byte header to it). */
uint64_t fpi8_pages_state_size(const uint32_t cfg[7], uint32_t prompt_bytes, uint32_t max_tokens);

/* Writes a host copy of a run's state in the page's format: the prompt's
 * bytes (those its ids came from) and the generated tokens' text (the
 * artifact's tokenizer, as fpi8_output_text) are added, the cache reordered
 * and widened.  out_len must be fpi8_pages_state_size.  Errors: 2 (no
 * tokenizer), 3 (not a state, or a frozen run: the page's state has no
 * error field), 6 (prompt too long or fewer bytes than the ids need), 4. */
int32_t fpi8_state_export(const uint8_t *h_section0, uint64_t section0_len, const uint8_t *state,
                          uint64_t state_len, const uint8_t *prompt, uint32_t prompt_len,
                          uint8_t *out, uint64_t out_len);

/* Reads a state in the page's format (after tokenizing: phase 3 to 20)
 * into this library's format; state_len must be fpi8_state_size for the
 * prompt-token count and max tokens in its header (offsets 32 and 36), and
 * state 8-byte aligned.  Errors: 1, 3, 4. */
int32_t fpi8_state_import(const uint32_t cfg[7], const uint8_t *pages, uint64_t pages_len,
                          uint8_t *state, uint64_t state_len);

/* Writes a fresh state in the page's format before tokenizing (phase 0;
 * "The Rust API", init_state): the prompt's bytes, max tokens, the
 * temperature and the seed (zero becomes 0x9E3779B97F4A7C15) in a host
 * buffer of exactly fpi8_pages_state_size bytes.  The prompt has at most
 * 1,024 bytes and no zero byte; max tokens lies in 1 to the context; the
 * temperature is at most 16 (Q16).  Errors 1, 6, 4 in that order. */
int32_t fpi8_pages_init(const uint32_t cfg[7], const uint8_t *prompt, uint32_t prompt_len,
                        uint32_t max_tokens, uint32_t temperature_q16, uint64_t seed, uint8_t *out,
                        uint64_t out_len);

/* Runs up to max_units units of phases 0 to 2 ("The forward pass, in
 * order") on a host state in the page's format, in place, with the
 * header's tokenizer fields (offsets 52 to 68) as the cursor, so it can
 * stop after any unit and go on in a later call.  A unit is phase 0; one
 * prompt character, or the step that ends phase 1; one pair looked up in a
 * merge scan, or the scan's end (apply its best merge, or check the context
 * and move to phase 3 at position 0).  It stops at phase 3; the state then
 * goes to fpi8_state_import.  *units_done (may be NULL) receives the units
 * run.  Errors: 2 (no tokenizer), 3 (not a page state, past tokenizing, or
 * a cursor out of range), 7 (the prompt's tokens and max tokens, less one,
 * exceed the context: the state is left at the scan's end). */
int32_t fpi8_pages_tokenize(const uint8_t *h_section0, uint64_t section0_len, uint8_t *pages,
                            uint64_t pages_len, uint64_t max_units, uint64_t *units_done);

/* The compute units the page's turn planner charges for the phases of one
 * position ("The turn planner", "Compute costs"), summed over layers, with
 * every chunk whole and its 160 units included: out[phase - 3] for phases 3
 * to 19.  position counts from 0 (the attention stages see position + 1
 * positions); generating selects phases 17 to 19; above temperature zero
 * sampling is three passes.  Not included: the 18,000 units of each turn,
 * and the setup and 160 units charged again where a turn boundary splits a
 * chunk.  Errors: 1, 6 (position at or past the context, temperature above
 * 16), 4 (out NULL). */
int32_t fpi8_position_charges(const uint32_t cfg[7], uint32_t position, int32_t generating,
                              uint32_t temperature_q16, uint64_t out[17]);

/* Checks a whole artifact held in host memory: 0, 1, 2 or 5.  cfg_out
 * (may be NULL) receives the configuration. */
int32_t fpi8_blob_check(const uint8_t *blob, uint64_t len, uint32_t cfg_out[7]);

/* ---- The state ("The resumable state") -----------------------------------
 * A 128-byte header tagged "FPI8ST01" (u32 phase 8, layer 12, row 16,
 * position 20, token 24, error 28, n_ids 32, max tokens 36, temperature 40,
 * generated 44, cache positions 48; u64 generator 72, turns 80; the other
 * words are zero at position boundaries), then 8-aligned buffers: ids
 * u32[n_ids], output tokens u32[max], activations and three working vectors
 * i64[dim], gate and up i64[hidden], logits i64[vocab], scores
 * i64[cache positions], keys and values i32[layers][kv_heads][cache
 * positions][head].                                                         */

/* Size of a state; UINT64_MAX for parameters out of range. */
uint64_t fpi8_state_size(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens);

/* Byte offsets of the buffers: ids, out, x, w1, w2, w3, gate, up, logits,
 * scores, keys, values, total size.  0, 1 or 6. */
int32_t fpi8_state_offsets(const uint32_t cfg[7], uint32_t n_ids, uint32_t max_tokens,
                           uint64_t out[13]);

/* Writes a fresh state into a host buffer of exactly fpi8_state_size bytes,
 * 8-byte aligned ("The Rust API", init_state).  A zero seed starts the
 * generator at 0x9E3779B97F4A7C15.  Errors 1, 6, 7, 4, 3 in that order. */
int32_t fpi8_init_state(const uint32_t cfg[7], uint8_t *state, uint64_t state_len,
                        const uint32_t *ids, uint32_t n_ids, uint32_t max_tokens,
                        uint32_t temperature_q16, uint64_t seed);

/* Reads the cursor of a host copy of a state: 0 or 3. */
int32_t fpi8_state_info(const uint8_t *state, uint64_t len, fpi8_info *out);

/* The generated ids of a host copy of a state (count receives how many);
 * NULL for an invalid state. */
const uint32_t *fpi8_output_tokens(const uint8_t *state, uint64_t len, uint32_t *count);

/* ---- The GPU engine ---------------------------------------------------- */

typedef struct fpi8_engine fpi8_engine;

/* Binds an artifact already in device memory.  h_section0 is a host copy of
 * its section zero (at least the length the section table names), d_blob
 * the whole artifact on the device, blob_len its length; max_runs bounds the
 * runs of one turn.  Errors 1, 2, 5; 101 when the context is too long for
 * the attention kernel's on-chip score buffer; 100 on a HIP failure. The
 * engine allocates its own workspace here, once, with a copy of every
 * matrix but the embedding repacked into the tiles its matrix-row kernels
 * load (about the artifact's size in device memory). */
int32_t fpi8_engine_create(const uint8_t *h_section0, uint64_t section0_len,
                           const uint8_t *d_blob, uint64_t blob_len, uint32_t max_runs,
                           fpi8_engine **out);

void fpi8_engine_destroy(fpi8_engine *engine);

/* Advances every run of a batch by up to max_positions whole positions
 * (phases 3-16 per layer, then 17-19 where a token is generated; "The forward
 * pass, in order").  d_states holds n_runs states at a fixed byte stride
 * (multiple of 8; each state no larger than the stride), written by
 * fpi8_init_state and copied to the device.  A state may also stand inside a
 * position ("The resumable state": the header's phase 3-19 and, for phases
 * 4-16, its layer), between two phases or inside one (the next row of a
 * matrix; the head, stage and index of attention; the pass and next entry of
 * sampling, with the largest score, chosen entry, sum and remainder), as a
 * turn that stops after any unit of work leaves it: the first position then
 * finishes from there, counted as one of max_positions, and the run's words
 * end as they would have without the stop.  A cursor no such turn can leave
 * is an invalid state (error 3).  Runs are
 * independent: a run that completes stops, others go on.  A run that is already complete is left
 * as it is (error 0); an invalid or frozen state gets error 3; a key or
 * value that does not fit 32 bits freezes the run with error 8, its cursor at
 * the failing phase and layer.  h_run_errors (may be NULL) receives one code
 * per run; the return value is the first nonzero of them, or a 100+ code.
 * Synchronizes the stream before returning. */
int32_t fpi8_turn(fpi8_engine *engine, uint8_t *d_states, uint64_t state_stride,
                  uint32_t n_runs, uint32_t max_positions, void *stream,
                  int32_t *h_run_errors);

/* Queued turns: turns that a caller can issue back to back on a stream
 * without waiting ("The Rust API", turn, over a batch of runs).
 * fpi8_turn_bind reads every run's header once (it synchronizes the
 * stream), checks it as fpi8_turn does (per-run errors into h_run_errors,
 * may be NULL; returns the first) and keeps the batch's run descriptors on
 * the device.  Each fpi8_turn_async then advances every run of the bound
 * batch by up to max_positions whole positions (the first one, after a
 * bind at a cursor inside a position, finished from there) with launches
 * only: no host transfer and no synchronization.  When d_run_errors
 * (device, n_runs int32) is not NULL, the per-run error numbers as they
 * stand after the turn's launches are copied there, on the stream.  Returns
 * 102 when no batch is bound, 100 on a launch failure, else 0.  A batch
 * stays bound until the next fpi8_turn_bind or a turn of any other kind on
 * this engine; the states must not be changed in between except by queued
 * turns. */
int32_t fpi8_turn_bind(fpi8_engine *engine, uint8_t *d_states, uint64_t state_stride, uint32_t n_runs,
                       void *stream, int32_t *h_run_errors);
int32_t fpi8_turn_async(fpi8_engine *engine, uint32_t max_positions, void *stream, int32_t *d_run_errors);

/* A turn of at most max_phases phases of each run (counted as "The forward
 * pass, in order" lists them: 3, 4-16 per layer, 17-19 where a token is
 * generated), as many positions as they reach.  Each run stops at the last
 * point within its budget where the engine's launches meet: a boundary
 * between two phases, except the one inside phase 11 (so before phase 4, 5,
 * 9, 10, 12, 15 or 17-19, or a position's start).  A run that cannot reach
 * such a point is left as it is.  The state it stops in holds what the
 * oracle's state holds at the same cursor, and a later turn of either
 * continues it.  Errors, arguments and synchronization as fpi8_turn;
 * max_phases 4294967295 counts as 4294967294. */
int32_t fpi8_turn_phases(fpi8_engine *engine, uint8_t *d_states, uint64_t state_stride,
                         uint32_t n_runs, uint32_t max_phases, void *stream,
                         int32_t *h_run_errors);

/* A turn of at most max_units units of work of each run, counted as "The
 * resumable state" cuts the pass: a row of a matrix, a position or output
 * element of an attention stage, a vocabulary entry of a sampling pass, or a
 * phase that is one vector operation.  Each run stops exactly where its
 * budget ends, inside a phase if it ends there, and its state holds what
 * the oracle's turn of the same units leaves: the rows done, the attention
 * head's stage values, the sampling pass's running maximum, choice, sum and
 * remainder, and the cursor.  Positions where a run starts or stops inside
 * run their launches one by one.  Errors, arguments and synchronization as
 * fpi8_turn; max_units 2^64 - 1 counts as 2^64 - 2. */
int32_t fpi8_turn_units(fpi8_engine *engine, uint8_t *d_states, uint64_t state_stride,
                        uint32_t n_runs, uint64_t max_units, void *stream,
                        int32_t *h_run_errors);

/* Which matrix-row kernel the engine's launches use: 0 the planner's choice
 * (the default), 1 always the kernel whose four waves split the contraction,
 * 2 the kernel whose waves share their runs' digits through LDS wherever it
 * can run (columns a multiple of 128, 16-byte aligned rows), 3 that kernel
 * with three of its four waves owning rows and the fourth only staging
 * digits, 4, 5 and 6 that kernel with 3, 6 or 12 waves (16, 32 or 64 runs
 * per workgroup), every one owning rows, one block of digits per stage
 * (where a launch has no such shape, the gate/up pair under 6, the
 * planner's choice), 7 the default choice with the multi-wave shapes the
 * default gives query/key/value, gate/up and classifier launches from 2048
 * columns on taken at every width.  Results are identical under every
 * setting; it exists for tests and tuning.  Error 102 for another value. */
int32_t fpi8_engine_set_row_kernel(fpi8_engine *engine, int32_t kind);

/* Whether a turn replays one position recorded as a HIP graph (nonzero, the
 * default) or launches every kernel of every position itself (0, also the
 * case while kernel timing is on).  Results are identical either way. */
int32_t fpi8_engine_set_graph(fpi8_engine *engine, int32_t enable);

/* How a turn spreads a batch over streams: 0 (the default) or 1 one stream;
 * 2 the runs split in two groups, each advanced by its own launch sequence
 * on its own stream (the caller's and one of the engine's), so one group's
 * matrix rows can overlap the other's attention.  Results are identical
 * under every setting.  Error 102 for another value. */
int32_t fpi8_engine_set_streams(fpi8_engine *engine, int32_t streams);

/* Kernel timing for measurement: while enabled, every launch of the kernel
 * class `kernel` is bracketed by HIP events on its stream.  Classes: 0 row
 * kernel (all matrices), 1 attention, 2 normalization, 3 sampling, 4 embedding.
 * fpi8_engine_timing returns the summed milliseconds and the launch count
 * since the last enable (it synchronizes on the recorded events). */
int32_t fpi8_engine_set_timing(fpi8_engine *engine, int32_t kernel, int32_t enable);
int32_t fpi8_engine_timing(fpi8_engine *engine, int32_t kernel, double *total_ms,
                           uint64_t *launches);

/* ---- The standalone matrix row ("A matrix row") ------------------------
 * y[b][r] = ((sum_c W[r][c] * x[b][c] - 128 * sum_c x[b][c]) * scale[r]) >> 24
 * in wrapping 64-bit arithmetic, for W rows x cols bytes (weight + 128,
 * row-major), scale u32 Q24, x [batch][cols] i64 Q16, y [batch][rows] i64.
 * x and y must be 8-byte aligned.  The workspace (device, 256-byte aligned, at
 * least fpi8_matrix_rows_workspace_size bytes) holds the byte digits of x
 * and an overflow word; its contents need no initialization, and a call of
 * one or two inputs over at most 16,384 columns (32,768 for one) may leave
 * it untouched, splitting x inside the row kernel.  Calls that share a
 * workspace must not overlap.  Runs on `stream` (the null stream if NULL)
 * and does not synchronize.  Errors 102 (sizes, null pointers, small or
 * misaligned workspace), 100. */
uint64_t fpi8_matrix_rows_workspace_size(uint32_t rows, uint32_t cols, uint32_t batch);
int32_t fpi8_matrix_rows(const uint8_t *d_W, const uint32_t *d_scale, uint32_t rows,
                         uint32_t cols, const int64_t *d_x, uint32_t batch, int64_t *d_y,
                         void *d_work, uint64_t work_len, void *stream);

/* ---- The turn planner ("The turn planner", "Compute costs") -----------
 * A turn is charged 18,000 compute units, then chunks of work (each 160 plus
 * its own charges from "Compute costs"), until the next chunk does not fit
 * what is left of 1,350,000, or needs a third matrix section, or the run is
 * complete (max tokens; a stop token ends a run sooner than planned).  A
 * chunk is a run of rows of one matrix, of units of one attention stage of
 * one head, of vocabulary entries of one sampling pass, or one whole vector
 * operation; it takes as many units as fit.  Units are those of
 * fpi8_turn_units, so the planned turn of a state runs as
 * fpi8_turn_units(..., plan.units, ...).  Readings where the page is
 * silent: the 18,000 count against the 1,350,000; a chunk continuing an
 * item from an earlier turn pays its setup and 160 again; the chunk that
 * ends a sampling pass carries its 4,000; matrix chunks and the embedding
 * need their matrix's section (the artifact's matrix descriptors), all else
 * section zero alone; above temperature zero three passes, each ending with
 * the 4,000, and a turn ends with the chunk that ends a draw pass: the draw
 * stops at the entry its remainder falls inside, known only when it runs,
 * so the plan charges every entry left (an upper bound), counts them in
 * units and sets ends_with_draw; such a turn runs as fpi8_turn(..., 1, ...)
 * (which finishes the position), every other one as a turn of its units.
 *
 * fpi8_plan_turn plans the next turn of the run in h_state (host copy of a
 * state, 8-byte aligned) over an artifact whose section zero is
 * h_section_zero: the compute units charged, the matrix sections read in
 * the order reached (section zero left out), the most tokens it completes
 * and the units of work it runs.  A complete run gives an all-zero plan.
 * fpi8_quote_turns counts the turns the run takes from its cursor to max
 * tokens.  Errors: 2 (section zero unreadable), 3 (bad state), 4 (a null
 * pointer), 1 (a single unit of work larger than a turn). */
typedef struct {
  uint32_t sections[2];
  uint32_t section_count;
  uint32_t estimated_cu;
  uint32_t max_generated;
  uint32_t ends_with_draw;  /* 1: the turn ends with a draw pass (see above) */
  uint64_t units;
} fpi8_turn_plan;
int32_t fpi8_plan_turn(const uint8_t *h_section_zero, uint64_t section_zero_len, const uint8_t *h_state,
                       uint64_t state_len, fpi8_turn_plan *out);
int32_t fpi8_quote_turns(const uint8_t *h_section_zero, uint64_t section_zero_len, const uint8_t *h_state,
                         uint64_t state_len, uint64_t *turns);

/* Timing of the standalone row for measurement: while enabled, the
 * row-kernel launch of every fpi8_matrix_rows / fpi8_matrix_rows_packed call
 * (not the launch that splits the inputs into digits) is bracketed by HIP
 * events on the call's stream.  fpi8_matrix_rows_timing returns the summed
 * milliseconds and the launch count since the last enable (it synchronizes
 * on the recorded events).  Not for calls made from several threads at
 * once while enabled. */
int32_t fpi8_matrix_rows_set_timing(int32_t enable);
int32_t fpi8_matrix_rows_timing(double *total_ms, uint64_t *launches);

/* Which arithmetic the standalone row uses over a packed matrix of many rows
 * ("A matrix row"; the same words either way): 0 (the default) and 1 the
 * int8 matrix cores, three signed byte digits of each input word; 2 the
 * vector ALU (v_dot4_i32_i8 over the same digits) for calls it applies to:
 * a packed matrix that takes the streaming kernel (at least 256 rows per
 * compute unit, columns filling a multiple of 8 blocks of 64), 1 to 4
 * inputs, and digits that fit 144 KB of LDS (3 bytes per input and column
 * rounded up to 512: 49,152 columns for one input, 12,288 for four).
 * Other calls run as under
 * 0.  For measuring one arithmetic against the other: on MI355X the matrix
 * cores stream closer to the HBM roof at every batch.  Process-wide, like
 * the timing switch.  Error 102 for another value. */
int32_t fpi8_matrix_rows_set_path(int32_t path);

/* The same matrix prepared once for many calls: its bytes packed into tiles
 * of 16 rows x 64 columns (bytes past the last row or column are 128, the
 * weight 0), the operand layout the matrix cores read, so that every load of
 * the row kernel fetches whole cache lines.  fpi8_matrix_packed_size gives
 * the bytes of the packed copy (UINT64_MAX for sizes out of range);
 * fpi8_matrix_pack writes it from d_W into d_P (device, 16-byte aligned);
 * fpi8_matrix_rows_packed is fpi8_matrix_rows reading d_P instead of d_W,
 * with the same result, workspace and errors. */
uint64_t fpi8_matrix_packed_size(uint32_t rows, uint32_t cols);
int32_t fpi8_matrix_pack(const uint8_t *d_W, uint32_t rows, uint32_t cols, uint8_t *d_P,
                         uint64_t p_len, void *stream);
int32_t fpi8_matrix_rows_packed(const uint8_t *d_P, const uint32_t *d_scale, uint32_t rows,
                                uint32_t cols, const int64_t *d_x, uint32_t batch, int64_t *d_y,
                                void *d_work, uint64_t work_len, void *stream);

/* ---- The standalone row for callers that cannot allocate ---------------
 * For code that may not call hipMalloc: work under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The same call as
 * fpi8_matrix_rows_packed, with the same result and errors, but its
 * workspace is a device array the library holds for each GPU (taken the
 * first time the call runs with that GPU current, kept until the process
 * ends), so the call allocates nothing.  Limits: at most
 * FPI8_NOALLOC_MAX_BATCH inputs of at most FPI8_NOALLOC_MAX_COLS columns
 * (the array is FPI8_NOALLOC_WORKSPACE_BYTES); beyond them error 102.  All
 * calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must not be made.
 * Runs on `stream` (the null stream if NULL) and does not synchronize. */
#define FPI8_NOALLOC_MAX_BATCH 128u
#define FPI8_NOALLOC_MAX_COLS 16384u
#define FPI8_NOALLOC_WORKSPACE_BYTES (256u + 3u * 128u * 16384u)
int32_t fpi8_matrix_rows_packed_noalloc(const uint8_t *d_P, const uint32_t *d_scale, uint32_t rows,
                                        uint32_t cols, const int64_t *d_x, uint32_t batch,
                                        int64_t *d_y, void *stream);

#ifdef __cplusplus
}
#endif
#endif
