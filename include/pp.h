/*
 * pp.h -- C ABI of the lockstep tick library (libpp.so) for MI355X (gfx950).
 *
 * One call of pp_step runs one 80 ms lockstep tick of a Moshi/PersonaPlex
 * RQ-Transformer for B concurrent session slots:
 *
 *   PersonaPlex recipe (vLLM-Omni), "Architecture (Moshi RQ-Transformer, all
 *   native)": a per-frame token column [B, 17, 1] (row 0 inner-monologue
 *   text, rows 1-8 agent audio, rows 9-16 user audio) goes through the
 *   temporal transformer (4096-d / 32 layers / 32 heads) decoding one frame
 *   against a ring KV cache with a 3000-frame sliding window and per-slot
 *   recycle; then the depformer (1024-d / 6 layers / 16 heads) runs
 *   autoregressively over 16 codebooks, reset each frame.  Each tick takes
 *   one user audio frame and gives one agent audio frame and one text token
 *   ("Why it is different from MiniCPM-o / JoyVL duplex").
 *
 *   vLLM-Omni PersonaPlex guide (mhpq.cn), "架构": RMSNorm with fp32 alpha,
 *   fused in-projection attention, interleaved RoPE at absolute positions,
 *   SiLU-gated MLP, fixed-capacity ring KV with static shapes so the whole
 *   step can be captured in a graph; "贪心解码与 Parity 约束": greedy only,
 *   one token per tick; "运维要点与注意事项": a recycled slot is bit-exact
 *   with a fresh engine for the same inputs.
 *
 * Conventions
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *   - Device pointers are plain HIP device addresses (for instance the
 *     data_ptr() of a torch tensor); host pointers are ordinary memory.
 *   - The caller allocates and owns every device buffer (weights, arena) and
 *     the stream; the library keeps raw pointers, so the buffers must stay
 *     alive until pp_destroy.  The library allocates no device memory; it
 *     allocates small pinned host staging buffers, one internal stream used
 *     to capture the tick's graphs, and one internal stream (default
 *     priority) that runs the user-stream half of the depformer (below).
 *   - Host arrays passed in are copied before the call returns.
 *   - A handle is single-threaded and bound to the stream given to pp_create.
 *   - Return codes: PP_OK, or a negative PP_E* code.  On every error except
 *     PP_EDEVICE no state changes (arguments are validated before anything
 *     is committed).  PP_EDEVICE means a HIP call failed; the handle is then
 *     poisoned and every later call returns PP_EDEVICE.  pp_last_error gives
 *     a message.  No C++ exception crosses this interface.
 */
#ifndef PP_H
#define PP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PP_OK       0
#define PP_EINVAL  (-1)  /* null pointer, bad dims, slot out of [0,B), token out of range, n > window */
#define PP_EBUSY   (-2)  /* prefill or fill on a slot that is already free-running (or fill after a prefill) */
#define PP_ENOSPC  (-3)  /* arena too small, or forced-frame queue full */
#define PP_EDEVICE (-4)  /* a HIP call failed; handle poisoned */

#define PP_MAX_BATCH     32    /* slots per handle */
#define PP_MAX_WINDOW    4096  /* ring frames per slot (the decode pass combines at most 16 splits of 256 keys) */
#define PP_MAX_QUEUE     4096  /* forced frames queued per slot */
#define PP_MAX_DELAY     4     /* acoustic delay, frames (pp_set_acoustic_delay) */
#define PP_COLUMN_ROWS   17    /* token column: text, 8 agent, 8 user */

/* Model shape.  Constraints (checked by pp_create / pp_arena_bytes):
 * n_q == 8, dep_q == 16, d % n_heads == 0 with head_dim in {32,64,128},
 * dep_d % dep_heads == 0 with head_dim in {32,64,128}, d, ffn, dep_d,
 * dep_ffn multiples of 32, text_card >= 2, audio_card >= 2. */
typedef struct pp_dims {
  int32_t d, n_layers, n_heads, ffn;   /* temporal transformer */
  int32_t text_card;                   /* text vocabulary (TEXT_INITIAL_TOKEN == text_card) */
  int32_t audio_card;                  /* codec cardinality (AUDIO_INITIAL_TOKEN == audio_card) */
  int32_t n_q;                         /* audio codebooks per stream in the column: 8 */
  int32_t dep_d, dep_layers, dep_heads, dep_ffn;
  int32_t dep_q;                       /* depformer codebooks per frame: 16 */
  float norm_eps;                      /* RMSNorm epsilon (inside the square root) */
  float rope_base;                     /* RoPE base; pair (2i,2i+1) turns by pos*base^(-2i/head_dim) */
} pp_dims;

/* Weights: device pointers, read-only, stacked per tensor kind.
 * L = n_layers, Ld = dep_layers, F = ffn, Fd = dep_ffn, A = audio_card,
 * Vt = text_card.  Tables and alphas are row-major.  Every matrix (y = W x,
 * W of M rows and K columns) is in the TILE LAYOUT produced by
 * pp_pack_matrix and occupies pp_packed_elems(M, K) elements; a stack of
 * matrices is those blocks back to back.  Tile layout: 16-row tiles, each
 * cut into K/32 steps of 32 columns; block (tile t, step s) is 512 elements
 * at offset (t*(K/32) + s)*512, in which element e of lane l (l < 64, e < 8)
 * is W[16t + l%16][32s + 8(l/16) + e]; rows past M are zero. */
typedef struct pp_weights {
  const uint16_t* emb_text;      /* [Vt+1][d]           table of column row 0 */
  const uint16_t* emb_audio;     /* [16][A+1][d]        tables of column rows 1..16 */
  const float*    attn_norm;     /* [L][d]              fp32 alpha */
  const uint16_t* wqkv;          /* L x [3d][d]         rows [q; k; v], heads contiguous */
  const uint16_t* wo;            /* L x [d][d] */
  const float*    mlp_norm;      /* [L][d] */
  const uint16_t* w_in;          /* L x [2F][d]         rows [gate; up] */
  const uint16_t* w_out;         /* L x [d][F] */
  const float*    out_norm;      /* [d] */
  const uint16_t* text_head;     /* [Vt][d] */
  const uint16_t* dep_in_proj;   /* [16*dep_d][d]       one projection per codebook step, stacked */
  const uint16_t* dep_emb_text;  /* [Vt+1][dep_d]       input table of step 0 */
  const uint16_t* dep_emb_audio; /* [15][A+1][dep_d]    input tables of steps 1..15 */
  const float*    dep_attn_norm; /* [Ld][dep_d] */
  const uint16_t* dep_wqkv;      /* Ld x [3dep_d][dep_d] */
  const uint16_t* dep_wo;        /* Ld x [dep_d][dep_d] */
  const float*    dep_mlp_norm;  /* [Ld][dep_d] */
  const uint16_t* dep_w_in;      /* Ld x [2Fd][dep_d] */
  const uint16_t* dep_w_out;     /* Ld x [dep_d][Fd] */
  const float*    dep_out_norm;  /* [dep_d] */
  const uint16_t* dep_heads;     /* 16 x [A][dep_d] */
} pp_weights;

/* Device views into the arena, valid after each pp_taps call (overwritten by
 * the next pp_step).  Strides are dense. */
typedef struct pp_taps_t {
  const float*   hidden;       /* [L+1][B][d]   embedding sum, then the residual stream after each layer */
  const float*   text_logits;  /* [B][Vt] */
  const float*   dep_logits;   /* [B][16][A] */
  const int32_t* tokens;       /* [B][32]: [0..8] predictions (text, agent 0..7),
                                  [9..16] user-stream predictions (depformer steps 8..15),
                                  [17..25] chosen tokens (forced where forced, else predicted) */
} pp_taps_t;

/* Sampling of the token choice (pp_set_sampling).  The guides' deployment
 * knobs: a sampling temperature of 0.7-0.8, a repetition penalty of about
 * 1.1 (the Korean Moshi guide's risk list), top_p 0.9 and a separate audio
 * temperature (the PersonaPlex configuration walkthrough); top-k as well. */
typedef struct pp_sampling {
  float text_temperature;   /* text row; 0 = greedy */
  float audio_temperature;  /* depformer codebooks 0-15; 0 = greedy */
  int   top_k;              /* 0 = off */
  float top_p;              /* (0, 1]; 1 = off */
  float repetition_penalty; /* >= 1 (1 = off), text row: the slot's last 64 chosen text tokens */
} pp_sampling;

typedef struct pp_handle pp_handle;

/* Elements of one [M][K] matrix in the tile layout: ceil(M/16)*16*K.
 * 0 if M < 1 or K is not a positive multiple of 32.  Pure host. */
size_t pp_packed_elems(int M, int K);

/* Repack a row-major bf16 matrix src [M][K] (device) into the tile layout at
 * dst (device, pp_packed_elems(M, K) elements, caller-allocated, must not
 * overlap src), asynchronously on `stream` (NULL = null stream).
 * PP_EINVAL on NULL pointers, M < 1, or K not a positive multiple of 32. */
int pp_pack_matrix(const uint16_t* src, int M, int K, uint16_t* dst, void* stream);

/* Bytes of device arena a handle needs for (dims, B, window).  Pure host
 * computation.  The arena holds the ring KV ([B][L][2][H][window][head_dim]
 * bf16), activations, taps and work buffers.  PP_EINVAL on bad arguments. */
int pp_arena_bytes(const pp_dims* dims, int B, int window, size_t* out_bytes);

/* Create a handle for B slots (1..PP_MAX_BATCH) and a ring of `window`
 * (1..PP_MAX_WINDOW) frames per slot.  arena: device buffer of at least pp_arena_bytes bytes,
 * 256-byte aligned.  stream: the hipStream_t every later call runs on (NULL =
 * the null stream).  Captures the tick graph.  All slots start reset.
 * PP_EINVAL (bad args), PP_ENOSPC (arena too small), PP_EDEVICE. */
int pp_create(const pp_dims* dims, int B, int window, const pp_weights* w,
              void* arena, size_t arena_bytes, void* stream, pp_handle** out);

/* Queue n forced frames (host int32 [n][17]) for `slot`, consumed one per
 * tick by the following pp_step calls (session open: voice codes force the
 * agent rows, persona tokens force the text row, silence frames between;
 * recipe "Architecture", guide "Persona Voice 注入").  Row layout: rows 0-8
 * are the token to choose for this tick's text / agent 0..7 output, or -1
 * for "use the greedy prediction"; rows 9-16 are this tick's user codes and
 * replace that slot's user_codes.  Ranges: row 0 in [-1,Vt), rows 1-8 in
 * [-1,A), rows 9-16 in [0,A).  Legal only before the slot's first
 * free-running tick (else PP_EBUSY, as persona/voice cannot change after
 * session open).  PP_ENOSPC if the queue would exceed PP_MAX_QUEUE.
 * With an acoustic delay D (pp_set_acoustic_delay) the frames are
 * frame-aligned: rows 1 and 9 (codebook 0) and row 0 act on their own tick,
 * rows 2-8 and 10-16 (codebooks 1-7) D ticks later. */
int pp_prefill_forced(pp_handle* h, int slot, const int32_t* frames, int n);

/* Queue n embedding-form prefill frames for `slot`, in the same queue as
 * pp_prefill_forced (recipe "Architecture": the prompt is assembled from
 * voice embedding rows, silence frames and persona-token embeddings; guide
 * "Persona Voice 注入").  x: host fp32 [n][d], the temporal input of each
 * frame's tick, which replaces the 17-row embedding gather-sum; it is copied
 * before the call returns.  force: host int32 [n][9] (rows as rows 0-8 of a
 * forced frame, -1 = free) or NULL for all free.  The frame gives no user
 * codes: with a delay, the user rows that would take them hold the initial
 * audio token.  Errors as pp_prefill_forced, and PP_EINVAL for a
 * non-finite input. */
int pp_prefill_embed(pp_handle* h, int slot, const float* x, const int32_t* force, int n);

/* One lockstep tick for all B slots.  user_codes: host int32 [B][8] in
 * [0,A) (ignored for slots consuming a forced frame).  tokens: host int32
 * [B][9] receives each slot's greedy predictions [text, agent 0..7] -- the
 * model's own predictions even on forced ticks.  Synchronous: returns after
 * the tokens are on the host.  A slot whose forced queue is empty at this
 * tick becomes free-running.  Every slot computes every tick.
 *
 * Pipelining: the depformer's user-stream codebooks (steps 8..15, which feed
 * only the taps, never the next column) are launched by the next pp_step, on
 * the library's internal stream, once that tick's temporal stack is done:
 * they run beside the next tick's agent codebooks, in a second set of
 * depformer buffers.  pp_taps, pp_time_kernel and pp_time_graph launch them
 * if still pending and wait for them; pp_destroy drops them.  The work and
 * its results are those of the plain sequence. */
int pp_step(pp_handle* h, const int32_t* user_codes, int32_t* tokens);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): the same tick as
 * pp_step, with the same arguments, errors and results, whose kernels keep
 * their work buffers (split-decode partials and tickets, large-batch GEMM
 * partials, per-launch inverse RMS) in an array of PP_STATIC_SCRATCH_BYTES
 * that the library holds on each GPU it runs on until the process ends,
 * instead of in the handle's arena.  Calls no allocation routine.  Every
 * call on one GPU shares that array and it keeps the last call's contents:
 * the tickets that must start at zero are cleared at the start of each tick,
 * and calls on one GPU that overlap in time (handles on different streams)
 * race.  pp_step and pp_step_static may be mixed on one handle.  PP_ENOSPC
 * if the handle's work buffers exceed PP_STATIC_SCRATCH_BYTES. */
#define PP_STATIC_SCRATCH_BYTES (64u << 20)
int pp_step_static(pp_handle* h, const int32_t* user_codes, int32_t* tokens);

/* Acoustic delay (recipe, interruption latency: an 80 ms frame plus an
 * 80 ms acoustic delay, i.e. D = 1 at 12.5 Hz): audio codebooks 1-7 of both
 * streams run D frames behind the text row and codebook 0.  user_codes (and
 * the user rows of forced frames) are frame-aligned: the column's row 9
 * takes this tick's codebook 0, rows 10-16 take codebooks 1-7 of the frame
 * given D ticks earlier (the initial audio token before the slot's first D
 * ticks).  Forced agent rows shift the same way.  The agent rows of the
 * column and the returned tokens stay per tick.  D in [0, PP_MAX_DELAY]
 * (PP_EINVAL); legal only while no slot has ticked since its reset
 * (PP_EBUSY).  Default 0. */
int pp_set_acoustic_delay(pp_handle* h, int frames);

/* Replace the greedy choice by sampling from the next tick on (NULL: back
 * to greedy, the default).  Per decision (one logits row): the repetition
 * penalty on the text row (a positive logit of a token among the slot's
 * last 64 chosen text tokens is divided by the penalty, a negative one
 * multiplied, each distinct token once); z = logit / T; top-k = the k first
 * of the order (z descending, index ascending); p = exp(z - max z) over the
 * kept entries; top-p = the shortest prefix of the order (p descending,
 * index ascending) whose sum reaches top_p of the total; the token = the
 * inverse CDF over the kept entries in index order at u times their sum.
 * u = Philox4x32-10 (Salmon et al., SC 2011) of counter (ticks since the
 * slot's reset as 64 bits, row, 0) and key (the slot's seed), first output
 * word >> 8, times 2^-24; row 0 is the text token, 1 + k codebook k.  The
 * sampled tokens are the model's own predictions (pp_step's tokens); forced
 * rows still override the choice.  PP_EINVAL for a negative or non-finite
 * temperature, top_k < 0, top_p outside (0, 1], a penalty below 1, or
 * logits rows wider than 32768.  Waits for the device work in flight. */
int pp_set_sampling(pp_handle* h, const pp_sampling* s);

/* The sampling seed of `slot` (default 0; kept across pp_slot_reset). */
int pp_slot_seed(pp_handle* h, int slot, uint64_t seed);

/* The agent audio frame completed by the last pp_step, per slot: frame
 * f = t - D gets codebook 0 chosen at tick f and codebooks 1-7 chosen at
 * tick t (chosen = forced where forced, else predicted).  frames: host
 * int32 [B][8]; valid: host int32 [B], 0 while the slot has ticked D times
 * or fewer since its reset (its row is then zeros). */
int pp_agent_frames(const pp_handle* h, int32_t* frames, int32_t* valid);

/* Recycle `slot`: position 0, column back to the initial tokens
 * [Vt, A x 8], forced queue cleared, ring logically empty.  A recycled slot
 * then computes bit-identically to a fresh handle fed the same inputs. */
int pp_slot_reset(pp_handle* h, int slot);

/* Test / measurement hook: set the ring of `slot` to n frames of given keys
 * and values at absolute positions 0..n-1 (host bf16 [L][n][H][head_dim]
 * each; the stored, already rotated values); the slot's next tick runs at
 * position n.  Legal only on a slot with no tick and no queued frame since
 * its last reset (else PP_EBUSY).  n in [0, window] (else PP_EINVAL). */
int pp_ring_fill(pp_handle* h, int slot, int n, const uint16_t* k, const uint16_t* v);

/* Device views of the last tick's intermediate results (see pp_taps_t).
 * Launches the tick's user-stream codebooks if still pending and waits for
 * them first. */
int pp_taps(const pp_handle* h, pp_taps_t* out);

/* Measurement hook: launch one kernel of the tick graph outside the graph,
 * on the handle's stream, with the arguments it has inside the graph, once
 * per layer in layer order (each launch streams that layer's own weights, as
 * in a tick), `iters` rounds; *avg_ms = mean duration of one launch from HIP
 * events.  which: 0 temporal fused QKV GEMM, 1 temporal attention (split-K
 * decode pass), 2 temporal out-projection, 3 temporal gate/up GEMM,
 * 4 temporal down projection, 5 text head (one launch per round).
 * *bytes = the algorithmic bytes of one launch (weights read, activations read
 * and written, keys/values read and written).  The launches recompute values
 * that the next tick recomputes before use, so slot state is not disturbed. */
int pp_time_kernel(pp_handle* h, int which, int iters, float* avg_ms, double* bytes);

/* Time `iters` back-to-back ticks (the graphs of each, pipelined as in
 * pp_step) with HIP events (no host copies); *avg_ms = mean device time per
 * tick, the last tick's user-stream codebooks included.  The
 * launches recompute the tick for the current tick inputs without advancing
 * any slot, so they leave slot state (positions, columns, queues) as is. */
int pp_time_graph(pp_handle* h, int iters, float* avg_ms);

/* Measurement hook: the depformer as one fused persistent launch per tick
 * (on = 1) or as per-layer kernel launches (on = 0, the default: the faster
 * of the two on MI355X at the 7B shape); both compute the same bits.  The fused loop applies to handles
 * of at most 2 slots with greedy choices and depformer dims it supports
 * (width <= 1024 and a multiple of 256, FFN a multiple of 256, heads
 * splitting evenly over 8 ranges); with sampling on, the per-layer launches
 * run.  PP_EINVAL for on = 1 where it cannot apply.  Waits for the device
 * work in flight and re-captures the tick's graphs. */
int pp_set_depformer_loop(pp_handle* h, int on);

/* 1 if the handle's ticks run the fused depformer loop, 0 if not (or a
 * negative PP_E* code). */
int pp_depformer_loop_active(const pp_handle* h);

/* Waits for the handle's device work, then frees its host resources. */
void pp_destroy(pp_handle* h);

/* Message of the last error on h (or of the last failed pp_create when h is
 * NULL).  Valid until the next call on h. */
const char* pp_last_error(const pp_handle* h);

#ifdef __cplusplus
}
#endif
#endif /* PP_H */
