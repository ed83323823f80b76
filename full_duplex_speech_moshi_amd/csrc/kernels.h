// Kernel launchers of the lockstep tick (gfx950).  Internal to libpp.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pp {

typedef uint16_t bf16_t;

// Per-tick device input, int32 [B][TI_STRIDE].
enum {
  TI_POS = 0,        // absolute position of this tick
  TI_COL = 1,        // 17 column rows: [1..9] previous chosen text+agent, [10..17] user codes
  TI_FORCE = 18,     // 9 forced choices for text, agent 0..7 (-1 = free)
  TI_XIN = 27,       // 1: the temporal input is the given row of EmbedArgs::xin, not the gather-sum
  TI_SEED = 28,      // 2: the slot's sampling seed (low, high word)
  TI_TICK = 30,      // 2: ticks since the slot's reset (low, high word)
  TI_STRIDE = 32
};

// Per-tick device output, int32 [B][TO_STRIDE].
enum {
  TO_PRED = 0,       // 9: text, agent 0..7 predictions
  TO_USER = 9,       // 8: depformer steps 8..15 predictions
  TO_CHOSEN = 17,    // 9: chosen text, agent 0..7
  TO_ERR = 26,       // slot 0's row: a fused depformer loop's error code (DL_ERR_*), else 0
  TO_STRIDE = 32
};

constexpr int ROWS = 16;           // MFMA row tile
constexpr int GEMM_WAVES = 8;      // waves per GEMM workgroup (split K)
constexpr int ATT_CHUNK = 256;     // keys per split of the flash-decoding pass
constexpr int ATT_MAX_SPLITS = 16; // splits per (slot, head): windows up to 4096 keys
constexpr int MAX_COLS = 32;       // slots per launch (two 16-wide column tiles)

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_GATED = 2, EPI_LOGITS = 3, EPI_STORE = 4 };

// Depformer attention of one codebook step: slot b, head h attends to the
// keys of steps 0..n_keys-1 of its own frame (n_keys <= DEP_MAX_KEYS).
constexpr int DEP_MAX_KEYS = 16;
constexpr int DEP_FUSE_B = 2;     // up to this batch the attention runs inside the out-projection
constexpr int DEP_FUSE_D = 1024;  // ... when the depformer width is at most this
struct DepAttnArgs {
  const float* q; int ldq;          // [B][ldq] fp32, head h at q + h*head_dim
  const bf16_t* kv;                 // per-frame cache of this layer: slot b at kv + b*slot_stride, V at +v_off
  long slot_stride, v_off;
  int n_heads, head_dim, window, n_keys, B;
  bf16_t* o; int ldo; long o_lo;    // [B][ldo] output as a bf16 hi/lo pair (standalone kernel)
};
void launch_dep_attention(const DepAttnArgs& a, hipStream_t s);

// Sampling of the token choice (device copy, set by pp_set_sampling).
struct SampleParams {
  int enabled;
  float t_text, t_audio;  // temperatures; 0 = greedy for that row
  int top_k;              // 0 = off
  float top_p;            // 1 = off
  float rho;              // repetition penalty on the text row; 1 = off
  int pad[2];
};
constexpr int SAMPLE_REP = 64;       // chosen text tokens the penalty looks back over
constexpr int SAMPLE_MAX_N = 32768;  // widest logits row that can be sampled (LDS)

struct FinishArgs {
  int B, step;          // step -1: text head; 0..dep_q-1: depformer codebook step
  int n_part;           // argmax partials per slot
  const float* amax_v; const int* amax_i; int ld_amax;
  const int* ti; int* to;
  // next depformer input (step + 1 < dep_q)
  int dep_q, dd;
  const float* u;        // [B][dep_q][dd] input projections of z
  const bf16_t* table;   // input table of step+1 ([rows][dd])
  const float* alpha;    // first depformer attention-norm alpha
  float* y; bf16_t* ya; long ya_lo; float* part;
  // sampling (sp->enabled): the row's full logits, the text row's recent
  // chosen tokens [B][SAMPLE_REP] (-1 empty), and each slot's (seed, tick)
  // [B][4]: written by the text finisher from the tick input, read by the
  // codebook finishers (which may run after the next tick input is in place)
  const SampleParams* sp;
  const float* logits; long ld_logits; int n_logits;
  const int* rep;
  unsigned* sctx;
};

struct GemmArgs {
  const bf16_t* W;      // [M][K] in the tile layout (gated: gate rows, up rows from row gate_off)
  int w_keep;           // W is re-read within the tick: load it cacheable (else non-temporal)
  int slot_grp;         // slots per workgroup of gemm_group_kernel (set by the launcher)
  int qkv_to_attn;      // EPI_QKV on the large-batch path: partials stored slot-major and no reduce
                        // launch; the decode pass finishes q, k and v (AttnArgs::qkv_part)
  const bf16_t* X;      // activations as a bf16 pair: hi plane [B][ldx], lo plane at X + x_lo
  long x_lo;
  int M, K, ldx, B;
  long gate_off;        // gated: row offset of the up half
  // inverse-RMS source: sum-of-squares partials [B][n_part] (one per 16 features)
  const float* part_in; int n_part; int feat; float eps;
  // EPI_QKV
  float* q_out;         // [B][ldq] fp32 (rotated queries)
  int ldq;
  bf16_t* kv;           // ring base for this layer: slot b at kv + b*kv_slot_stride; K at +0, V at +kv_v_off
  long kv_slot_stride, kv_v_off;
  int n_heads, head_dim, window;
  const int* ti;        // tick input (positions) or null
  int pos_const;        // position when ti == null
  const double* inv_freq; // [head_dim/2] or null (no rotation)
  const float* rope;      // [B][head_dim]: (cos, sin) of each frequency at the slot's position, or null
  // EPI_RESID
  float* x;             // [B][ldres] residual stream (read-modify-write)
  int ldres;
  bf16_t* xa_out;       // [B][ldres] x * alpha_next as a bf16 hi/lo pair (lo plane at + xa_lo)
  long xa_lo;
  const float* alpha_next;
  float* part_out;      // [B][M/16] sum of squares per 16 rows
  float* tap;           // [B][ldres] copy of x (nullable)
  // EPI_GATED / EPI_STORE / EPI_LOGITS
  bf16_t* m_out; int ldm;        // gated: [B][ldm] silu(g)*u as a bf16 hi/lo pair
  long m_lo;
  float* f_out; long ldf;        // store / logits: [B][ldf] fp32
  float* amax_v; int* amax_i; int ld_amax;  // logits: per-workgroup (max, argmax) [B][ld_amax]
  // large-batch path (B >= WIDE_MIN_B): per-tile partial sums, and the slots' inverse
  // RMS (computed once per launch by the main kernel, read by the reduce)
  float* split_part;    // [weight tile][8 ranges][512] fp32
  float* wide_rms;      // [MAX_COLS] fp32
  // EPI_RESID with B <= DEP_FUSE_B: the input X is the depformer attention
  // output, computed by every workgroup from `att` instead of read from X
  int fuse_att;
  DepAttnArgs att;
  // EPI_QKV with B <= DEP_FUSE_B: the input X (and its norm partials) is the
  // previous step's finisher output, computed by every workgroup from `fin`
  // (greedy choice only); workgroup 0 also writes the tokens and y
  int fuse_fin;
  FinishArgs fin;
};

// Large-batch path: weight tiles (gate and up tiles counted apart) and
// partial floats (8 ranges x 512 per weight tile).
// The smallest batch at which any GEMM takes the large-batch path (split
// k-ranges, activation slice in LDS; K >= 4096): the temporal QKV, from B = 9.
// Each GEMM has its own threshold at or above it; the partial buffer exists
// from this batch on.
constexpr int WIDE_MIN_B = 9;
inline long wide_tiles(int epi, int M) { return (epi == EPI_GATED ? 2L : 1L) * ((M + ROWS - 1) / ROWS); }
inline long wide_part_floats(int epi, int M) { return wide_tiles(epi, M) * 8 * 512; }

void launch_gemm(Epi epi, const GemmArgs& a, hipStream_t s);
// True when launch_gemm takes the large-batch (k-range split) path for `a`.
bool gemm_splits_k(Epi epi, const GemmArgs& a);
// Columns (slots) the large-batch path carries for `a`: 16 when every slot
// fits one MFMA column tile, else 32.  Its partials hold that many slots.
int gemm_wide_cols(const GemmArgs& a);
void launch_pack(const bf16_t* src, int M, int K, bf16_t* dst, hipStream_t s);
inline long packed_elems(int M, int K) { return (long)((M + ROWS - 1) / ROWS) * ROWS * K; }

struct AttnArgs {
  const float* q;       // [B][ldq], head h at q + h*head_dim
  int ldq;
  bf16_t* kv;           // ring base of this layer (see GemmArgs); written only on the large-batch path
  long kv_slot_stride, kv_v_off;
  int n_heads, head_dim, window, B;
  const int* ti; int pos_const;
  float* part;          // [B][n_heads][max_chunks][head_dim + 2] (m, l, o...)
  int max_chunks;
  bf16_t* o;            // [B][ldo] output as a bf16 hi/lo pair (lo plane at o + o_lo)
  int ldo;
  long o_lo;
  unsigned* cnt;        // [B][n_heads] split tickets, zero between launches (unused with one split)
  // Large-batch path: q, k and v are not formed by the QKV launch.  Each
  // workgroup sums its head's q rows from the QKV k-range partials
  // ([tile][8 ranges][qkv_cols slots][16 rows] fp32), scales them by the slot's
  // inverse RMS and rotates them (rope: [B][head_dim] cos/sin); the last
  // split also forms k and v and writes them to the ring.  Null otherwise.
  const float* qkv_part;
  int qkv_cols;           // slots per partial block (gemm_wide_cols)
  const float* qkv_rms;   // [MAX_COLS]
  const float* rope;
};

void launch_attention(const AttnArgs& a, hipStream_t s);

struct EmbedArgs {
  const int* ti; int B, d;
  const double* inv_freq; int head_dim; float* rope;  // RoPE table of the tick (see GemmArgs::rope)
  const bf16_t* emb_text; const bf16_t* emb_audio; int text_rows, audio_rows;
  const float* xin;  // [B][d] given temporal inputs (embedding-form prefill frames), read where TI_XIN is set
  const float* alpha;   // first attention-norm alpha
  float* x; bf16_t* xa; long xa_lo; float* part; float* tap;
};
void launch_embed(const EmbedArgs& a, hipStream_t s);

void launch_finish(const FinishArgs& a, hipStream_t s);
void finish_prepare();  // once per process, before the first finisher launch

// ---------------------------------------------------------------------------
// Fused depformer loop (dep_loop.hip): one persistent launch runs the 8
// codebook steps of one or two depformer halves for a few columns, with the
// tick's GEMM arithmetic (the 8 k-ranges of the contract map onto the 8
// XCDs).  A column is one slot of one half: the agent half (codebooks 0..7 of
// this tick) or the user half (codebooks 8..15 of the previous tick).
// ---------------------------------------------------------------------------
constexpr int DL_MAX_COLS = 4;   // MFMA columns in use: up to 2 slots x 2 halves
constexpr int DL_XCDS = 8;       // XCDs of the part (= ranges of the GEMM contract)
constexpr int DL_GRID = 256;     // workgroups: one per compute unit, DL_GRID / DL_XCDS per XCD
constexpr int DL_MAX_DD = 1024;  // depformer width held in LDS per column
constexpr int DL_MAX_KW = 12;    // k-steps a wave holds for one job (down-projection range)

// Error codes the loop leaves in its control block (ctl[2]).
enum { DL_OK = 0, DL_ERR_PLACEMENT = 1, DL_ERR_TIMEOUT = 2 };

struct DepLoopCol {
  int slot;              // slot of the tick input / output blocks and taps
  int k0;                // first codebook: 0 (agent half) or n_q (user half)
  int set;               // depformer buffer set: input projections, first input, key/value cache
};

struct DepLoopArgs {
  int ncols;
  DepLoopCol col[DL_MAX_COLS];
  // per buffer set: input projections of z [B][dep_q][dd]; the user half's
  // first input y = u_8 + table_8[chosen codebook 7] [B][dd] (written by the
  // agent half's last step, read by the user half)
  const float* u[2];
  float* y[2];
  float* logits;         // depformer logits [B][dep_q][A] (taps)
  int dd, dH, dhd, dF, Ld, A, dep_q, n_q;
  float eps;
  // weights (tile layout for matrices)
  const bf16_t *wqkv, *wo, *w_in, *w_out, *heads;  // stacked per layer / per codebook
  const bf16_t *emb_text, *emb_audio;              // input tables: text [Vt+1][dd]; audio [dep_q-1][A+1][dd]
  const float *attn_norm, *mlp_norm, *out_norm;
  // tick I/O: the text head's per-tile argmax partials (agent columns' first
  // choice), the tick input (forced choices) and output blocks
  const float* tamax_v; const int* tamax_i; int ld_amax; int n_tpart;
  const int* ti; int* to;
  // exchange memory (tagged 8-byte words), laid out by dep_loop_layout
  uint64_t* xq;          // per (step, layer): queries [C][dd]
  uint64_t* xo;          // per (step, layer): out-projection partials [8][C][dd] + done words [8][32]
  uint64_t* xm;          // per (step, layer): gate/up outputs [C][dF]
  uint64_t* xd;          // per (step, layer): down-projection partials [8][C][dd] + done words [8][32]
  uint64_t* xh;          // per step: head tile argmax [2][A/16][C][2]
  uint64_t* kv;          // per set and slot: key/value cache [Ld][2][dH][16][dhd/2], tagged pairs
  uint32_t* kvtag;       // [set * PP_MAX_BATCH + slot]: the launch tag of the agent half's cache entries
  long kv_slot_words, kv_set_words;
  uint32_t* ctl;         // [0] last launch tag, [1] exit count, [2] error, [4..11] per-XCD arrival counts
  long spin_limit;       // polls before a wait gives up (DL_ERR_TIMEOUT)
};

// Words of exchange memory for C columns (xq, xo, xm, xd, xh in that order):
// per (step, layer) queries [C][dd], out-projection partials [8][C][dd] and 64
// done words, gate/up outputs [C][dF], down-projection partials [8][C][dd]
// and 64 done words; per step the head tiles' (max, argmax) [2][A/16][C][2].
struct DepLoopLayout { long q, o, m, d, h, total; };
inline DepLoopLayout dep_loop_layout(int dd, int dF, int Ld, int A, int C) {
  DepLoopLayout l{};
  const long sl = 8L * Ld;
  l.q = 0;
  l.o = l.q + sl * C * dd;
  l.m = l.o + sl * (8L * C * dd + 64);
  l.d = l.m + sl * (long)C * dF;
  l.h = l.d + sl * (8L * C * dd + 64);
  l.total = l.h + 8L * 2 * (A / 16) * C * 2;
  return l;
}
// Words of the tagged key/value cache of one slot of one buffer set.
inline long dep_loop_kv_words(int dd, int Ld) { return (long)Ld * 2 * 16 * dd / 2; }
// Whether the loop supports these depformer dims: dd <= DL_MAX_DD, dd and dF
// multiples of 256, heads aligned with the 8 k-ranges, one job per
// workgroup per phase, every head tile a workgroup.  *why: the reason when not.
inline bool dep_loop_supported(int dd, int dH, int dF, int A, const char** why) {
  auto no = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (dd > DL_MAX_DD || dd % 256 || dF % 256) return no("depformer width above 1024, or width or FFN not a multiple of 256");
  if (dH % DL_XCDS || (dd / DL_XCDS) % (dd / dH)) return no("depformer heads do not split evenly over the 8 k-ranges");
  if (2 * (dd / 256) > DL_MAX_KW || dF / 256 > DL_MAX_KW) return no("a k-range too long for one wave's registers");
  const int per = DL_GRID / DL_XCDS;
  if (3 * dd / 128 > per || dF / 128 > per || dd / 128 > per) return no("more than one job per workgroup in a phase");
  if (A % 16 || 2 * (A / 16) > DL_GRID) return no("more head tiles than workgroups");
  return true;
}
void launch_dep_loop(const DepLoopArgs& a, hipStream_t s);
void dep_loop_prepare();  // once per process, before the first launch

// The library's own work-buffer array for the allocation-free entry point
// (pp_step_static): STATIC_SCRATCH_BYTES of device memory per GPU, held until
// the process ends.  static_scratch() returns its device address on the
// current device, looked up once per device; launch_zero_u32 clears n words.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;
hipError_t static_scratch(void** out);
void launch_zero_u32(unsigned* p, long n, hipStream_t s);

}  // namespace pp
