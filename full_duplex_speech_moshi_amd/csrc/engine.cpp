// Host side of libpp.so: argument validation, per-slot session state
// (position, previous column, forced-frame queue), arena layout, and the tick
// graph (all kernels of one tick captured once per handle and replayed each
// tick; guide "架构": static shapes and a fixed-capacity ring so the whole
// step can be captured).
#include <hip/hip_runtime.h>

#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <functional>
#include <string>
#include <vector>

#include "../../include/pp.h"
#include "kernels.h"

using namespace pp;

namespace {

constexpr size_t ALIGN = 256;
constexpr int DEP_WINDOW = 16;  // depformer per-frame keys (one per codebook step)
static_assert(DEP_WINDOW <= DEP_MAX_KEYS, "depformer attention holds at most DEP_MAX_KEYS keys");

struct Layout {
  // byte offsets into the arena
  size_t ring, x, xa, part, q, att_part, o, m, hidden, text_logits, tamax_v, tamax_i, dep_logits, ti, to, inv_freq,
      split_part, wide_rms, rope, att_cnt, xin, total;
  // depformer buffers, two sets: the agent codebooks of tick t+1 run beside
  // the user-stream codebooks of tick t, which keep using the other set
  size_t dkv[2], amax_v[2], amax_i[2], u[2], y[2], ya[2], dpart[2], dq[2], dout[2], dm[2], sctx[2];
  size_t samp, rep;  // sampling parameters; recent chosen text tokens [B][SAMPLE_REP]
  // the same work buffers laid out in the library's static array (pp_step_static)
  size_t s_att_cnt, s_wide_rms, s_att_part, s_split_part, s_total;
  // fused depformer loop (B <= 2 and supported dims): exchange words, tagged
  // key/value cache [2 sets][B slots], the agent halves' cache tags, control
  bool dl_ok;
  size_t dl_x, dl_kv, dl_kvtag, dl_ctl;
  DepLoopLayout dl;
  long dl_kv_slot_words;
  long wide_part_max;
  int max_chunks, n_amax;
  long ring_slot_elems, ring_layer_elems, ring_v_off;
  long dkv_slot_elems, dkv_layer_elems, dkv_v_off;
};

bool dims_ok(const pp_dims* dm, std::string* why) {
  auto fail = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (!dm) return fail("dims is NULL");
  if (dm->n_q != 8 || dm->dep_q != 16) return fail("n_q must be 8 and dep_q 16 (17-row column)");
  if (dm->d <= 0 || dm->n_layers <= 0 || dm->n_heads <= 0 || dm->ffn <= 0) return fail("bad temporal dims");
  if (dm->dep_d <= 0 || dm->dep_layers <= 0 || dm->dep_heads <= 0 || dm->dep_ffn <= 0) return fail("bad depformer dims");
  if (dm->d % dm->n_heads || dm->dep_d % dm->dep_heads) return fail("d not divisible by heads");
  const int hd = dm->d / dm->n_heads, dhd = dm->dep_d / dm->dep_heads;
  if ((hd != 32 && hd != 64 && hd != 128) || (dhd != 32 && dhd != 64 && dhd != 128))
    return fail("head_dim must be 32, 64 or 128");
  if (dm->d % 32 || dm->ffn % 32 || dm->dep_d % 32 || dm->dep_ffn % 32) return fail("d and ffn must be multiples of 32");
  if (dm->text_card < 2 || dm->audio_card < 2) return fail("vocabulary too small");
  if (!(dm->norm_eps >= 0.f) || !(dm->rope_base > 0.f)) return fail("bad eps or rope base");
  return true;
}

Layout make_layout(const pp_dims& dm, int B, int W) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + ALIGN - 1) / ALIGN * ALIGN;
    return o;
  };
  const long d = dm.d, H = dm.n_heads, hd = d / H, F = dm.ffn, Vt = dm.text_card, A = dm.audio_card;
  const long dd = dm.dep_d, dH = dm.dep_heads, dhd = dd / dH, dF = dm.dep_ffn, Q = dm.dep_q;
  L.ring_layer_elems = 2 * H * (long)W * hd;
  L.ring_slot_elems = dm.n_layers * L.ring_layer_elems;
  L.ring_v_off = H * (long)W * hd;
  L.dkv_layer_elems = 2 * dH * DEP_WINDOW * dhd;
  L.dkv_slot_elems = dm.dep_layers * L.dkv_layer_elems;
  L.dkv_v_off = dH * DEP_WINDOW * dhd;
  L.max_chunks = (W + ATT_CHUNK - 1) / ATT_CHUNK;  // <= ATT_MAX_SPLITS for W <= PP_MAX_WINDOW
  L.n_amax = (int)((std::max(Vt, A) + ROWS - 1) / ROWS);
  L.ring = take((size_t)B * L.ring_slot_elems * 2);
  L.x = take(B * d * 4);
  L.xa = take(2 * B * d * 2);  // activations feeding GEMMs: bf16 hi plane then lo plane
  L.part = take(B * (d / 16) * 4);
  L.q = take(B * d * 4);
  L.att_part = take((size_t)B * H * L.max_chunks * (hd + 2) * 4);
  L.o = take(2 * B * d * 2);
  L.m = take(2 * B * F * 2);
  L.hidden = take((size_t)(dm.n_layers + 1) * B * d * 4);
  L.text_logits = take(B * Vt * 4);
  // argmax partials of the text head (its own: the user-stream codebooks of
  // the previous tick may run beside it)
  L.tamax_v = take((size_t)B * L.n_amax * 4);
  L.tamax_i = take((size_t)B * L.n_amax * 4);
  for (int s = 0; s < 2; ++s) {
    L.dkv[s] = take((size_t)B * L.dkv_slot_elems * 2);
    L.amax_v[s] = take((size_t)B * L.n_amax * 4);
    L.amax_i[s] = take((size_t)B * L.n_amax * 4);
    L.u[s] = take(B * Q * dd * 4);
    L.y[s] = take(B * dd * 4);
    L.ya[s] = take(2 * B * dd * 2);
    L.dpart[s] = take(B * (dd / 16) * 4);
    L.dq[s] = take(B * dd * 4);
    L.dout[s] = take(2 * B * dd * 2);
    L.dm[s] = take(2 * B * dF * 2);
    L.sctx[s] = take((size_t)B * 4 * 4);
  }
  L.dep_logits = take(B * Q * A * 4);
  L.ti = take(B * TI_STRIDE * 4);
  L.xin = take((size_t)B * d * 4);
  L.to = take(B * TO_STRIDE * 4);
  L.inv_freq = take((hd / 2) * 8);
  // scratch of the large-batch GEMM path: the largest partial area of any GEMM
  // that may take it (the temporal stack, the text head and the depformer
  // input projections; the depformer layers and heads are given no scratch
  // and never take that path)
  const struct { Epi epi; long M; } wide[] = {{EPI_QKV, 3L * d}, {EPI_RESID, d}, {EPI_GATED, F}, {EPI_LOGITS, Vt},
                                             {EPI_STORE, (long)Q * dd}};
  L.wide_part_max = 0;
  for (const auto& g : wide) L.wide_part_max = std::max(L.wide_part_max, wide_part_floats(g.epi, (int)g.M));
  L.split_part = B >= WIDE_MIN_B ? take((size_t)L.wide_part_max * 4) : take(0);
  L.wide_rms = take(MAX_COLS * 4);
  L.rope = take((size_t)B * hd * 4);
  L.samp = take(sizeof(SampleParams));
  L.rep = take((size_t)B * SAMPLE_REP * 4);
  L.att_cnt = take((size_t)B * H * 4);
  L.dl_ok = B <= 2 && dep_loop_supported((int)dd, (int)dH, (int)dF, (int)A, nullptr);
  L.dl = dep_loop_layout((int)dd, (int)dF, dm.dep_layers, (int)A, 2 * B);
  L.dl_kv_slot_words = dep_loop_kv_words((int)dd, dm.dep_layers);
  L.dl_x = take(L.dl_ok ? (size_t)L.dl.total * 8 : 0);
  L.dl_kv = take(L.dl_ok ? (size_t)2 * B * L.dl_kv_slot_words * 8 : 0);
  L.dl_kvtag = take(L.dl_ok ? 2 * PP_MAX_BATCH * 4 : 0);
  L.dl_ctl = take(L.dl_ok ? 64 : 0);
  L.total = off;
  // work buffers only (partials, tickets, inverse RMS), for the static array
  off = 0;
  L.s_att_cnt = take((size_t)B * H * 4);
  L.s_wide_rms = take(MAX_COLS * 4);
  L.s_att_part = take((size_t)B * H * L.max_chunks * (hd + 2) * 4);
  L.s_split_part = B >= WIDE_MIN_B ? take((size_t)L.wide_part_max * 4) : take(0);
  L.s_total = off;
  return L;
}

// A queued prefill frame: rows 0-8 the tokens to choose (-1 free), rows
// 9-16 the user codes; an embedding-form frame also carries the tick's
// temporal input x (d floats) and no user codes.
struct Frame {
  std::array<int32_t, 17> tok;
  std::vector<float> x;
};

using Row8 = std::array<int32_t, 8>;

struct Slot {
  int64_t pos = 0;
  int32_t prev[9];
  std::deque<Frame> queue;
  bool live = false, ticked = false;
  // Acoustic delay D: frame-aligned user frames and forced agent rows of the
  // last ticks (newest last; a user row of -1s = none given) feed codebooks
  // 1-7 of the column D ticks later; the chosen agent rows of the last D + 1
  // ticks form the completed agent frame.
  std::deque<Row8> user_hist, force_hist, chosen_hist;
  int64_t ticks = 0;  // ticks since the last reset
  uint64_t seed = 0;  // sampling seed (kept across resets)
  std::deque<int32_t> text_hist;  // chosen text tokens of the last SAMPLE_REP ticks
  Row8 frame_out{};
  bool frame_valid = false;
  // this tick's frame-aligned user frame and forced agent row (set with the
  // tick input, committed to the history once the tick has run)
  Row8 tick_user{}, tick_force{};
};

thread_local std::string g_create_error;

}  // namespace

struct pp_handle {
  pp_dims dm;
  int B, W;
  pp_weights w;
  Layout lay;
  char* arena = nullptr;
  // The tick is three phases: PH_TEMPORAL (embedding, temporal stack, text
  // head) and PH_AGENT (input projections, text finisher, codebooks 0..n_q-1)
  // on the caller's stream, and PH_USER (the user-stream codebooks n_q..) on
  // `side`.  PH_USER of tick t is launched by tick t+1, after its
  // PH_TEMPORAL, so that it runs beside PH_AGENT of tick t+1; the two use
  // different depformer buffer sets (set = tick parity), one graph each.
  // exec[0] = PH_TEMPORAL, exec[1 + s] = PH_AGENT on set s, exec[3 + s] =
  // PH_USER on set s.
  hipStream_t stream = nullptr, cap = nullptr, side = nullptr;
  hipGraph_t graph[5] = {};
  hipGraphExec_t exec[5] = {};
  // PH_TEMPORAL and the two PH_AGENT graphs again, with the work buffers in
  // the library's static array (pp_step_static); PH_USER uses none of them
  char* sptr = nullptr;    // device address of that array on this handle's device
  bool static_ok = false;  // this handle's work buffers fit in it
  hipGraph_t graph_s[3] = {};
  hipGraphExec_t exec_s[3] = {};
  // The fused depformer loop (B <= 2, greedy, supported dims): the depformer
  // of a tick is one persistent launch after the input projections.  The
  // user-stream half of tick t runs as extra columns of tick t+1's launch, on
  // the caller's stream.  exec_f[ds] = agent half on set ds with the pending
  // user half (set 1 - ds); exec_f[2 + ds] = agent half alone; exec_f[4 + ds] =
  // user half of set ds alone (flushes).
  bool dl_on = false;         // use the fused loop where it applies (pp_set_depformer_loop)
  bool fused = false;         // it applies now (dl_ok, dl_on and greedy)
  bool pending_fused = false; // the pending user half belongs to the fused path
  hipGraph_t graph_f[6] = {};
  hipGraphExec_t exec_f[6] = {};
  hipEvent_t temporal_done = nullptr, agent_done = nullptr, user_done[2] = {nullptr, nullptr};
  int parity = 0;             // depformer buffer set of the next tick
  bool user_pending = false;  // PH_USER of the last tick not launched yet
  int32_t* ti_host = nullptr;
  int32_t* to_host = nullptr;
  float* xin_host = nullptr;  // [B][d] given temporal inputs of embedding-form frames
  int32_t* rep_host = nullptr;  // [B][SAMPLE_REP] recent chosen text tokens (-1 empty)
  SampleParams samp{};        // host copy of the device sampling parameters
  int delay = 0;              // acoustic delay of codebooks 1-7, frames
  std::vector<Slot> slots;
  std::vector<std::function<void(hipStream_t)>> timed[6];  // per layer
  double timed_bytes[6] = {0, 0, 0, 0, 0, 0};
  std::string err;
  bool poisoned = false;

  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(arena + off); }

  int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    if (code == PP_EDEVICE) poisoned = true;
    return code;
  }
};

#define HIP_OR_FAIL(h, call)                                                                  \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess) return (h)->fail(PP_EDEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

namespace {

void reset_slot(const pp_dims& dm, Slot& s) {
  s.pos = 0;
  s.prev[0] = dm.text_card;
  for (int i = 1; i < 9; ++i) s.prev[i] = dm.audio_card;
  s.queue.clear();
  s.live = false;
  s.ticked = false;
  s.user_hist.clear();
  s.force_hist.clear();
  s.chosen_hist.clear();
  s.ticks = 0;
  s.text_hist.clear();
  s.frame_out.fill(0);
  s.frame_valid = false;
}

enum Phase { PH_TEMPORAL = 0, PH_AGENT = 1, PH_USER = 2 };

// Record the kernels of one phase of the tick on stream s.
// `ds`: the depformer buffer set (PH_AGENT and PH_USER of one tick share one).
// `stat`: the work buffers are in the library's static array, not the arena.
void record_tick(pp_handle* h, hipStream_t s, Phase phase, int ds, bool keep_timed, bool stat = false) {
  const pp_dims& dm = h->dm;
  const Layout& L = h->lay;
  const int B = h->B, W = h->W;
  const int d = dm.d, H = dm.n_heads, hd = d / H, F = dm.ffn, Vt = dm.text_card, A = dm.audio_card;
  const int dd = dm.dep_d, dH = dm.dep_heads, dhd = dd / dH, dF = dm.dep_ffn, Q = dm.dep_q;
  const pp_weights& w = h->w;
  const int* ti = h->at<int>(L.ti);
  int* to = h->at<int>(L.to);
  const double* inv_freq = h->at<double>(L.inv_freq);
  float* split_part = stat ? reinterpret_cast<float*>(h->sptr + L.s_split_part) : h->at<float>(L.split_part);
  float* wide_rms = stat ? reinterpret_cast<float*>(h->sptr + L.s_wide_rms) : h->at<float>(L.wide_rms);
  float* att_part = stat ? reinterpret_cast<float*>(h->sptr + L.s_att_part) : h->at<float>(L.att_part);
  unsigned* att_cnt = stat ? reinterpret_cast<unsigned*>(h->sptr + L.s_att_cnt) : h->at<unsigned>(L.att_cnt);

  if (phase == PH_TEMPORAL) {
    // the split tickets must start at zero: the static array keeps whatever
    // the last call on this GPU left there
    if (stat) launch_zero_u32(att_cnt, (long)B * H, s);
    EmbedArgs ea{};
    ea.ti = ti;
    ea.B = B;
    ea.d = d;
    ea.emb_text = w.emb_text;
    ea.emb_audio = w.emb_audio;
    ea.xin = h->at<float>(L.xin);
    ea.text_rows = Vt + 1;
    ea.audio_rows = A + 1;
    ea.alpha = w.attn_norm;
    ea.x = h->at<float>(L.x);
    ea.xa = h->at<bf16_t>(L.xa);
    ea.xa_lo = (long)B * d;
    ea.part = h->at<float>(L.part);
    ea.tap = h->at<float>(L.hidden);
    ea.inv_freq = inv_freq;
    ea.head_dim = hd;
    ea.rope = h->at<float>(L.rope);
    launch_embed(ea, s);

    for (int l = 0; l < dm.n_layers; ++l) {
      bf16_t* ring_l = h->at<bf16_t>(L.ring) + (long)l * L.ring_layer_elems;
      // fused QKV + rotation + ring write
      GemmArgs g{};
      g.W = w.wqkv + (long)l * 3 * d * d;
      g.X = h->at<bf16_t>(L.xa);
      g.x_lo = (long)B * d;
      g.M = 3 * d;
      g.K = d;
      g.ldx = d;
      g.B = B;
      g.part_in = h->at<float>(L.part);
      g.n_part = d / 16;
      g.feat = d;
      g.eps = dm.norm_eps;
      g.q_out = h->at<float>(L.q);
      g.ldq = d;
      g.kv = ring_l;
      g.kv_slot_stride = L.ring_slot_elems;
      g.kv_v_off = L.ring_v_off;
      g.n_heads = H;
      g.head_dim = hd;
      g.window = W;
      g.ti = ti;
      g.inv_freq = inv_freq;
      g.rope = h->at<float>(L.rope);
      g.split_part = split_part;
      g.wide_rms = wide_rms;
      // large-batch path: the decode pass below finishes q, k and v itself
      g.qkv_to_attn = gemm_splits_k(EPI_QKV, g) ? 1 : 0;
      launch_gemm(EPI_QKV, g, s);
      if (keep_timed) h->timed[0].push_back([g](hipStream_t st) { launch_gemm(EPI_QKV, g, st); });
      if (keep_timed && l == 0) {
        h->timed_bytes[0] = 2.0 * 3 * d * d + B * (4.0 * d + 4.0 * d / 16 + 4.0 * d + 4.0 * d);
      }

      AttnArgs at{};
      at.q = h->at<float>(L.q);
      at.ldq = d;
      at.kv = ring_l;
      at.kv_slot_stride = L.ring_slot_elems;
      at.kv_v_off = L.ring_v_off;
      at.n_heads = H;
      at.head_dim = hd;
      at.window = W;
      at.B = B;
      at.ti = ti;
      at.part = att_part;
      at.max_chunks = L.max_chunks;
      at.o = h->at<bf16_t>(L.o);
      at.ldo = d;
      at.o_lo = (long)B * d;
      at.cnt = att_cnt;
      if (g.qkv_to_attn) {
        at.qkv_part = split_part;
        at.qkv_cols = gemm_wide_cols(g);
        at.qkv_rms = wide_rms;
        at.rope = h->at<float>(L.rope);
      }
      launch_attention(at, s);
      if (keep_timed) h->timed[1].push_back([at](hipStream_t st) { launch_attention(at, st); });
      if (keep_timed && l == 0) {
        h->timed_bytes[1] = -1;  // depends on positions; computed at timing
      }

      GemmArgs go{};
      go.W = w.wo + (long)l * d * d;
      go.X = h->at<bf16_t>(L.o);
      go.x_lo = (long)B * d;
      go.M = d;
      go.K = d;
      go.ldx = d;
      go.B = B;
      go.x = h->at<float>(L.x);
      go.ldres = d;
      go.xa_out = h->at<bf16_t>(L.xa);
      go.xa_lo = (long)B * d;
      go.alpha_next = w.mlp_norm + (long)l * d;
      go.part_out = h->at<float>(L.part);
      go.split_part = split_part;
      go.wide_rms = wide_rms;
      launch_gemm(EPI_RESID, go, s);
      if (keep_timed) h->timed[2].push_back([go](hipStream_t st) { launch_gemm(EPI_RESID, go, st); });
      if (keep_timed && l == 0) {
        h->timed_bytes[2] = 2.0 * d * d + B * (4.0 * d + 4.0 * d + 4.0 * d + 4.0 * d + 4.0 * d / 16);
      }

      GemmArgs gu{};
      gu.W = w.w_in + (long)l * 2 * F * d;
      gu.X = h->at<bf16_t>(L.xa);
      gu.x_lo = (long)B * d;
      gu.M = F;
      gu.K = d;
      gu.ldx = d;
      gu.B = B;
      gu.gate_off = F;
      gu.part_in = h->at<float>(L.part);
      gu.n_part = d / 16;
      gu.feat = d;
      gu.eps = dm.norm_eps;
      gu.m_out = h->at<bf16_t>(L.m);
      gu.ldm = F;
      gu.m_lo = (long)B * F;
      gu.split_part = split_part;
      gu.wide_rms = wide_rms;
      launch_gemm(EPI_GATED, gu, s);
      if (keep_timed) h->timed[3].push_back([gu](hipStream_t st) { launch_gemm(EPI_GATED, gu, st); });
      if (keep_timed && l == 0) {
        h->timed_bytes[3] = 2.0 * 2 * F * d + B * (4.0 * d + 4.0 * d / 16 + 4.0 * F);
      }

      GemmArgs gd{};
      gd.W = w.w_out + (long)l * d * F;
      gd.X = h->at<bf16_t>(L.m);
      gd.x_lo = (long)B * F;
      gd.M = d;
      gd.K = F;
      gd.ldx = F;
      gd.B = B;
      gd.x = h->at<float>(L.x);
      gd.ldres = d;
      gd.xa_out = h->at<bf16_t>(L.xa);
      gd.xa_lo = (long)B * d;
      gd.alpha_next = (l + 1 < dm.n_layers) ? w.attn_norm + (long)(l + 1) * d : w.out_norm;
      gd.part_out = h->at<float>(L.part);
      gd.tap = h->at<float>(L.hidden) + (long)(l + 1) * B * d;
      gd.split_part = split_part;
      gd.wide_rms = wide_rms;
      launch_gemm(EPI_RESID, gd, s);
      if (keep_timed) h->timed[4].push_back([gd](hipStream_t st) { launch_gemm(EPI_RESID, gd, st); });
      if (keep_timed && l == 0) {
        h->timed_bytes[4] = 2.0 * d * F + B * (4.0 * F + 4.0 * d + 4.0 * d + 4.0 * d + 4.0 * d + 4.0 * d / 16);
      }
    }

    // text head + greedy partials
    GemmArgs gt{};
    gt.W = w.text_head;
    gt.X = h->at<bf16_t>(L.xa);
    gt.x_lo = (long)B * d;
    gt.M = Vt;
    gt.K = d;
    gt.ldx = d;
    gt.B = B;
    gt.part_in = h->at<float>(L.part);
    gt.n_part = d / 16;
    gt.feat = d;
    gt.eps = dm.norm_eps;
    gt.f_out = h->at<float>(L.text_logits);
    gt.ldf = Vt;
    gt.amax_v = h->at<float>(L.tamax_v);
    gt.amax_i = h->at<int>(L.tamax_i);
    gt.ld_amax = L.n_amax;
    gt.split_part = split_part;
    gt.wide_rms = wide_rms;
    launch_gemm(EPI_LOGITS, gt, s);
    if (keep_timed) {
      h->timed[5].push_back([gt](hipStream_t st) { launch_gemm(EPI_LOGITS, gt, st); });
      h->timed_bytes[5] = 2.0 * Vt * d + B * (4.0 * d + 4.0 * d / 16 + 4.0 * Vt);
    }

  }  // PH_TEMPORAL: embedding, temporal stack, text head

  // the text finisher (greedy text token -> depformer step 0 input); the
  // codebook finishers below copy it
  FinishArgs fa{};
  fa.B = B;
  fa.step = -1;
  fa.n_part = (Vt + ROWS - 1) / ROWS;
  fa.amax_v = h->at<float>(L.tamax_v);
  fa.amax_i = h->at<int>(L.tamax_i);
  fa.ld_amax = L.n_amax;
  fa.ti = ti;
  fa.to = to;
  fa.dep_q = Q;
  fa.dd = dd;
  fa.u = h->at<float>(L.u[ds]);
  fa.table = w.dep_emb_text;
  fa.alpha = w.dep_attn_norm;
  fa.y = h->at<float>(L.y[ds]);
  fa.ya = h->at<bf16_t>(L.ya[ds]);
  fa.ya_lo = (long)B * dd;
  fa.part = h->at<float>(L.dpart[ds]);
  fa.sp = h->at<SampleParams>(L.samp);
  fa.logits = h->at<float>(L.text_logits);
  fa.ld_logits = Vt;
  fa.n_logits = Vt;
  fa.rep = h->at<int>(L.rep);
  fa.sctx = h->at<unsigned>(L.sctx[ds]);

  // depformer input projections u_k = P_k z for codebooks [c0, c1), one GEMM
  auto in_proj = [&](int c0, int c1) {
    GemmArgs gp{};
    gp.W = w.dep_in_proj + (long)c0 * packed_elems(dd, d);
    gp.X = h->at<bf16_t>(L.xa);
    gp.x_lo = (long)B * d;
    gp.M = (c1 - c0) * dd;
    gp.K = d;
    gp.ldx = d;
    gp.B = B;
    gp.part_in = h->at<float>(L.part);
    gp.n_part = d / 16;
    gp.feat = d;
    gp.eps = dm.norm_eps;
    gp.f_out = h->at<float>(L.u[ds]) + (long)c0 * dd;
    gp.ldf = (long)Q * dd;
    gp.split_part = split_part;
    gp.wide_rms = wide_rms;
    launch_gemm(EPI_STORE, gp, s);
  };

  // All 16 projections run here: z (the normalised final hidden state) is
  // overwritten by the next tick's temporal stack, which runs before this
  // tick's user-stream codebooks.
  // Greedy ticks at B <= DEP_FUSE_B fold each finisher into the next step's
  // first QKV projection, except codebook 7's (its tokens are returned by
  // pp_step before the user-stream codebooks run) and the last codebook's.
  const bool fuse_fin = B <= DEP_FUSE_B && dd <= DEP_FUSE_D && !h->samp.enabled;
  auto finish_of = [&](int k) {  // the finisher of codebook step k
    FinishArgs f = fa;
    f.step = k;
    f.n_part = (A + ROWS - 1) / ROWS;
    f.amax_v = h->at<float>(L.amax_v[ds]);
    f.amax_i = h->at<int>(L.amax_i[ds]);
    f.table = (k + 1 < Q) ? w.dep_emb_audio + (long)k * (A + 1) * dd : nullptr;
    f.logits = h->at<float>(L.dep_logits) + (long)k * A;
    f.ld_logits = (long)Q * A;
    f.n_logits = A;
    f.rep = nullptr;
    return f;
  };
  if (phase == PH_AGENT) {
    in_proj(0, Q);
    if (!fuse_fin) launch_finish(fa, s);
  }

  // codebook steps: the agent stream in PH_AGENT, the user stream in PH_USER
  if (phase == PH_TEMPORAL) return;
  const int k0 = phase == PH_AGENT ? 0 : dm.n_q, k1 = phase == PH_AGENT ? dm.n_q : Q;
  for (int k = k0; k < k1; ++k) {
    for (int l = 0; l < dm.dep_layers; ++l) {
      bf16_t* dkv_l = h->at<bf16_t>(L.dkv[ds]) + (long)l * L.dkv_layer_elems;
      GemmArgs g{};
      g.W = w.dep_wqkv + (long)l * 3 * dd * dd;
      g.w_keep = 1;  // re-read at every codebook step
      g.X = h->at<bf16_t>(L.ya[ds]);
      g.x_lo = (long)B * dd;
      g.M = 3 * dd;
      g.K = dd;
      g.ldx = dd;
      g.B = B;
      g.part_in = h->at<float>(L.dpart[ds]);
      g.n_part = dd / 16;
      g.feat = dd;
      g.eps = dm.norm_eps;
      g.q_out = h->at<float>(L.dq[ds]);
      g.ldq = dd;
      g.kv = dkv_l;
      g.kv_slot_stride = L.dkv_slot_elems;
      g.kv_v_off = L.dkv_v_off;
      g.n_heads = dH;
      g.head_dim = dhd;
      g.window = DEP_WINDOW;
      g.ti = nullptr;
      g.pos_const = k;
      g.inv_freq = nullptr;
      if (l == 0 && fuse_fin && k != dm.n_q) {
        g.fuse_fin = 1;
        g.fin = k == 0 ? fa : finish_of(k - 1);
      }
      launch_gemm(EPI_QKV, g, s);

      // attention over steps 0..k of this frame: inside the out-projection at
      // small batch, else its own launch (same arithmetic either way)
      DepAttnArgs da{};
      da.q = h->at<float>(L.dq[ds]);
      da.ldq = dd;
      da.kv = dkv_l;
      da.slot_stride = L.dkv_slot_elems;
      da.v_off = L.dkv_v_off;
      da.n_heads = dH;
      da.head_dim = dhd;
      da.window = DEP_WINDOW;
      da.n_keys = k + 1;
      da.B = B;
      da.o = h->at<bf16_t>(L.dout[ds]);
      da.ldo = dd;
      da.o_lo = (long)B * dd;
      const bool fuse_att = B <= DEP_FUSE_B && dd <= DEP_FUSE_D;
      if (!fuse_att) launch_dep_attention(da, s);

      GemmArgs go{};
      go.W = w.dep_wo + (long)l * dd * dd;
      go.w_keep = 1;  // re-read at every codebook step
      go.X = h->at<bf16_t>(L.dout[ds]);
      go.x_lo = (long)B * dd;
      go.M = dd;
      go.K = dd;
      go.ldx = dd;
      go.B = B;
      go.x = h->at<float>(L.y[ds]);
      go.ldres = dd;
      go.xa_out = h->at<bf16_t>(L.ya[ds]);
      go.xa_lo = (long)B * dd;
      go.alpha_next = w.dep_mlp_norm + (long)l * dd;
      go.part_out = h->at<float>(L.dpart[ds]);
      go.fuse_att = fuse_att;
      go.att = da;
      launch_gemm(EPI_RESID, go, s);

      GemmArgs gu{};
      gu.W = w.dep_w_in + (long)l * 2 * dF * dd;
      gu.w_keep = 1;  // re-read at every codebook step
      gu.X = h->at<bf16_t>(L.ya[ds]);
      gu.x_lo = (long)B * dd;
      gu.M = dF;
      gu.K = dd;
      gu.ldx = dd;
      gu.B = B;
      gu.gate_off = dF;
      gu.part_in = h->at<float>(L.dpart[ds]);
      gu.n_part = dd / 16;
      gu.feat = dd;
      gu.eps = dm.norm_eps;
      gu.m_out = h->at<bf16_t>(L.dm[ds]);
      gu.ldm = dF;
      gu.m_lo = (long)B * dF;
      launch_gemm(EPI_GATED, gu, s);

      GemmArgs gd{};
      gd.W = w.dep_w_out + (long)l * dd * dF;
      gd.w_keep = 1;  // re-read at every codebook step
      gd.X = h->at<bf16_t>(L.dm[ds]);
      gd.x_lo = (long)B * dF;
      gd.M = dd;
      gd.K = dF;
      gd.ldx = dF;
      gd.B = B;
      gd.x = h->at<float>(L.y[ds]);
      gd.ldres = dd;
      gd.xa_out = h->at<bf16_t>(L.ya[ds]);
      gd.xa_lo = (long)B * dd;
      gd.alpha_next = (l + 1 < dm.dep_layers) ? w.dep_attn_norm + (long)(l + 1) * dd : w.dep_out_norm;
      gd.part_out = h->at<float>(L.dpart[ds]);
      launch_gemm(EPI_RESID, gd, s);
    }
    GemmArgs gh{};
    gh.W = w.dep_heads + (long)k * packed_elems(A, dd);
    gh.X = h->at<bf16_t>(L.ya[ds]);
    gh.x_lo = (long)B * dd;
    gh.M = A;
    gh.K = dd;
    gh.ldx = dd;
    gh.B = B;
    gh.part_in = h->at<float>(L.dpart[ds]);
    gh.n_part = dd / 16;
    gh.feat = dd;
    gh.eps = dm.norm_eps;
    gh.f_out = h->at<float>(L.dep_logits) + (long)k * A;
    gh.ldf = (long)Q * A;
    gh.amax_v = h->at<float>(L.amax_v[ds]);
    gh.amax_i = h->at<int>(L.amax_i[ds]);
    gh.ld_amax = L.n_amax;
    launch_gemm(EPI_LOGITS, gh, s);

    if (!fuse_fin || k == dm.n_q - 1 || k == Q - 1) launch_finish(finish_of(k), s);
  }
}

// Record the depformer of a tick as one fused launch on stream s: the input
// projections of set ds (with the agent half) and the loop over the agent
// half of set ds and / or the user half of set su.
void record_fused(pp_handle* h, hipStream_t s, bool agent, int ds, bool user, int su) {
  const pp_dims& dm = h->dm;
  const Layout& L = h->lay;
  const int B = h->B, d = dm.d, dd = dm.dep_d, Q = dm.dep_q, A = dm.audio_card, Vt = dm.text_card;
  const pp_weights& w = h->w;
  if (agent) {
    GemmArgs gp{};
    gp.W = w.dep_in_proj;
    gp.X = h->at<bf16_t>(L.xa);
    gp.x_lo = (long)B * d;
    gp.M = Q * dd;
    gp.K = d;
    gp.ldx = d;
    gp.B = B;
    gp.part_in = h->at<float>(L.part);
    gp.n_part = d / 16;
    gp.feat = d;
    gp.eps = dm.norm_eps;
    gp.f_out = h->at<float>(L.u[ds]);
    gp.ldf = (long)Q * dd;
    launch_gemm(EPI_STORE, gp, s);  // B <= 2: the small-batch path, no scratch
  }
  DepLoopArgs a{};
  int c = 0;
  for (int half = 0; half < 2; ++half) {
    if (half == 0 ? !agent : !user) continue;
    const int set = half == 0 ? ds : su;
    for (int b = 0; b < B; ++b, ++c) {
      a.col[c].slot = b;
      a.col[c].k0 = half == 0 ? 0 : dm.n_q;
      a.col[c].set = set;
    }
  }
  a.ncols = c;
  for (int set = 0; set < 2; ++set) {
    a.u[set] = h->at<float>(L.u[set]);
    a.y[set] = h->at<float>(L.y[set]);
  }
  a.logits = h->at<float>(L.dep_logits);
  a.dd = dd;
  a.dH = dm.dep_heads;
  a.dhd = dd / dm.dep_heads;
  a.dF = dm.dep_ffn;
  a.Ld = dm.dep_layers;
  a.A = A;
  a.dep_q = Q;
  a.n_q = dm.n_q;
  a.eps = dm.norm_eps;
  a.wqkv = w.dep_wqkv;
  a.wo = w.dep_wo;
  a.w_in = w.dep_w_in;
  a.w_out = w.dep_w_out;
  a.heads = w.dep_heads;
  a.emb_text = w.dep_emb_text;
  a.emb_audio = w.dep_emb_audio;
  a.attn_norm = w.dep_attn_norm;
  a.mlp_norm = w.dep_mlp_norm;
  a.out_norm = w.dep_out_norm;
  a.tamax_v = h->at<float>(L.tamax_v);
  a.tamax_i = h->at<int>(L.tamax_i);
  a.ld_amax = L.n_amax;
  a.n_tpart = (Vt + ROWS - 1) / ROWS;
  a.ti = h->at<int>(L.ti);
  a.to = h->at<int>(L.to);
  uint64_t* x = h->at<uint64_t>(L.dl_x);
  const DepLoopLayout xl = dep_loop_layout(dd, dm.dep_ffn, dm.dep_layers, A, c);
  a.xq = x + xl.q;
  a.xo = x + xl.o;
  a.xm = x + xl.m;
  a.xd = x + xl.d;
  a.xh = x + xl.h;
  a.kv = h->at<uint64_t>(L.dl_kv);
  a.kv_slot_words = L.dl_kv_slot_words;
  a.kv_set_words = (long)B * L.dl_kv_slot_words;
  a.kvtag = h->at<uint32_t>(L.dl_kvtag);
  a.ctl = h->at<uint32_t>(L.dl_ctl);
  a.spin_limit = 1L << 20;  // polls (about a microsecond each) before a wait gives up
  launch_dep_loop(a, s);
}

// Fill the tick-input staging buffer from slot state; frames[b] = prefill
// frame consumed this tick or nullptr.  Reads the delay history without
// changing it.  Text row and codebook 0 take this tick's frame; codebooks
// 1-7 (user rows 10-16 and the forced choices of agent rows 2-8) take the
// frame D ticks back: the initial audio token and no force before the first.
void build_tick_input(pp_handle* h, const int32_t* user_codes, const Frame** frames) {
  const int A = h->dm.audio_card, D = h->delay;
  for (int b = 0; b < h->B; ++b) {
    int32_t* t = h->ti_host + b * TI_STRIDE;
    Slot& s = h->slots[b];
    t[TI_POS] = (int32_t)s.pos;
    for (int i = 0; i < 9; ++i) t[TI_COL + i] = s.prev[i];
    const Frame* f = frames ? frames[b] : nullptr;
    const bool has_x = f && !f->x.empty();
    int32_t force_text = -1;
    for (int i = 0; i < 8; ++i) {
      s.tick_user[i] = has_x ? -1 : f ? f->tok[9 + i] : (user_codes ? user_codes[b * 8 + i] : 0);
      s.tick_force[i] = f ? f->tok[1 + i] : -1;
    }
    if (f) force_text = f->tok[0];
    const Row8* u_old = nullptr;
    const Row8* f_old = nullptr;
    if (D == 0) {
      u_old = &s.tick_user;
      f_old = &s.tick_force;
    } else {
      if ((int)s.user_hist.size() >= D) u_old = &s.user_hist[s.user_hist.size() - D];
      if ((int)s.force_hist.size() >= D) f_old = &s.force_hist[s.force_hist.size() - D];
    }
    if (u_old && (*u_old)[0] < 0) u_old = nullptr;  // that tick gave no user codes
    t[TI_COL + 9] = s.tick_user[0] >= 0 ? s.tick_user[0] : A;
    for (int i = 1; i < 8; ++i) t[TI_COL + 9 + i] = u_old ? (*u_old)[i] : A;
    t[TI_FORCE] = force_text;
    t[TI_FORCE + 1] = s.tick_force[0];
    for (int i = 1; i < 8; ++i) t[TI_FORCE + 1 + i] = f_old ? (*f_old)[i] : -1;
    t[TI_XIN] = has_x ? 1 : 0;
    t[TI_SEED] = (int32_t)(uint32_t)s.seed;
    t[TI_SEED + 1] = (int32_t)(uint32_t)(s.seed >> 32);
    t[TI_TICK] = (int32_t)(uint32_t)s.ticks;
    t[TI_TICK + 1] = (int32_t)(uint32_t)((uint64_t)s.ticks >> 32);
  }
}

// After a tick has run: this tick's frame-aligned rows join the delay
// history, and the agent frame completed by it (codebook 0 chosen D ticks
// ago, codebooks 1-7 chosen now) is kept for pp_agent_frames.
void commit_history(pp_handle* h, Slot& s, const int32_t* chosen_agent) {
  s.text_hist.push_back(chosen_agent[-1]);  // the chosen text token precedes the agent rows
  while (s.text_hist.size() > (size_t)SAMPLE_REP) s.text_hist.pop_front();
  const size_t keep = (size_t)std::max(h->delay, 1);
  Row8 c;
  std::memcpy(c.data(), chosen_agent, sizeof c);
  s.user_hist.push_back(s.tick_user);
  s.force_hist.push_back(s.tick_force);
  s.chosen_hist.push_back(c);
  while (s.user_hist.size() > keep) s.user_hist.pop_front();
  while (s.force_hist.size() > keep) s.force_hist.pop_front();
  while (s.chosen_hist.size() > (size_t)h->delay + 1) s.chosen_hist.pop_front();
  s.ticks += 1;
  s.frame_valid = s.ticks > h->delay;
  if (s.frame_valid) {
    s.frame_out[0] = s.chosen_hist.front()[0];
    for (int i = 1; i < 8; ++i) s.frame_out[i] = s.chosen_hist.back()[i];
  }
}

// Capture the five graphs of the tick (replacing any earlier ones), from the
// handle's current settings.  The caller has no device work in flight.
hipError_t capture_graphs(pp_handle* h) {
  hipError_t e;
  for (auto& t : h->timed) t.clear();
  for (int g = 0; g < 5; ++g) {
    if (h->exec[g]) (void)hipGraphExecDestroy(h->exec[g]);
    if (h->graph[g]) (void)hipGraphDestroy(h->graph[g]);
    h->exec[g] = nullptr;
    h->graph[g] = nullptr;
  }
  for (int g = 0; g < 5; ++g) {
    const Phase ph = g == 0 ? PH_TEMPORAL : g < 3 ? PH_AGENT : PH_USER;
    const int ds = g == 0 ? 0 : (g - 1) % 2;
    if ((e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal)) != hipSuccess) return e;
    record_tick(h, h->cap, ph, ds, ph == PH_TEMPORAL);
    if ((e = hipStreamEndCapture(h->cap, &h->graph[g])) != hipSuccess) return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipGraphInstantiate(&h->exec[g], h->graph[g], nullptr, nullptr, 0)) != hipSuccess) return e;
  }
  h->fused = h->lay.dl_ok && h->dl_on && !h->samp.enabled;
  for (int g = 0; g < 6; ++g) {
    if (h->exec_f[g]) (void)hipGraphExecDestroy(h->exec_f[g]);
    if (h->graph_f[g]) (void)hipGraphDestroy(h->graph_f[g]);
    h->exec_f[g] = nullptr;
    h->graph_f[g] = nullptr;
    if (!h->fused) continue;
    const int ds = g & 1, kind = g >> 1;  // 0 agent + pending user, 1 agent, 2 user
    if ((e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal)) != hipSuccess) return e;
    record_fused(h, h->cap, kind != 2, ds, kind != 1, kind == 0 ? 1 - ds : ds);
    if ((e = hipStreamEndCapture(h->cap, &h->graph_f[g])) != hipSuccess) return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipGraphInstantiate(&h->exec_f[g], h->graph_f[g], nullptr, nullptr, 0)) != hipSuccess) return e;
  }
  for (int g = 0; g < 3; ++g) {
    if (h->exec_s[g]) (void)hipGraphExecDestroy(h->exec_s[g]);
    if (h->graph_s[g]) (void)hipGraphDestroy(h->graph_s[g]);
    h->exec_s[g] = nullptr;
    h->graph_s[g] = nullptr;
    if (!h->static_ok) continue;
    const Phase ph = g == 0 ? PH_TEMPORAL : PH_AGENT;
    const int ds = g == 0 ? 0 : g - 1;
    if ((e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal)) != hipSuccess) return e;
    record_tick(h, h->cap, ph, ds, false, true);
    if ((e = hipStreamEndCapture(h->cap, &h->graph_s[g])) != hipSuccess) return e;
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipGraphInstantiate(&h->exec_s[g], h->graph_s[g], nullptr, nullptr, 0)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Launch the last tick's PH_USER on the side stream, after that tick's
// PH_AGENT (the most recent record of `agent_done`) and, when `after` is
// given, after that event too.
hipError_t launch_user(pp_handle* h, hipEvent_t after) {
  if (!h->user_pending) return hipSuccess;
  const int ds = 1 - h->parity;
  hipError_t e;
  if (h->pending_fused) {  // the fused loop's user half alone, on the caller's stream
    if ((e = hipGraphLaunch(h->exec_f[4 + ds], h->stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(h->user_done[ds], h->stream)) != hipSuccess) return e;
    h->user_pending = false;
    return hipSuccess;
  }
  if ((e = hipStreamWaitEvent(h->side, h->agent_done, 0)) != hipSuccess) return e;
  if (after && (e = hipStreamWaitEvent(h->side, after, 0)) != hipSuccess) return e;
  if ((e = hipGraphLaunch(h->exec[3 + ds], h->side)) != hipSuccess) return e;
  if ((e = hipEventRecord(h->user_done[ds], h->side)) != hipSuccess) return e;
  h->user_pending = false;
  return hipSuccess;
}

// Launch one tick: PH_TEMPORAL; then the previous tick's PH_USER on the side
// stream; then, once PH_USER of two ticks back has released this tick's
// buffer set, PH_AGENT.  This tick's PH_USER is left pending.  `stat`: the
// graphs whose work buffers are in the library's static array.
hipError_t launch_tick(pp_handle* h, bool stat = false) {
  const int ds = h->parity;
  hipError_t e;
  const bool fz = h->fused && !stat;  // pp_step_static takes the per-launch graphs
  // a pending user half of the other kind completes first, in its own way;
  // before a fused launch the caller's stream waits for it (the persistent
  // launch needs every compute unit)
  if (h->user_pending && h->pending_fused != fz) {
    if ((e = launch_user(h, nullptr)) != hipSuccess) return e;
    if (fz && (e = hipStreamWaitEvent(h->stream, h->user_done[1 - ds], 0)) != hipSuccess) return e;
  }
  if (fz) {
    // the temporal stack, then one launch for the agent half of this tick
    // and the pending user half of the last one (all on the caller's stream)
    if ((e = hipGraphLaunch(h->exec[0], h->stream)) != hipSuccess) return e;
    // a user half of set ds run on the second stream (by a per-launch tick)
    // must be done before this tick's agent half reuses the set
    if ((e = hipStreamWaitEvent(h->stream, h->user_done[ds], 0)) != hipSuccess) return e;
    if ((e = hipGraphLaunch(h->exec_f[(h->user_pending ? 0 : 2) + ds], h->stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(h->user_done[1 - ds], h->stream)) != hipSuccess) return e;
    h->user_pending = true;
    h->pending_fused = true;
    h->parity = 1 - ds;
    return hipSuccess;
  }
  if ((e = hipGraphLaunch(stat ? h->exec_s[0] : h->exec[0], h->stream)) != hipSuccess) return e;
  if ((e = hipEventRecord(h->temporal_done, h->stream)) != hipSuccess) return e;
  if ((e = launch_user(h, h->temporal_done)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(h->stream, h->user_done[ds], 0)) != hipSuccess) return e;
  if ((e = hipGraphLaunch(stat ? h->exec_s[1 + ds] : h->exec[1 + ds], h->stream)) != hipSuccess) return e;
  if ((e = hipEventRecord(h->agent_done, h->stream)) != hipSuccess) return e;
  h->user_pending = true;
  h->pending_fused = false;
  h->parity = 1 - ds;
  return hipSuccess;
}

// Launch the pending PH_USER, if any, and make `s` wait for every PH_USER.
hipError_t flush_user(pp_handle* h, hipStream_t s) {
  hipError_t e;
  if ((e = launch_user(h, nullptr)) != hipSuccess) return e;
  for (int i = 0; i < 2; ++i)
    if ((e = hipStreamWaitEvent(s, h->user_done[i], 0)) != hipSuccess) return e;
  return hipSuccess;
}

// A fused depformer loop left an error code in the tick output: the
// handle is poisoned (the tick's outputs are not valid).
int loop_error(pp_handle* h, int code) {
  return h->fail(PP_EDEVICE, "fused depformer loop: %s (code %d)",
                 code == DL_ERR_PLACEMENT ? "a workgroup ran on an unexpected XCD"
                                          : "a wait for another workgroup's results gave up",
                 code);
}

// After device work that may include a fused user half outside pp_step:
// read the error word.
int check_loop_error(pp_handle* h) {
  if (!h->lay.dl_ok) return PP_OK;
  int32_t code = 0;
  HIP_OR_FAIL(h, hipMemcpy(&code, h->at<int>(h->lay.to) + TO_ERR, 4, hipMemcpyDeviceToHost));
  return code ? loop_error(h, code) : PP_OK;
}

}  // namespace

extern "C" {

int pp_arena_bytes(const pp_dims* dims, int B, int window, size_t* out_bytes) {
  std::string why;
  if (!out_bytes || !dims_ok(dims, &why) || B < 1 || B > PP_MAX_BATCH || window < 1 ||
      window > PP_MAX_WINDOW)
    return PP_EINVAL;
  *out_bytes = make_layout(*dims, B, window).total;
  return PP_OK;
}

int pp_create(const pp_dims* dims, int B, int window, const pp_weights* w, void* arena, size_t arena_bytes,
              void* stream, pp_handle** out) {
  std::string why;
  if (!out) { g_create_error = "out is NULL"; return PP_EINVAL; }
  *out = nullptr;
  if (!dims_ok(dims, &why)) { g_create_error = why; return PP_EINVAL; }
  if (B < 1 || B > PP_MAX_BATCH) { g_create_error = "B out of [1, 32]"; return PP_EINVAL; }
  if (window < 1 || window > PP_MAX_WINDOW) { g_create_error = "window outside 1..PP_MAX_WINDOW"; return PP_EINVAL; }
  if (!w || !arena) { g_create_error = "weights or arena is NULL"; return PP_EINVAL; }
  const void* const* wp = reinterpret_cast<const void* const*>(w);
  for (size_t i = 0; i < sizeof(pp_weights) / sizeof(void*); ++i)
    if (!wp[i]) { g_create_error = "a weight pointer is NULL"; return PP_EINVAL; }
  if (reinterpret_cast<uintptr_t>(arena) % ALIGN) { g_create_error = "arena not 256-byte aligned"; return PP_EINVAL; }
  const Layout lay = make_layout(*dims, B, window);
  if (arena_bytes < lay.total) { g_create_error = "arena too small"; return PP_ENOSPC; }

  pp_handle* h = new (std::nothrow) pp_handle();
  if (!h) { g_create_error = "out of host memory"; return PP_ENOSPC; }
  h->dm = *dims;
  h->B = B;
  h->W = window;
  h->w = *w;
  h->lay = lay;
  h->arena = static_cast<char*>(arena);
  h->stream = static_cast<hipStream_t>(stream);
  h->slots.resize(B);
  for (auto& s : h->slots) reset_slot(*dims, s);

  auto bail = [&](const char* what, hipError_t e) {
    g_create_error = std::string(what) + ": " + hipGetErrorString(e);
    pp_destroy(h);
    return PP_EDEVICE;
  };
  hipError_t e;
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->ti_host), B * TI_STRIDE * 4, hipHostMallocDefault)) != hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->to_host), B * TO_STRIDE * 4, hipHostMallocDefault)) != hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->xin_host), (size_t)B * dims->d * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->rep_host), (size_t)B * SAMPLE_REP * 4,
                         hipHostMallocDefault)) != hipSuccess)
    return bail("hipHostMalloc", e);
  std::memset(h->ti_host, 0, B * TI_STRIDE * 4);
  std::memset(h->xin_host, 0, (size_t)B * dims->d * 4);
  std::memset(h->to_host, 0, B * TO_STRIDE * 4);

  // RoPE frequencies base^(-2i/head_dim), fp64 host math.
  const int hd = dims->d / dims->n_heads;
  std::vector<double> freq(hd / 2);
  for (int i = 0; i < hd / 2; ++i) freq[i] = std::pow((double)dims->rope_base, -2.0 * i / hd);
  if ((e = hipMemcpyAsync(h->at<double>(lay.inv_freq), freq.data(), freq.size() * 8, hipMemcpyHostToDevice,
                          h->stream)) != hipSuccess)
    return bail("hipMemcpyAsync", e);
  build_tick_input(h, nullptr, nullptr);
  if ((e = hipMemcpyAsync(h->at<int>(lay.ti), h->ti_host, B * TI_STRIDE * 4, hipMemcpyHostToDevice, h->stream)) !=
      hipSuccess)
    return bail("hipMemcpyAsync", e);
  if ((e = hipStreamSynchronize(h->stream)) != hipSuccess) return bail("hipStreamSynchronize", e);

  if ((e = hipMemsetAsync(h->at<char>(lay.att_cnt), 0, (size_t)B * dims->n_heads * 4, h->stream)) != hipSuccess)
    return bail("hipMemsetAsync", e);
  if ((e = hipMemsetAsync(h->at<char>(lay.to), 0, (size_t)B * TO_STRIDE * 4, h->stream)) != hipSuccess)
    return bail("hipMemsetAsync", e);
  // the fused loop's memory starts at zero: no word carries a launch tag yet
  if (lay.dl_ok && (e = hipMemsetAsync(h->at<char>(lay.dl_x), 0, lay.total - lay.dl_x, h->stream)) != hipSuccess)
    return bail("hipMemsetAsync", e);
  if ((e = hipMemcpyAsync(h->at<char>(lay.samp), &h->samp, sizeof(SampleParams), hipMemcpyHostToDevice, h->stream)) !=
      hipSuccess)
    return bail("hipMemcpyAsync", e);
  if ((e = hipStreamSynchronize(h->stream)) != hipSuccess) return bail("hipStreamSynchronize", e);
  finish_prepare();
  dep_loop_prepare();
  {
    void* sp = nullptr;
    if ((e = static_scratch(&sp)) != hipSuccess) return bail("hipGetSymbolAddress (static work buffers)", e);
    h->sptr = static_cast<char*>(sp);
    h->static_ok = lay.s_total <= STATIC_SCRATCH_BYTES;
  }
  if ((e = hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking)) != hipSuccess) return bail("hipStreamCreate", e);
  if ((e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking)) != hipSuccess) return bail("hipStreamCreate", e);
  for (hipEvent_t* ev : {&h->temporal_done, &h->agent_done, &h->user_done[0], &h->user_done[1]}) {
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return bail("hipEventCreate", e);
    if ((e = hipEventRecord(*ev, h->side)) != hipSuccess) return bail("hipEventRecord", e);
  }
  if ((e = capture_graphs(h)) != hipSuccess) return bail("graph capture", e);
  *out = h;
  return PP_OK;
}

int pp_prefill_forced(pp_handle* h, int slot, const int32_t* frames, int n) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (slot < 0 || slot >= h->B) return h->fail(PP_EINVAL, "slot %d out of [0,%d)", slot, h->B);
  if (n < 0 || (n > 0 && !frames)) return h->fail(PP_EINVAL, "bad frame count or NULL frames");
  Slot& s = h->slots[slot];
  if (s.live) return h->fail(PP_EBUSY, "slot %d is free-running; persona and voice are fixed at open", slot);
  if (s.queue.size() + (size_t)n > PP_MAX_QUEUE) return h->fail(PP_ENOSPC, "forced queue full");
  const int Vt = h->dm.text_card, A = h->dm.audio_card;
  for (int i = 0; i < n; ++i) {
    const int32_t* f = frames + i * 17;
    if (f[0] < -1 || f[0] >= Vt) return h->fail(PP_EINVAL, "frame %d: text token %d out of range", i, f[0]);
    for (int r = 1; r < 9; ++r)
      if (f[r] < -1 || f[r] >= A) return h->fail(PP_EINVAL, "frame %d: agent code %d out of range", i, f[r]);
    for (int r = 9; r < 17; ++r)
      if (f[r] < 0 || f[r] >= A) return h->fail(PP_EINVAL, "frame %d: user code %d out of range", i, f[r]);
  }
  for (int i = 0; i < n; ++i) {
    Frame fr;
    std::memcpy(fr.tok.data(), frames + i * 17, sizeof fr.tok);
    s.queue.push_back(std::move(fr));
  }
  return PP_OK;
}

int pp_prefill_embed(pp_handle* h, int slot, const float* x, const int32_t* force, int n) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (slot < 0 || slot >= h->B) return h->fail(PP_EINVAL, "slot %d out of [0,%d)", slot, h->B);
  if (n < 0 || (n > 0 && !x)) return h->fail(PP_EINVAL, "bad frame count or NULL inputs");
  Slot& s = h->slots[slot];
  if (s.live) return h->fail(PP_EBUSY, "slot %d is free-running; persona and voice are fixed at open", slot);
  if (s.queue.size() + (size_t)n > PP_MAX_QUEUE) return h->fail(PP_ENOSPC, "forced queue full");
  const int Vt = h->dm.text_card, A = h->dm.audio_card, d = h->dm.d;
  for (int i = 0; i < n; ++i) {
    if (force) {
      const int32_t* f = force + i * 9;
      if (f[0] < -1 || f[0] >= Vt) return h->fail(PP_EINVAL, "frame %d: text token %d out of range", i, f[0]);
      for (int r = 1; r < 9; ++r)
        if (f[r] < -1 || f[r] >= A) return h->fail(PP_EINVAL, "frame %d: agent code %d out of range", i, f[r]);
    }
    for (int j = 0; j < d; ++j)
      if (!std::isfinite(x[(size_t)i * d + j])) return h->fail(PP_EINVAL, "frame %d: input %d not finite", i, j);
  }
  for (int i = 0; i < n; ++i) {
    Frame fr;
    fr.tok.fill(0);
    for (int r = 0; r < 9; ++r) fr.tok[r] = force ? force[i * 9 + r] : -1;
    fr.x.assign(x + (size_t)i * d, x + (size_t)(i + 1) * d);
    s.queue.push_back(std::move(fr));
  }
  return PP_OK;
}

int pp_set_acoustic_delay(pp_handle* h, int frames) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (frames < 0 || frames > PP_MAX_DELAY) return h->fail(PP_EINVAL, "delay %d outside [0,%d]", frames, PP_MAX_DELAY);
  for (int b = 0; b < h->B; ++b)
    if (h->slots[b].ticked) return h->fail(PP_EBUSY, "slot %d has ticked since its reset", b);
  h->delay = frames;
  return PP_OK;
}

int pp_set_sampling(pp_handle* h, const pp_sampling* sp) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  SampleParams p{};
  if (sp) {
    const bool ok = std::isfinite(sp->text_temperature) && sp->text_temperature >= 0.f &&
                    std::isfinite(sp->audio_temperature) && sp->audio_temperature >= 0.f && sp->top_k >= 0 &&
                    sp->top_p > 0.f && sp->top_p <= 1.f && std::isfinite(sp->repetition_penalty) &&
                    sp->repetition_penalty >= 1.f;
    if (!ok) return h->fail(PP_EINVAL, "sampling parameters out of range");
    if (h->dm.text_card > SAMPLE_MAX_N || h->dm.audio_card > SAMPLE_MAX_N)
      return h->fail(PP_EINVAL, "logits rows wider than %d cannot be sampled", SAMPLE_MAX_N);
    p.enabled = 1;
    p.t_text = sp->text_temperature;
    p.t_audio = sp->audio_temperature;
    p.top_k = sp->top_k;
    p.top_p = sp->top_p;
    p.rho = sp->repetition_penalty;
  }
  // the pending user-stream codebooks belong to the last tick: they keep its parameters
  HIP_OR_FAIL(h, launch_user(h, nullptr));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->side));
  HIP_OR_FAIL(h, hipMemcpyAsync(h->at<char>(h->lay.samp), &p, sizeof p, hipMemcpyHostToDevice, h->stream));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  if (const int rc = check_loop_error(h)) return rc;
  const bool recapture = p.enabled != h->samp.enabled;  // greedy ticks fold the finishers into the QKV launches
  h->samp = p;
  if (recapture) HIP_OR_FAIL(h, capture_graphs(h));
  return PP_OK;
}

int pp_set_depformer_loop(pp_handle* h, int on) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (on != 0 && on != 1) return h->fail(PP_EINVAL, "on must be 0 or 1");
  const char* why = "more than 2 slots";
  if (on && !h->lay.dl_ok && (h->B > 2 || !dep_loop_supported(h->dm.dep_d, h->dm.dep_heads, h->dm.dep_ffn,
                                                                h->dm.audio_card, &why)))
    return h->fail(PP_EINVAL, "the fused depformer loop does not apply to this handle: %s", why);
  // the pending user half completes in its own way before the graphs change
  HIP_OR_FAIL(h, launch_user(h, nullptr));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->side));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  if (const int rc = check_loop_error(h)) return rc;
  h->dl_on = on != 0;
  HIP_OR_FAIL(h, capture_graphs(h));
  return PP_OK;
}

int pp_depformer_loop_active(const pp_handle* h) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  return h->fused ? 1 : 0;
}

int pp_slot_seed(pp_handle* h, int slot, uint64_t seed) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (slot < 0 || slot >= h->B) return h->fail(PP_EINVAL, "slot %d out of [0,%d)", slot, h->B);
  h->slots[slot].seed = seed;
  return PP_OK;
}

int pp_agent_frames(const pp_handle* h, int32_t* frames, int32_t* valid) {
  if (!h || !frames || !valid) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  for (int b = 0; b < h->B; ++b) {
    const Slot& s = h->slots[b];
    valid[b] = s.frame_valid ? 1 : 0;
    for (int i = 0; i < 8; ++i) frames[b * 8 + i] = s.frame_valid ? s.frame_out[i] : 0;
  }
  return PP_OK;
}

}  // extern "C"

namespace {

// One tick (pp_step, and pp_step_static with `stat`).  Allocates no memory:
// the frames in use sit in a fixed array.
int step_impl(pp_handle* h, const int32_t* user_codes, int32_t* tokens, bool stat) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (!user_codes || !tokens) return h->fail(PP_EINVAL, "NULL user_codes or tokens");
  if (stat && !h->static_ok)
    return h->fail(PP_ENOSPC, "work buffers of %zu bytes exceed the static array of %zu bytes", h->lay.s_total,
                   STATIC_SCRATCH_BYTES);
  const int A = h->dm.audio_card;
  for (int b = 0; b < h->B; ++b) {
    if (h->slots[b].pos >= 0x7fffffff) return h->fail(PP_EINVAL, "slot %d position overflow", b);
    if (!h->slots[b].queue.empty()) continue;  // codes of this slot are replaced by the forced frame
    for (int i = 0; i < 8; ++i) {
      const int32_t c = user_codes[b * 8 + i];
      if (c < 0 || c >= A) return h->fail(PP_EINVAL, "slot %d user code %d out of range", b, c);
    }
  }
  std::array<const Frame*, PP_MAX_BATCH> frames{};
  bool any_x = false;
  for (int b = 0; b < h->B; ++b)
    if (!h->slots[b].queue.empty()) {
      frames[b] = &h->slots[b].queue.front();
      if (!frames[b]->x.empty()) {
        std::memcpy(h->xin_host + (size_t)b * h->dm.d, frames[b]->x.data(), (size_t)h->dm.d * 4);
        any_x = true;
      }
    }
  build_tick_input(h, user_codes, frames.data());
  HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(h->lay.ti), h->ti_host, h->B * TI_STRIDE * 4, hipMemcpyHostToDevice,
                                h->stream));
  if (any_x)
    HIP_OR_FAIL(h, hipMemcpyAsync(h->at<float>(h->lay.xin), h->xin_host, (size_t)h->B * h->dm.d * 4,
                                  hipMemcpyHostToDevice, h->stream));
  if (h->samp.enabled && h->samp.rho != 1.f) {
    for (int b = 0; b < h->B; ++b) {
      int32_t* r = h->rep_host + (size_t)b * SAMPLE_REP;
      const auto& th = h->slots[b].text_hist;
      for (int i = 0; i < SAMPLE_REP; ++i) r[i] = i < (int)th.size() ? th[i] : -1;
    }
    HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(h->lay.rep), h->rep_host, (size_t)h->B * SAMPLE_REP * 4,
                                  hipMemcpyHostToDevice, h->stream));
  }
  HIP_OR_FAIL(h, launch_tick(h, stat));
  // the agent outputs only (the user-stream codebooks may still be writing theirs)
  HIP_OR_FAIL(h, hipMemcpy2DAsync(h->to_host + TO_PRED, TO_STRIDE * 4, h->at<int>(h->lay.to) + TO_PRED, TO_STRIDE * 4,
                                  9 * 4, h->B, hipMemcpyDeviceToHost, h->stream));
  HIP_OR_FAIL(h, hipMemcpy2DAsync(h->to_host + TO_CHOSEN, TO_STRIDE * 4, h->at<int>(h->lay.to) + TO_CHOSEN,
                                  TO_STRIDE * 4, (TO_ERR + 1 - TO_CHOSEN) * 4, h->B, hipMemcpyDeviceToHost,
                                  h->stream));
  HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  if (h->to_host[TO_ERR] != 0) return loop_error(h, h->to_host[TO_ERR]);
  for (int b = 0; b < h->B; ++b) {
    Slot& s = h->slots[b];
    const int32_t* o = h->to_host + b * TO_STRIDE;
    for (int i = 0; i < 9; ++i) {
      tokens[b * 9 + i] = o[TO_PRED + i];
      s.prev[i] = o[TO_CHOSEN + i];
    }
    commit_history(h, s, o + TO_CHOSEN + 1);
    if (frames[b]) s.queue.pop_front();
    else s.live = true;
    s.ticked = true;
    s.pos += 1;
  }
  return PP_OK;
}

}  // namespace

extern "C" {

int pp_step(pp_handle* h, const int32_t* user_codes, int32_t* tokens) {
  return step_impl(h, user_codes, tokens, false);
}

int pp_step_static(pp_handle* h, const int32_t* user_codes, int32_t* tokens) {
  return step_impl(h, user_codes, tokens, true);
}

int pp_slot_reset(pp_handle* h, int slot) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (slot < 0 || slot >= h->B) return h->fail(PP_EINVAL, "slot %d out of [0,%d)", slot, h->B);
  reset_slot(h->dm, h->slots[slot]);
  return PP_OK;
}

int pp_ring_fill(pp_handle* h, int slot, int n, const uint16_t* k, const uint16_t* v) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (slot < 0 || slot >= h->B) return h->fail(PP_EINVAL, "slot %d out of [0,%d)", slot, h->B);
  if (n < 0 || n > h->W) return h->fail(PP_EINVAL, "fill of %d frames outside [0, window=%d]", n, h->W);
  if (n > 0 && (!k || !v)) return h->fail(PP_EINVAL, "NULL keys or values");
  Slot& s = h->slots[slot];
  if (s.ticked || !s.queue.empty()) return h->fail(PP_EBUSY, "fill only before any tick or prefill of the slot");
  const int L = h->dm.n_layers, H = h->dm.n_heads, hd = h->dm.d / H;
  std::vector<uint16_t> tmp((size_t)H * n * hd);
  for (int l = 0; l < L && n > 0; ++l) {
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = (kv ? v : k) + (size_t)l * n * H * hd;
      for (int p = 0; p < n; ++p)
        for (int hh = 0; hh < H; ++hh)
          std::memcpy(&tmp[((size_t)hh * n + p) * hd], src + ((size_t)p * H + hh) * hd, hd * 2);
      bf16_t* dst = h->at<bf16_t>(h->lay.ring) + (long)slot * h->lay.ring_slot_elems + (long)l * h->lay.ring_layer_elems +
                    (kv ? h->lay.ring_v_off : 0);
      HIP_OR_FAIL(h, hipMemcpy2DAsync(dst, (size_t)h->W * hd * 2, tmp.data(), (size_t)n * hd * 2, (size_t)n * hd * 2,
                                      H, hipMemcpyHostToDevice, h->stream));
      HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
    }
  }
  s.pos = n;
  return PP_OK;
}

int pp_taps(const pp_handle* h, pp_taps_t* out) {
  if (!h || !out) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  // the last tick's user-stream codebooks write the depformer logits and
  // predictions: launch them if still pending, and wait
  pp_handle* hm = const_cast<pp_handle*>(h);
  if (flush_user(hm, hm->side) != hipSuccess || hipStreamSynchronize(hm->side) != hipSuccess) {
    hm->poisoned = true;
    return PP_EDEVICE;
  }
  if (const int rc = check_loop_error(hm)) return rc;
  out->hidden = h->at<float>(h->lay.hidden);
  out->text_logits = h->at<float>(h->lay.text_logits);
  out->dep_logits = h->at<float>(h->lay.dep_logits);
  out->tokens = h->at<int32_t>(h->lay.to);
  return PP_OK;
}

int pp_time_kernel(pp_handle* h, int which, int iters, float* avg_ms, double* bytes) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (which < 0 || which > 5 || iters < 1 || !avg_ms) return h->fail(PP_EINVAL, "bad kernel id, iters or output");
  double by = h->timed_bytes[which];
  if (which == 1) {  // attention: KV bytes from each slot's current window
    const int H = h->dm.n_heads, hd = h->dm.d / H;
    by = 0;
    for (int b = 0; b < h->B; ++b) {
      const long n = std::min<long>(h->slots[b].pos + 1, h->W);
      by += 2.0 * n * H * hd * 2 + 4.0 * h->dm.d + 4.0 * h->dm.d;
    }
  }
  if (bytes) *bytes = by;
  HIP_OR_FAIL(h, flush_user(h, h->stream));
  build_tick_input(h, nullptr, nullptr);
  HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(h->lay.ti), h->ti_host, h->B * TI_STRIDE * 4, hipMemcpyHostToDevice,
                                h->stream));
  hipEvent_t e0, e1;
  HIP_OR_FAIL(h, hipEventCreate(&e0));
  HIP_OR_FAIL(h, hipEventCreate(&e1));
  // One round = the kernel for every layer in order, each with that layer's
  // weights, as in the tick (weights are not cache-resident between uses).
  const auto& fns = h->timed[which];
  for (const auto& f : fns) f(h->stream);  // warm
  HIP_OR_FAIL(h, hipEventRecord(e0, h->stream));
  for (int i = 0; i < iters; ++i)
    for (const auto& f : fns) f(h->stream);
  HIP_OR_FAIL(h, hipEventRecord(e1, h->stream));
  HIP_OR_FAIL(h, hipEventSynchronize(e1));
  float ms = 0;
  HIP_OR_FAIL(h, hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  HIP_OR_FAIL(h, hipGetLastError());
  if (const int rc = check_loop_error(h)) return rc;
  *avg_ms = ms / (iters * (float)fns.size());
  return PP_OK;
}

int pp_time_graph(pp_handle* h, int iters, float* avg_ms) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (iters < 1 || !avg_ms) return h->fail(PP_EINVAL, "bad iters or output");
  build_tick_input(h, nullptr, nullptr);
  HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(h->lay.ti), h->ti_host, h->B * TI_STRIDE * 4, hipMemcpyHostToDevice,
                                h->stream));
  hipEvent_t e0, e1;
  HIP_OR_FAIL(h, hipEventCreate(&e0));
  HIP_OR_FAIL(h, hipEventCreate(&e1));
  // steady state of back-to-back ticks, timed from the end of the previous
  // tick's PH_USER to the end of the last one (the timer includes it)
  HIP_OR_FAIL(h, flush_user(h, h->stream));
  HIP_OR_FAIL(h, hipEventRecord(e0, h->stream));
  for (int i = 0; i < iters; ++i) HIP_OR_FAIL(h, launch_tick(h));
  HIP_OR_FAIL(h, flush_user(h, h->stream));
  HIP_OR_FAIL(h, hipEventRecord(e1, h->stream));
  HIP_OR_FAIL(h, hipEventSynchronize(e1));
  float ms = 0;
  HIP_OR_FAIL(h, hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (const int rc = check_loop_error(h)) return rc;
  *avg_ms = ms / iters;
  return PP_OK;
}

size_t pp_packed_elems(int M, int K) {
  if (M < 1 || K < 32 || K % 32) return 0;
  return (size_t)packed_elems(M, K);
}

int pp_pack_matrix(const uint16_t* src, int M, int K, uint16_t* dst, void* stream) {
  if (!src || !dst || M < 1 || K < 32 || K % 32) return PP_EINVAL;
  launch_pack(src, M, K, dst, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? PP_OK : PP_EDEVICE;
}

void pp_destroy(pp_handle* h) {
  if (!h) return;
  // a pending PH_USER is dropped: nothing reads its results after this
  if (h->side) (void)hipStreamSynchronize(h->side);
  (void)hipStreamSynchronize(h->stream);
  for (int g = 0; g < 5; ++g) {
    if (h->exec[g]) (void)hipGraphExecDestroy(h->exec[g]);
    if (h->graph[g]) (void)hipGraphDestroy(h->graph[g]);
  }
  for (int g = 0; g < 3; ++g) {
    if (h->exec_s[g]) (void)hipGraphExecDestroy(h->exec_s[g]);
    if (h->graph_s[g]) (void)hipGraphDestroy(h->graph_s[g]);
  }
  for (int g = 0; g < 6; ++g) {
    if (h->exec_f[g]) (void)hipGraphExecDestroy(h->exec_f[g]);
    if (h->graph_f[g]) (void)hipGraphDestroy(h->graph_f[g]);
  }
  for (hipEvent_t ev : {h->temporal_done, h->agent_done, h->user_done[0], h->user_done[1]})
    if (ev) (void)hipEventDestroy(ev);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->cap) (void)hipStreamDestroy(h->cap);
  if (h->ti_host) (void)hipHostFree(h->ti_host);
  if (h->xin_host) (void)hipHostFree(h->xin_host);
  if (h->rep_host) (void)hipHostFree(h->rep_host);
  if (h->to_host) (void)hipHostFree(h->to_host);
  delete h;
}

const char* pp_last_error(const pp_handle* h) {
  if (!h) return g_create_error.c_str();
  return h->err.c_str();
}

}  // extern "C"
