// Host side of the streaming codec (codec.h), decoder and encoder:
// validation, the arena layout, the slots' frame positions in each direction,
// and eight captured graphs (per direction two for calls, two for timing
// launches).
//
// A decode call turns one frame of 8 codes per slot into 1920 samples; an
// encode call turns 1920 samples per slot into 8 codes (chenxutan.com
// PersonaPlex article, section 2.3: Mimi maps 24 kHz audio to 12.5 Hz frames
// of 8 codebooks and back, causally; recipe "Architecture": 1920 samples per
// frame).  A decode graph runs the latent sum, the transformer layers on the
// tick's GEMM and ring-decode launchers, the output norm, the convolution
// stack and the state update; an encode graph runs the convolution stack,
// the transformer, the residual quantiser and the state update.  The two
// directions share the transformer's activation buffers (their calls never
// overlap) and keep separate rings, positions and histories.
// The convolutions' histories are double-buffered: a call's graph reads set
// p and writes set 1 - p, and consecutive calls alternate; timing launches
// write a third set, which no call reads.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/codec.h"
#include "codec_kernels.h"
#include "kernels.h"

namespace pp {
namespace {

constexpr size_t ALIGN = 256;
std::string g_codec_create_error;

bool codec_dims_ok(const pp_codec_dims* dm, std::string* why) {
  auto fail = [&](const char* m) {
    if (why) *why = m;
    return false;
  };
  if (!dm) return fail("dims is NULL");
  if (dm->n_q < 1 || dm->n_q > 16 || dm->card < 1) return fail("n_q must be 1..16 and card >= 1");
  if (dm->d <= 0 || dm->d % 32 || dm->n_layers <= 0 || dm->n_heads <= 0 || dm->ffn <= 0 || dm->ffn % 32)
    return fail("d and ffn must be positive multiples of 32");
  if (dm->d > 8192) return fail("d must be at most 8192");
  if (dm->d % dm->n_heads) return fail("d not divisible by n_heads");
  const int hd = dm->d / dm->n_heads;
  if (hd != 32 && hd != 64 && hd != 128) return fail("head_dim must be 32, 64 or 128");
  if (dm->window < 1 || dm->window > PP_CODEC_MAX_WINDOW) return fail("window outside 1..PP_CODEC_MAX_WINDOW");
  if (dm->conv_k < 1 || dm->res_k < 1 || dm->conv_k > 8 || dm->res_k > 8) return fail("kernels must be 1..8");
  if (dm->n_stages < 1 || dm->n_stages > PP_CODEC_MAX_STAGES) return fail("n_stages outside 1..PP_CODEC_MAX_STAGES");
  long samples = 1;
  for (int i = 0; i < dm->n_stages; ++i) {
    if (dm->strides[i] < 1 || dm->strides[i] > 8) return fail("strides must be 1..8");
    samples *= dm->strides[i];
    if (samples > (1 << 20)) return fail("too many samples per frame");
  }
  for (int i = 0; i <= dm->n_stages; ++i)
    if (dm->channels[i] < 1 || (i > 0 && dm->channels[i] % 2)) return fail("channels must be >= 1, even after stage 0");
  if (!(dm->norm_eps >= 0.f) || !(dm->rope_base > 0.f)) return fail("bad eps or rope base");
  return true;
}

long codec_samples(const pp_codec_dims& dm) {
  long s = 1;
  for (int i = 0; i < dm.n_stages; ++i) s *= dm.strides[i];
  return s;
}

// History entries: conv_in, then per stage the upsampling and the residual
// unit's first convolution, then conv_out (entries with H = 0 are left out).
// Each holds its convolution's input as fed: z for conv_in, the ELU'd
// signals for the others.
struct HistSpec {
  int C, H;
  size_t off[3];  // per set: two that calls alternate between, one that timing launches write
};

struct CodecLayout {
  size_t ti, codes, inv_freq, rope, x, xa, part, q, o, m, ring, att_part, att_cnt, z;
  size_t h0a, pcm;  // h0a: ELU of the first convolution's output
  // per stage: the upsampled signal u (raw, the residual unit's skip) and its
  // ELU, the ELU of the residual unit's first convolution, and the ELU of the
  // stage's output (each consumer's input as it is fed)
  size_t u[PP_CODEC_MAX_STAGES], ua[PP_CODEC_MAX_STAGES], ra[PP_CODEC_MAX_STAGES], ha[PP_CODEC_MAX_STAGES];
  long T[PP_CODEC_MAX_STAGES + 1];  // samples per call at each rate: T[0] = 1
  long ring_layer_elems, ring_slot_elems, ring_v_off;
  std::vector<HistSpec> hist;  // 0: conv_in, then up_i / res_a_i, then conv_out
  int h_conv_in, h_up[PP_CODEC_MAX_STAGES], h_res[PP_CODEC_MAX_STAGES], h_conv_out;
  // encoder: input samples, positions, RoPE table, ring, the latent y fed to
  // the transformer, its output z, the codes; per stage j the stage's input
  // (raw for the residual skip, and after ELU), the ELU of the residual
  // unit's first convolution, the ELU of the residual unit's output
  size_t pcm_in, e_ti, e_rope, e_ring, e_y, e_z, e_codes, e_qv, e_qi, e_qr;
  size_t e_h[PP_CODEC_MAX_STAGES + 1], e_ha[PP_CODEC_MAX_STAGES + 1], e_ra[PP_CODEC_MAX_STAGES],
      e_h2a[PP_CODEC_MAX_STAGES];
  long eT[PP_CODEC_MAX_STAGES + 1];  // samples per call at each encoder stage: eT[0] = samples per frame
  std::vector<HistSpec> ehist;      // conv_in, then res_a_j / down_j, then conv_out
  int e_conv_in, e_res[PP_CODEC_MAX_STAGES], e_down[PP_CODEC_MAX_STAGES], e_conv_out;
  size_t total;
};

CodecLayout make_codec_layout(const pp_codec_dims& dm, int B) {
  CodecLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + ALIGN - 1) / ALIGN * ALIGN;
    return o;
  };
  const long d = dm.d, H = dm.n_heads, hd = d / H, F = dm.ffn, W = dm.window;
  L.ring_layer_elems = 2 * H * W * hd;
  L.ring_slot_elems = dm.n_layers * L.ring_layer_elems;
  L.ring_v_off = H * W * hd;
  L.ti = take((size_t)B * TI_STRIDE * 4);
  L.codes = take((size_t)B * 16 * 4);
  L.inv_freq = take((size_t)hd / 2 * 8);
  L.rope = take((size_t)B * hd * 4);
  L.x = take((size_t)B * d * 4);
  L.xa = take((size_t)2 * B * d * 2);
  L.part = take((size_t)B * (d / 16) * 4);
  L.q = take((size_t)B * d * 4);
  L.o = take((size_t)2 * B * d * 2);
  L.m = take((size_t)2 * B * F * 2);
  L.ring = take((size_t)B * L.ring_slot_elems * 2);
  L.att_part = take((size_t)B * H * (hd + 2) * 4);
  L.att_cnt = take((size_t)B * H * 4);
  L.z = take((size_t)B * d * 4);
  L.T[0] = 1;
  for (int i = 0; i < dm.n_stages; ++i) L.T[i + 1] = L.T[i] * dm.strides[i];
  L.h0a = take((size_t)B * dm.channels[0] * 4);
  for (int i = 0; i < dm.n_stages; ++i) {
    const long co = dm.channels[i + 1], T = L.T[i + 1];
    L.u[i] = take((size_t)B * co * T * 4);
    L.ua[i] = take((size_t)B * co * T * 4);
    L.ra[i] = take((size_t)B * (co / 2) * T * 4);
    L.ha[i] = take((size_t)B * co * T * 4);
  }
  L.pcm = take((size_t)B * L.T[dm.n_stages] * 4);
  auto add_hist = [&](int C, int Hh) {
    if (Hh <= 0) return -1;
    HistSpec s{C, Hh, {0, 0, 0}};
    L.hist.push_back(s);
    return (int)L.hist.size() - 1;
  };
  L.h_conv_in = add_hist(dm.d, dm.conv_k - 1);
  for (int i = 0; i < dm.n_stages; ++i) {
    L.h_up[i] = add_hist(dm.channels[i], 1);
    L.h_res[i] = add_hist(dm.channels[i + 1], dm.res_k - 1);
  }
  L.h_conv_out = add_hist(dm.channels[dm.n_stages], dm.conv_k - 1);
  for (int set = 0; set < 3; ++set)
    for (auto& s : L.hist) s.off[set] = take((size_t)B * s.C * s.H * 4);

  const int n = dm.n_stages;
  const long S = L.T[n];
  L.pcm_in = take((size_t)B * S * 4);
  L.e_ti = take((size_t)B * TI_STRIDE * 4);
  L.e_rope = take((size_t)B * hd * 4);
  L.e_ring = take((size_t)B * L.ring_slot_elems * 2);
  L.e_y = take((size_t)B * d * 4);
  L.e_z = take((size_t)B * d * 4);
  L.e_codes = take((size_t)B * 16 * 4);
  L.e_qv = take((size_t)2 * B * rvq_tiles(dm.card) * 4);
  L.e_qi = take((size_t)2 * B * rvq_tiles(dm.card) * 4);
  L.e_qr = take((size_t)2 * B * d * 4);
  L.eT[0] = S;
  for (int j = 0; j < n; ++j) L.eT[j + 1] = L.eT[j] / dm.strides[n - 1 - j];
  for (int j = 0; j <= n; ++j) {
    const long C = dm.channels[n - j];
    L.e_h[j] = take((size_t)B * C * L.eT[j] * 4);
    L.e_ha[j] = take((size_t)B * C * L.eT[j] * 4);
    if (j < n) {
      L.e_ra[j] = take((size_t)B * (C / 2) * L.eT[j] * 4);
      L.e_h2a[j] = take((size_t)B * C * L.eT[j] * 4);
    }
  }
  auto add_ehist = [&](int C, int Hh) {
    if (Hh <= 0) return -1;
    L.ehist.push_back(HistSpec{C, Hh, {0, 0, 0}});
    return (int)L.ehist.size() - 1;
  };
  L.e_conv_in = add_ehist(1, dm.conv_k - 1);
  for (int j = 0; j < n; ++j) {
    L.e_res[j] = add_ehist(dm.channels[n - j], dm.res_k - 1);
    L.e_down[j] = add_ehist(dm.channels[n - j], dm.strides[n - 1 - j]);
  }
  L.e_conv_out = add_ehist(dm.channels[0], dm.conv_k - 1);
  for (int set = 0; set < 3; ++set)
    for (auto& s : L.ehist) s.off[set] = take((size_t)B * s.C * s.H * 4);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace pp

using namespace pp;

struct pp_codec {
  pp_codec_dims dm{};
  int B = 0;
  long S = 0;
  pp_codec_weights w{};
  CodecLayout lay;
  char* arena = nullptr;
  hipStream_t stream = nullptr;  // caller's
  hipStream_t cap = nullptr;     // capture stream
  // graphs [p][o]: read history set p, write set o = 1 - p (decode calls)
  // or set 2 (timing launches)
  hipGraph_t graph[2][2] = {};
  hipGraphExec_t exec[2][2] = {};
  hipGraph_t e_graph[2][2] = {};  // the encoder's, the same way
  hipGraphExec_t e_exec[2][2] = {};
  int parity = 0, e_parity = 0;
  std::vector<int> pos, e_pos;
  int32_t* ti_host = nullptr;     // pinned [B][TI_STRIDE]
  int32_t* codes_host = nullptr;  // pinned [B][16]
  float* pcm_host = nullptr;      // pinned [B][S]
  int32_t* e_ti_host = nullptr;   // pinned [B][TI_STRIDE]
  float* pcm_in_host = nullptr;   // pinned [B][S]
  int32_t* e_codes_host = nullptr;  // pinned [B][16]
  bool poisoned = false;
  std::string err;

  template <class T>
  T* at(size_t off) const {
    return reinterpret_cast<T*>(arena + off);
  }
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

#define CODEC_HIP_OR_FAIL(h, call)                                                       \
  do {                                                                                   \
    const hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) return (h)->fail(PP_EDEVICE, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

namespace {

// One direction's transformer weights.
struct TfWeights {
  const uint16_t *wqkv, *wo, *w_in, *w_out;
  const float *attn_norm, *mlp_norm, *out_norm;
};

// The transformer for one frame per slot: its input (the codebook sum of
// `codes`, or the latent y), the layers against the ring at `ring` with
// positions at `ti`, and the output norm into `z`.
void record_transformer(pp_codec* h, hipStream_t s, const TfWeights& tw, size_t ti_off, size_t rope_off,
                        size_t ring_off, size_t z_off, const float* y, const int* codes) {
  const pp_codec_dims& dm = h->dm;
  const CodecLayout& L = h->lay;
  const int B = h->B, d = dm.d, H = dm.n_heads, hd = d / H, F = dm.ffn, W = dm.window;
  const int* ti = h->at<int>(ti_off);

  CodecEmbedArgs ea{};
  ea.y = y;
  ea.codes = codes;
  ea.ti = ti;
  ea.B = B;
  ea.d = d;
  ea.n_q = dm.n_q;
  ea.card = dm.card;
  ea.codebooks = reinterpret_cast<const bf16_t*>(h->w.codebooks);
  ea.alpha = tw.attn_norm;
  ea.x = h->at<float>(L.x);
  ea.xa = h->at<bf16_t>(L.xa);
  ea.xa_lo = (long)B * d;
  ea.part = h->at<float>(L.part);
  ea.inv_freq = h->at<double>(L.inv_freq);
  ea.head_dim = hd;
  ea.rope = h->at<float>(rope_off);
  launch_codec_embed(ea, s);

  const long pq = packed_elems(3 * d, d), pwo = packed_elems(d, d), pi = packed_elems(2 * F, d),
             pd = packed_elems(d, F);
  // From 8 slots on, the codec's matrices (a few MB per layer) are loaded as
  // cache-resident weights: that lets the GEMMs split the batch into slot
  // groups, each re-reading the weights from the cache with fewer activation
  // bytes per workgroup (decode call at B = 32: 0.545 against 0.638 ms; at
  // B = 8: 0.396 against 0.417 ms; at B = 1 streamed weights stay faster,
  // 0.288 against 0.300 ms).  The arithmetic is the same either way.
  const int KEEP = B >= 8 ? 1 : 0;
  for (int l = 0; l < dm.n_layers; ++l) {
    bf16_t* ring_l = h->at<bf16_t>(ring_off) + (long)l * L.ring_layer_elems;
    GemmArgs g{};
    g.W = reinterpret_cast<const bf16_t*>(tw.wqkv) + (long)l * pq;
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
    g.inv_freq = h->at<double>(L.inv_freq);
    g.rope = h->at<float>(rope_off);
    g.w_keep = KEEP;
    launch_gemm(EPI_QKV, g, s);

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
    at.part = h->at<float>(L.att_part);
    at.max_chunks = 1;
    at.o = h->at<bf16_t>(L.o);
    at.ldo = d;
    at.o_lo = (long)B * d;
    at.cnt = h->at<unsigned>(L.att_cnt);
    launch_attention(at, s);

    GemmArgs go{};
    go.W = reinterpret_cast<const bf16_t*>(tw.wo) + (long)l * pwo;
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
    go.alpha_next = tw.mlp_norm + (long)l * d;
    go.part_out = h->at<float>(L.part);
    go.w_keep = KEEP;
    launch_gemm(EPI_RESID, go, s);

    GemmArgs gu{};
    gu.W = reinterpret_cast<const bf16_t*>(tw.w_in) + (long)l * pi;
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
    gu.w_keep = KEEP;
    launch_gemm(EPI_GATED, gu, s);

    GemmArgs gd{};
    gd.W = reinterpret_cast<const bf16_t*>(tw.w_out) + (long)l * pd;
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
    gd.alpha_next = (l + 1 < dm.n_layers) ? tw.attn_norm + (long)(l + 1) * d : tw.out_norm;
    gd.part_out = h->at<float>(L.part);
    gd.w_keep = KEEP;
    launch_gemm(EPI_RESID, gd, s);
  }

  CodecNormArgs na{};
  na.x = h->at<float>(L.x);
  na.part = h->at<float>(L.part);
  na.alpha = tw.out_norm;
  na.eps = dm.norm_eps;
  na.B = B;
  na.d = d;
  na.z = h->at<float>(z_off);
  launch_codec_norm(na, s);
}

// The whole decode of one call, recorded on stream s; reads history set p,
// writes set po.
void record_codec(pp_codec* h, hipStream_t s, int p, int po) {
  const pp_codec_dims& dm = h->dm;
  const CodecLayout& L = h->lay;
  const int B = h->B, d = dm.d;
  const pp_codec_weights& w = h->w;
  record_transformer(h, s, TfWeights{w.wqkv, w.wo, w.w_in, w.w_out, w.attn_norm, w.mlp_norm, w.out_norm}, L.ti,
                     L.rope, L.ring, L.z, nullptr, h->at<int>(L.codes));

  auto hist_in = [&](int e) { return e < 0 ? nullptr : h->at<float>(L.hist[e].off[p]); };
  auto hist_H = [&](int e) { return e < 0 ? 0 : L.hist[e].H; };
  const int* ch = dm.channels;

  ConvArgs c0{};
  c0.x = h->at<float>(L.z);
  c0.C_in = d;
  c0.T_in = 1;
  c0.hist = hist_in(L.h_conv_in);
  c0.H = hist_H(L.h_conv_in);
  c0.w = reinterpret_cast<const bf16_t*>(w.conv_in_w);
  c0.bias = w.conv_in_b;
  c0.C_out = ch[0];
  c0.K = dm.conv_k;
  c0.stride = 1;
  c0.ya = h->at<float>(L.h0a);
  c0.B = B;
  launch_codec_conv(c0, s);

  const float* hin = h->at<float>(L.h0a);  // the current stage's input, after its ELU
  for (int i = 0; i < dm.n_stages; ++i) {
    const int ci = ch[i], co = ch[i + 1];
    ConvArgs up{};
    up.x = hin;
    up.C_in = ci;
    up.T_in = (int)L.T[i];
    up.hist = hist_in(L.h_up[i]);
    up.H = 1;
    up.w = reinterpret_cast<const bf16_t*>(w.up_w[i]);
    up.bias = w.up_b[i];
    up.C_out = co;
    up.K = 2 * dm.strides[i];
    up.stride = dm.strides[i];
    up.transposed = 1;
    up.y = h->at<float>(L.u[i]);
    up.ya = h->at<float>(L.ua[i]);
    up.B = B;
    launch_codec_conv(up, s);

    ConvArgs ra{};
    ra.x = h->at<float>(L.ua[i]);
    ra.C_in = co;
    ra.T_in = (int)L.T[i + 1];
    ra.hist = hist_in(L.h_res[i]);
    ra.H = hist_H(L.h_res[i]);
    ra.w = reinterpret_cast<const bf16_t*>(w.res_a_w[i]);
    ra.bias = w.res_a_b[i];
    ra.C_out = co / 2;
    ra.K = dm.res_k;
    ra.stride = 1;
    ra.ya = h->at<float>(L.ra[i]);
    ra.B = B;
    launch_codec_conv(ra, s);

    ConvArgs rb{};
    rb.x = h->at<float>(L.ra[i]);
    rb.C_in = co / 2;
    rb.T_in = (int)L.T[i + 1];
    rb.hist = nullptr;
    rb.H = 0;
    rb.w = reinterpret_cast<const bf16_t*>(w.res_b_w[i]);
    rb.bias = w.res_b_b[i];
    rb.C_out = co;
    rb.K = 1;
    rb.stride = 1;
    rb.skip = h->at<float>(L.u[i]);
    rb.ya = h->at<float>(L.ha[i]);
    rb.B = B;
    launch_codec_conv(rb, s);
    hin = h->at<float>(L.ha[i]);
  }

  ConvArgs cz{};
  cz.x = hin;
  cz.C_in = ch[dm.n_stages];
  cz.T_in = (int)L.T[dm.n_stages];
  cz.hist = hist_in(L.h_conv_out);
  cz.H = hist_H(L.h_conv_out);
  cz.w = reinterpret_cast<const bf16_t*>(w.conv_out_w);
  cz.bias = w.conv_out_b;
  cz.C_out = 1;
  cz.K = dm.conv_k;
  cz.stride = 1;
  cz.y = h->at<float>(L.pcm);
  cz.B = B;
  launch_codec_conv(cz, s);

  // the histories for the next call
  HistArgs ha{};
  ha.B = B;
  auto entry = [&](int e, const float* x, int T) {
    if (e < 0) return;
    HistEntry& he = ha.e[ha.n++];
    he.x = x;
    he.C = L.hist[e].C;
    he.T = T;
    he.H = L.hist[e].H;
    he.old_h = h->at<float>(L.hist[e].off[p]);
    he.new_h = h->at<float>(L.hist[e].off[po]);
  };
  entry(L.h_conv_in, h->at<float>(L.z), 1);
  const float* xin = h->at<float>(L.h0a);
  for (int i = 0; i < dm.n_stages; ++i) {
    entry(L.h_up[i], xin, (int)L.T[i]);
    entry(L.h_res[i], h->at<float>(L.ua[i]), (int)L.T[i + 1]);
    xin = h->at<float>(L.ha[i]);
  }
  entry(L.h_conv_out, xin, (int)L.T[dm.n_stages]);
  launch_codec_hist(ha, s);
}

// The whole encode of one call, recorded on stream s; reads history set p,
// writes set po.
void record_encoder(pp_codec* h, hipStream_t s, int p, int po) {
  const pp_codec_dims& dm = h->dm;
  const CodecLayout& L = h->lay;
  const int B = h->B, d = dm.d, n = dm.n_stages;
  const pp_codec_weights& w = h->w;
  const int* ch = dm.channels;
  auto hist_in = [&](int e) { return e < 0 ? nullptr : h->at<float>(L.ehist[e].off[p]); };
  auto hist_H = [&](int e) { return e < 0 ? 0 : L.ehist[e].H; };

  ConvArgs c0{};
  c0.x = h->at<float>(L.pcm_in);
  c0.C_in = 1;
  c0.T_in = (int)L.eT[0];
  c0.hist = hist_in(L.e_conv_in);
  c0.H = hist_H(L.e_conv_in);
  c0.w = reinterpret_cast<const bf16_t*>(w.enc_conv_in_w);
  c0.bias = w.enc_conv_in_b;
  c0.C_out = ch[n];
  c0.K = dm.conv_k;
  c0.stride = 1;
  c0.y = h->at<float>(L.e_h[0]);
  c0.ya = h->at<float>(L.e_ha[0]);
  c0.B = B;
  launch_codec_conv(c0, s);
  for (int j = 0; j < n; ++j) {
    const int C = ch[n - j], st = dm.strides[n - 1 - j];
    const int T = (int)L.eT[j];
    ConvArgs ra{};
    ra.x = h->at<float>(L.e_ha[j]);
    ra.C_in = C;
    ra.T_in = T;
    ra.hist = hist_in(L.e_res[j]);
    ra.H = hist_H(L.e_res[j]);
    ra.w = reinterpret_cast<const bf16_t*>(w.enc_res_a_w[j]);
    ra.bias = w.enc_res_a_b[j];
    ra.C_out = C / 2;
    ra.K = dm.res_k;
    ra.stride = 1;
    ra.ya = h->at<float>(L.e_ra[j]);
    ra.B = B;
    launch_codec_conv(ra, s);

    ConvArgs rb{};
    rb.x = h->at<float>(L.e_ra[j]);
    rb.C_in = C / 2;
    rb.T_in = T;
    rb.w = reinterpret_cast<const bf16_t*>(w.enc_res_b_w[j]);
    rb.bias = w.enc_res_b_b[j];
    rb.C_out = C;
    rb.K = 1;
    rb.stride = 1;
    rb.skip = h->at<float>(L.e_h[j]);
    rb.ya = h->at<float>(L.e_h2a[j]);
    rb.B = B;
    launch_codec_conv(rb, s);

    ConvArgs dn{};
    dn.x = h->at<float>(L.e_h2a[j]);
    dn.C_in = C;
    dn.T_in = T;
    dn.hist = hist_in(L.e_down[j]);
    dn.H = hist_H(L.e_down[j]);
    dn.w = reinterpret_cast<const bf16_t*>(w.enc_down_w[j]);
    dn.bias = w.enc_down_b[j];
    dn.C_out = ch[n - 1 - j];
    dn.K = 2 * st;
    dn.stride = st;
    dn.strided = 1;
    dn.y = h->at<float>(L.e_h[j + 1]);
    dn.ya = h->at<float>(L.e_ha[j + 1]);
    dn.B = B;
    launch_codec_conv(dn, s);
  }
  ConvArgs cz{};
  cz.x = h->at<float>(L.e_ha[n]);
  cz.C_in = ch[0];
  cz.T_in = 1;
  cz.hist = hist_in(L.e_conv_out);
  cz.H = hist_H(L.e_conv_out);
  cz.w = reinterpret_cast<const bf16_t*>(w.enc_conv_out_w);
  cz.bias = w.enc_conv_out_b;
  cz.C_out = d;
  cz.K = dm.conv_k;
  cz.stride = 1;
  cz.y = h->at<float>(L.e_y);
  cz.B = B;
  launch_codec_conv(cz, s);

  record_transformer(h, s,
                     TfWeights{w.enc_wqkv, w.enc_wo, w.enc_w_in, w.enc_w_out, w.enc_attn_norm, w.enc_mlp_norm,
                               w.enc_out_norm},
                     L.e_ti, L.e_rope, L.e_ring, L.e_z, h->at<float>(L.e_y), nullptr);

  RvqArgs qa{};
  qa.z = h->at<float>(L.e_z);
  qa.B = B;
  qa.d = d;
  qa.n_q = dm.n_q;
  qa.card = dm.card;
  qa.codebooks = reinterpret_cast<const bf16_t*>(w.codebooks);
  qa.codes = h->at<int>(L.e_codes);
  qa.part_v = h->at<float>(L.e_qv);
  qa.part_i = h->at<int>(L.e_qi);
  qa.res = h->at<float>(L.e_qr);
  launch_codec_rvq(qa, s);

  HistArgs ha{};
  ha.B = B;
  auto entry = [&](int e, const float* x, int T) {
    if (e < 0) return;
    HistEntry& he = ha.e[ha.n++];
    he.x = x;
    he.C = L.ehist[e].C;
    he.T = T;
    he.H = L.ehist[e].H;
    he.old_h = h->at<float>(L.ehist[e].off[p]);
    he.new_h = h->at<float>(L.ehist[e].off[po]);
  };
  entry(L.e_conv_in, h->at<float>(L.pcm_in), (int)L.eT[0]);
  for (int j = 0; j < n; ++j) {
    entry(L.e_res[j], h->at<float>(L.e_ha[j]), (int)L.eT[j]);
    entry(L.e_down[j], h->at<float>(L.e_h2a[j]), (int)L.eT[j]);
  }
  entry(L.e_conv_out, h->at<float>(L.e_ha[n]), 1);
  launch_codec_hist(ha, s);
}

hipError_t capture_codec(pp_codec* h) {
  hipError_t e;
  for (int dir = 0; dir < 2; ++dir)
    for (int p = 0; p < 2; ++p)
      for (int t = 0; t < 2; ++t) {
        hipGraph_t& g = dir ? h->e_graph[p][t] : h->graph[p][t];
        hipGraphExec_t& x = dir ? h->e_exec[p][t] : h->exec[p][t];
        if ((e = hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal)) != hipSuccess) return e;
        if (dir) record_encoder(h, h->cap, p, t ? 2 : 1 - p);
        else record_codec(h, h->cap, p, t ? 2 : 1 - p);
        if ((e = hipStreamEndCapture(h->cap, &g)) != hipSuccess) return e;
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0)) != hipSuccess) return e;
      }
  return hipSuccess;
}

}  // namespace

extern "C" {

int pp_codec_samples(const pp_codec_dims* dims) {
  if (!codec_dims_ok(dims, nullptr)) return PP_EINVAL;
  return (int)codec_samples(*dims);
}

int pp_codec_arena_bytes(const pp_codec_dims* dims, int B, size_t* out_bytes) {
  if (!out_bytes || !codec_dims_ok(dims, nullptr) || B < 1 || B > PP_CODEC_MAX_BATCH) return PP_EINVAL;
  *out_bytes = make_codec_layout(*dims, B).total;
  return PP_OK;
}

int pp_codec_create(const pp_codec_dims* dims, int B, const pp_codec_weights* w, void* arena, size_t arena_bytes,
                    void* stream, pp_codec** out) {
  std::string why;
  if (!out) { g_codec_create_error = "out is NULL"; return PP_EINVAL; }
  *out = nullptr;
  if (!codec_dims_ok(dims, &why)) { g_codec_create_error = why; return PP_EINVAL; }
  if (B < 1 || B > PP_CODEC_MAX_BATCH) { g_codec_create_error = "B outside 1..PP_CODEC_MAX_BATCH"; return PP_EINVAL; }
  if (!w || !arena) { g_codec_create_error = "weights or arena is NULL"; return PP_EINVAL; }
  {
    const void* req[] = {w->codebooks, w->attn_norm, w->wqkv, w->wo, w->mlp_norm, w->w_in, w->w_out,
                         w->out_norm, w->conv_in_w, w->conv_in_b, w->conv_out_w, w->conv_out_b};
    for (const void* p : req)
      if (!p) { g_codec_create_error = "a weight pointer is NULL"; return PP_EINVAL; }
    const void* ereq[] = {w->enc_conv_in_w, w->enc_conv_in_b, w->enc_conv_out_w, w->enc_conv_out_b,
                          w->enc_attn_norm, w->enc_wqkv, w->enc_wo, w->enc_mlp_norm, w->enc_w_in, w->enc_w_out,
                          w->enc_out_norm};
    for (const void* p : ereq)
      if (!p) { g_codec_create_error = "an encoder weight pointer is NULL"; return PP_EINVAL; }
    for (int i = 0; i < dims->n_stages; ++i)
      if (!w->up_w[i] || !w->up_b[i] || !w->res_a_w[i] || !w->res_a_b[i] || !w->res_b_w[i] || !w->res_b_b[i] ||
          !w->enc_res_a_w[i] || !w->enc_res_a_b[i] || !w->enc_res_b_w[i] || !w->enc_res_b_b[i] || !w->enc_down_w[i] ||
          !w->enc_down_b[i]) {
        g_codec_create_error = "a stage weight pointer is NULL";
        return PP_EINVAL;
      }
  }
  if (reinterpret_cast<uintptr_t>(arena) % ALIGN) { g_codec_create_error = "arena not 256-byte aligned"; return PP_EINVAL; }
  CodecLayout lay = make_codec_layout(*dims, B);
  if (arena_bytes < lay.total) { g_codec_create_error = "arena too small"; return PP_ENOSPC; }

  pp_codec* h = new (std::nothrow) pp_codec();
  if (!h) { g_codec_create_error = "out of host memory"; return PP_ENOSPC; }
  h->dm = *dims;
  h->B = B;
  h->S = codec_samples(*dims);
  h->w = *w;
  h->lay = lay;
  h->arena = static_cast<char*>(arena);
  h->stream = static_cast<hipStream_t>(stream);
  h->pos.assign(B, 0);
  h->e_pos.assign(B, 0);
  auto bail = [&](const char* what, hipError_t e) {
    g_codec_create_error = std::string(what) + ": " + hipGetErrorString(e);
    pp_codec_destroy(h);
    return PP_EDEVICE;
  };
  hipError_t e;
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->ti_host), (size_t)B * TI_STRIDE * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->codes_host), (size_t)B * 16 * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->pcm_host), (size_t)B * h->S * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->e_ti_host), (size_t)B * TI_STRIDE * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->pcm_in_host), (size_t)B * h->S * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->e_codes_host), (size_t)B * 16 * 4, hipHostMallocDefault)) !=
      hipSuccess)
    return bail("hipHostMalloc", e);
  std::memset(h->ti_host, 0, (size_t)B * TI_STRIDE * 4);
  std::memset(h->codes_host, 0, (size_t)B * 16 * 4);
  std::memset(h->e_ti_host, 0, (size_t)B * TI_STRIDE * 4);
  std::memset(h->pcm_in_host, 0, (size_t)B * h->S * 4);

  const int hd = dims->d / dims->n_heads;
  std::vector<double> freq(hd / 2);
  for (int i = 0; i < hd / 2; ++i) freq[i] = std::pow((double)dims->rope_base, -2.0 * i / hd);
  if ((e = hipMemcpyAsync(h->at<double>(lay.inv_freq), freq.data(), freq.size() * 8, hipMemcpyHostToDevice,
                          h->stream)) != hipSuccess)
    return bail("hipMemcpyAsync", e);
  // every slot fresh: positions 0, zero histories (both sets), tickets zero
  if ((e = hipMemcpyAsync(h->at<int>(lay.ti), h->ti_host, (size_t)B * TI_STRIDE * 4, hipMemcpyHostToDevice,
                          h->stream)) != hipSuccess)
    return bail("hipMemcpyAsync", e);
  if ((e = hipMemcpyAsync(h->at<int>(lay.codes), h->codes_host, (size_t)B * 16 * 4, hipMemcpyHostToDevice,
                          h->stream)) != hipSuccess)
    return bail("hipMemcpyAsync", e);
  if ((e = hipMemcpyAsync(h->at<int>(lay.e_ti), h->e_ti_host, (size_t)B * TI_STRIDE * 4, hipMemcpyHostToDevice,
                          h->stream)) != hipSuccess)
    return bail("hipMemcpyAsync", e);
  if ((e = hipMemcpyAsync(h->at<float>(lay.pcm_in), h->pcm_in_host, (size_t)B * h->S * 4, hipMemcpyHostToDevice,
                          h->stream)) != hipSuccess)
    return bail("hipMemcpyAsync", e);
  if ((e = hipMemsetAsync(h->at<char>(lay.att_cnt), 0, (size_t)B * dims->n_heads * 4, h->stream)) != hipSuccess)
    return bail("hipMemsetAsync", e);
  for (const auto* hv : {&lay.hist, &lay.ehist})
    for (const auto& s : *hv)
      for (int set = 0; set < 3; ++set)
        if ((e = hipMemsetAsync(h->at<char>(s.off[set]), 0, (size_t)B * s.C * s.H * 4, h->stream)) != hipSuccess)
          return bail("hipMemsetAsync", e);
  if ((e = hipStreamSynchronize(h->stream)) != hipSuccess) return bail("hipStreamSynchronize", e);
  if ((e = hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking)) != hipSuccess) return bail("hipStreamCreate", e);
  if ((e = capture_codec(h)) != hipSuccess) return bail("graph capture", e);
  *out = h;
  return PP_OK;
}

int pp_codec_decode(pp_codec* h, const int32_t* codes, float* pcm) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (!codes || !pcm) return h->fail(PP_EINVAL, "codes or pcm is NULL");
  const int B = h->B, nq = h->dm.n_q;
  for (int b = 0; b < B; ++b)
    for (int q = 0; q < nq; ++q) {
      const int c = codes[b * nq + q];
      if (c < 0 || c >= h->dm.card) return h->fail(PP_EINVAL, "slot %d codebook %d: code %d outside [0, %d)", b, q, c, h->dm.card);
    }
  for (int b = 0; b < B; ++b) {
    h->ti_host[b * TI_STRIDE + TI_POS] = h->pos[b];
    for (int q = 0; q < nq; ++q) h->codes_host[b * nq + q] = codes[b * nq + q];
  }
  const CodecLayout& L = h->lay;
  CODEC_HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(L.ti), h->ti_host, (size_t)B * TI_STRIDE * 4, hipMemcpyHostToDevice,
                                      h->stream));
  CODEC_HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(L.codes), h->codes_host, (size_t)B * nq * 4, hipMemcpyHostToDevice,
                                      h->stream));
  CODEC_HIP_OR_FAIL(h, hipGraphLaunch(h->exec[h->parity][0], h->stream));
  CODEC_HIP_OR_FAIL(h, hipMemcpyAsync(h->pcm_host, h->at<float>(L.pcm), (size_t)B * h->S * 4, hipMemcpyDeviceToHost,
                                      h->stream));
  CODEC_HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  std::memcpy(pcm, h->pcm_host, (size_t)B * h->S * 4);
  for (int b = 0; b < B; ++b) ++h->pos[b];
  h->parity ^= 1;
  return PP_OK;
}

int pp_codec_encode(pp_codec* h, const float* pcm, int32_t* codes) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (!codes || !pcm) return h->fail(PP_EINVAL, "pcm or codes is NULL");
  const int B = h->B, nq = h->dm.n_q;
  const long S = h->S;
  for (long i = 0; i < (long)B * S; ++i)
    if (!std::isfinite(pcm[i])) return h->fail(PP_EINVAL, "slot %ld sample %ld is not finite", i / S, i % S);
  for (int b = 0; b < B; ++b) h->e_ti_host[b * TI_STRIDE + TI_POS] = h->e_pos[b];
  std::memcpy(h->pcm_in_host, pcm, (size_t)B * S * 4);
  const CodecLayout& L = h->lay;
  CODEC_HIP_OR_FAIL(h, hipMemcpyAsync(h->at<int>(L.e_ti), h->e_ti_host, (size_t)B * TI_STRIDE * 4,
                                      hipMemcpyHostToDevice, h->stream));
  CODEC_HIP_OR_FAIL(h, hipMemcpyAsync(h->at<float>(L.pcm_in), h->pcm_in_host, (size_t)B * S * 4,
                                      hipMemcpyHostToDevice, h->stream));
  CODEC_HIP_OR_FAIL(h, hipGraphLaunch(h->e_exec[h->e_parity][0], h->stream));
  CODEC_HIP_OR_FAIL(h, hipMemcpyAsync(h->e_codes_host, h->at<int>(L.e_codes), (size_t)B * nq * 4,
                                      hipMemcpyDeviceToHost, h->stream));
  CODEC_HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  std::memcpy(codes, h->e_codes_host, (size_t)B * nq * 4);
  for (int b = 0; b < B; ++b) ++h->e_pos[b];
  h->e_parity ^= 1;
  return PP_OK;
}

int pp_codec_reset(pp_codec* h, int slot) {
  if (!h) return PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  if (slot < 0 || slot >= h->B) return h->fail(PP_EINVAL, "slot %d outside [0, %d)", slot, h->B);
  // the set the next call reads
  for (const auto& s : h->lay.hist)
    CODEC_HIP_OR_FAIL(h, hipMemsetAsync(h->at<char>(s.off[h->parity]) + (size_t)slot * s.C * s.H * 4, 0,
                                        (size_t)s.C * s.H * 4, h->stream));
  for (const auto& s : h->lay.ehist)
    CODEC_HIP_OR_FAIL(h, hipMemsetAsync(h->at<char>(s.off[h->e_parity]) + (size_t)slot * s.C * s.H * 4, 0,
                                        (size_t)s.C * s.H * 4, h->stream));
  CODEC_HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  h->pos[slot] = 0;
  h->e_pos[slot] = 0;
  return PP_OK;
}

namespace {
int time_graphs(pp_codec* h, hipGraphExec_t (&ex)[2][2], int parity, int iters, float* avg_ms) {
  if (!avg_ms || iters < 1) return h->fail(PP_EINVAL, "bad arguments");
  if (h->poisoned) return PP_EDEVICE;
  // the last call's work again: it reads the history set the last call read
  // and writes the timing set, so the set the next call reads is untouched;
  // the ring entry it rewrites (the last call's position) gets the same key
  // and value, or, for a slot reset since, lies outside that slot's window
  // until the slot's own calls overwrite it
  const int p = parity ^ 1;
  hipEvent_t e0, e1;
  CODEC_HIP_OR_FAIL(h, hipEventCreate(&e0));
  CODEC_HIP_OR_FAIL(h, hipEventCreate(&e1));
  CODEC_HIP_OR_FAIL(h, hipGraphLaunch(ex[p][1], h->stream));  // warm
  CODEC_HIP_OR_FAIL(h, hipEventRecord(e0, h->stream));
  for (int i = 0; i < iters; ++i) CODEC_HIP_OR_FAIL(h, hipGraphLaunch(ex[p][1], h->stream));
  CODEC_HIP_OR_FAIL(h, hipEventRecord(e1, h->stream));
  CODEC_HIP_OR_FAIL(h, hipEventSynchronize(e1));
  float ms = 0.f;
  CODEC_HIP_OR_FAIL(h, hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *avg_ms = ms / iters;
  return PP_OK;
}
}  // namespace

int pp_codec_time(pp_codec* h, int iters, float* avg_ms) {
  return h ? time_graphs(h, h->exec, h->parity, iters, avg_ms) : PP_EINVAL;
}

int pp_codec_time_encode(pp_codec* h, int iters, float* avg_ms) {
  return h ? time_graphs(h, h->e_exec, h->e_parity, iters, avg_ms) : PP_EINVAL;
}

int pp_codec_taps(pp_codec* h, pp_codec_taps_t* out) {
  if (!h || !out) return h ? h->fail(PP_EINVAL, "out is NULL") : PP_EINVAL;
  if (h->poisoned) return PP_EDEVICE;
  CODEC_HIP_OR_FAIL(h, hipStreamSynchronize(h->stream));
  out->ring = h->at<uint16_t>(h->lay.ring);
  out->z = h->at<float>(h->lay.z);
  out->enc_ring = h->at<uint16_t>(h->lay.e_ring);
  out->enc_y = h->at<float>(h->lay.e_y);
  out->enc_z = h->at<float>(h->lay.e_z);
  return PP_OK;
}

void pp_codec_destroy(pp_codec* h) {
  if (!h) return;
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  for (int p = 0; p < 2; ++p)
    for (int t = 0; t < 2; ++t) {
      if (h->exec[p][t]) (void)hipGraphExecDestroy(h->exec[p][t]);
      if (h->graph[p][t]) (void)hipGraphDestroy(h->graph[p][t]);
      if (h->e_exec[p][t]) (void)hipGraphExecDestroy(h->e_exec[p][t]);
      if (h->e_graph[p][t]) (void)hipGraphDestroy(h->e_graph[p][t]);
    }
  if (h->cap) (void)hipStreamDestroy(h->cap);
  if (h->ti_host) (void)hipHostFree(h->ti_host);
  if (h->codes_host) (void)hipHostFree(h->codes_host);
  if (h->pcm_host) (void)hipHostFree(h->pcm_host);
  if (h->e_ti_host) (void)hipHostFree(h->e_ti_host);
  if (h->pcm_in_host) (void)hipHostFree(h->pcm_in_host);
  if (h->e_codes_host) (void)hipHostFree(h->e_codes_host);
  delete h;
}

const char* pp_codec_last_error(const pp_codec* h) {
  return h ? h->err.c_str() : g_codec_create_error.c_str();
}

}  // extern "C"
