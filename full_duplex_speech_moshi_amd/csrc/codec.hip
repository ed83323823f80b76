// Streaming codec kernels for gfx950, both directions: the transformer's
// input (the codebook sum, or the encoder's latent), the output norm, the
// causal, transposed and strided convolutions, residual vector quantisation,
// and the streaming-state update.
//
// chenxutan.com PersonaPlex article, section 2.3 on Mimi: a causal codec of
// the SoundStream / EnCodec family between 24 kHz audio and 12.5 Hz frames
// of codebook indices; PersonaPlex recipe, "Architecture": 8 codebooks of
// 2048 entries, 1920 samples per 80 ms frame.  The layer structure is this
// library's reading of that family (codec.h).  The work is small and
// latency-bound (at most a few hundred thousand outputs per call, each a sum
// of 8 to 3584 products), so the convolutions are direct sums on the vector
// ALU in fp32, each output's sum in an order fixed by the layer's shape, so
// that a slot's result depends only on its own inputs.
#include "codec_kernels.h"
#include "device.h"

namespace pp {

// ---------------------------------------------------------------------------
// Transformer input: x = the sum of the n_q codebooks' rows in codebook order
// (fp32; the decoder) or the given latent (the encoder), with x * alpha as a
// bf16 pair and the per-16 sums of squares for the first layer's QKV launch,
// and the frame's RoPE table.  One thread per 8 features.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void codec_embed_kernel(CodecEmbedArgs a) {
  const int b = blockIdx.y;
  if (blockIdx.x == 0) {
    const int pos = a.ti[b * TI_STRIDE + TI_POS];
    for (int i = threadIdx.x; i < a.head_dim / 2; i += blockDim.x) {
      const double th = (double)pos * a.inv_freq[i];
      a.rope[(long)b * a.head_dim + 2 * i] = (float)cos(th);
      a.rope[(long)b * a.head_dim + 2 * i + 1] = (float)sin(th);
    }
  }
  const int g8 = blockIdx.x * blockDim.x + threadIdx.x;
  if (g8 >= a.d / 8) return;  // d % 16 == 0: 16-feature groups stay whole
  const int* c = a.codes + (long)b * a.n_q;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = a.y ? a.y[(long)b * a.d + g8 * 8 + i] : 0.f;
  for (int q = 0; q < (a.y ? 0 : a.n_q); ++q) {
    const u32x4 v = ld16(a.codebooks + ((long)q * a.card + c[q]) * a.d + g8 * 8);
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += f[i];
  }
  const long off = (long)b * a.d + g8 * 8;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a.x[off + i] = acc[i];
    store_split(a.xa + off + i, a.xa_lo, acc[i] * a.alpha[g8 * 8 + i]);
    ss += acc[i] * acc[i];
  }
  ss += __shfl_xor(ss, 1);  // the two halves of a 16-feature group are adjacent lanes
  if ((g8 & 1) == 0) a.part[(long)b * (a.d / 16) + g8 / 2] = ss;
}

void launch_codec_embed(const CodecEmbedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(codec_embed_kernel, dim3((a.d / 8 + 255) / 256, a.B), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// Output norm: z = x * alpha / sqrt(mean(x^2) + eps), the mean from the last
// down-projection's per-16 sums of squares added in a fixed tree.  One
// workgroup per slot.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void codec_norm_kernel(CodecNormArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ float red[256];
  const int np = a.d / 16;
  float s = 0.f;
  for (int i = tid; i < np; i += 256) s += a.part[(long)b * np + i];
  red[tid] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / (float)a.d + a.eps);
  for (int i = tid; i < a.d; i += 256) a.z[(long)b * a.d + i] = a.x[(long)b * a.d + i] * a.alpha[i] * inv;
}

void launch_codec_norm(const CodecNormArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(codec_norm_kernel, dim3(a.B), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// Convolutions.  Every form is a sum over (input channel i, tap k) of
// w[o][i][k] x_ext(i, tau), where x_ext is this call's input after the
// stream's history (times -H .. -1) and tau depends on the form: causal
// t - (K-1) + k; strided t s - s + k; transposed (output m s + r, taps r and
// r + s) m and m - 1.  The inputs arrive already activated.  The output is
// bias + sum (+ skip), stored raw and/or after ELU.
//
// The order of the sum is fixed by the layer's shape alone, never by the
// batch or the launch shape, so every batch size gives the same bits:
//   * few input channels (at most CONV_CHAIN_C): one FMA chain per output
//     over i ascending and, within i, k ascending (transposed: tap r, then
//     tap r + s), from zero (codec_conv_chain_kernel);
//   * more input channels: the LANES lanes of a workgroup (256 above
//     CONV_WIDE_KD terms per output, else 64) take the reduction index
//     kd = lane, lane + LANES, ... (kd = i K + k; transposed kd = 2 i + j for
//     tap r + j s), each as one FMA chain from zero; lane sums are then added
//     in runs of 32 lanes, each run in lane order from zero, and the run sums
//     in run order from zero (codec_conv_split_kernel).
// ---------------------------------------------------------------------------
constexpr int CONV_CHAIN_C = 32;    // input channels up to which one lane sums an output
constexpr int CONV_WIDE_KD = 256;   // terms per output above which 256 lanes share a sum

__device__ __forceinline__ float elu_f(float v) { return v > 0.f ? v : expm1f(v); }

// x_ext(i, tau) of slot b, tau >= -H
__device__ __forceinline__ float conv_x(const ConvArgs& a, int b, int i, int tau) {
  return tau >= 0 ? a.x[((long)b * a.C_in + i) * a.T_in + tau] : a.hist[((long)b * a.C_in + i) * a.H + a.H + tau];
}

// the per-slot output columns and the rows of the form (transposed: rows
// (o, r), row o s + r)
__device__ __forceinline__ int conv_cols(const ConvArgs& a) { return a.strided ? a.T_in / a.stride : a.T_in; }
__device__ __forceinline__ int conv_rows(const ConvArgs& a) { return a.transposed ? a.C_out * a.stride : a.C_out; }

// bias + v (+ skip) of (row, slot b, column t), stored raw and/or after ELU
__device__ __forceinline__ void conv_out(const ConvArgs& a, int row, int b, int t, float v) {
  int o = row, to = t, T_out = a.T_in;
  if (a.transposed) {
    o = row / a.stride;
    to = t * a.stride + (row - o * a.stride);
    T_out = a.T_in * a.stride;
  } else if (a.strided) {
    T_out = a.T_in / a.stride;
  }
  const long idx = ((long)b * a.C_out + o) * T_out + to;
  float y = a.bias[o] + v;
  if (a.skip) y += a.skip[idx];
  if (a.y) a.y[idx] = y;
  if (a.ya) a.ya[idx] = elu_f(y);
}

// Split sums: a workgroup of LANES lanes (64 or 256) computes OC rows x NC
// columns (column = slot * columns per slot + t), E = OC NC <= 32 outputs.
template <int LANES, int OC, int NC>
__global__ __launch_bounds__(LANES) void codec_conv_split_kernel(ConvArgs a) {
  constexpr int E = OC * NC, RUNS = LANES / 32;
  static_assert(E <= 32 && LANES % 32 == 0, "at most 32 outputs; runs of 32 lanes");
  __shared__ float red[LANES][E + 1];
  __shared__ float run[RUNS][E];
  const int tid = threadIdx.x;
  const int Tc = conv_cols(a), Mr = conv_rows(a), KK = a.transposed ? 2 : a.K, Kd = a.C_in * KK;
  const int s = a.stride, row0 = blockIdx.y * OC;
  const long ncols = (long)a.B * Tc, col0 = (long)blockIdx.x * NC;
  int cb[NC], ct[NC];
  bool cok[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const long col = col0 + c;
    cok[c] = col < ncols;
    const long cc = cok[c] ? col : 0;
    cb[c] = (int)(cc / Tc);
    ct[c] = (int)(cc - (long)cb[c] * Tc);
  }
  // weight row offsets (transposed: o's row and the phase r)
  long wro[OC];
  int wph[OC];
  bool rok[OC];
#pragma unroll
  for (int oc = 0; oc < OC; ++oc) {
    const int row = row0 + oc;
    rok[oc] = row < Mr;
    const int rr = rok[oc] ? row : 0;
    const int o = a.transposed ? rr / s : rr;
    wph[oc] = a.transposed ? rr - o * s : 0;
    wro[oc] = (long)o * a.C_in * a.K;
  }
  float acc[OC][NC];
#pragma unroll
  for (int oc = 0; oc < OC; ++oc)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[oc][c] = 0.f;
  // four reduction steps' loads in flight at once
#pragma unroll 4
  for (int kd = tid; kd < Kd; kd += LANES) {
    const int i = kd / KK, k = kd - i * KK;
    float wv[OC];
#pragma unroll
    for (int oc = 0; oc < OC; ++oc) {
      const int tap = a.transposed ? wph[oc] + k * s : k;
      wv[oc] = rok[oc] ? bf2f(a.w[wro[oc] + (long)i * a.K + tap]) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!cok[c]) continue;  // uniform over the workgroup
      const int tau = a.transposed ? ct[c] - k : a.strided ? ct[c] * s - s + k : ct[c] - (a.K - 1) + k;
      const float xv = conv_x(a, cb[c], i, tau);
#pragma unroll
      for (int oc = 0; oc < OC; ++oc) acc[oc][c] = __builtin_fmaf(wv[oc], xv, acc[oc][c]);
    }
  }
#pragma unroll
  for (int oc = 0; oc < OC; ++oc)
#pragma unroll
    for (int c = 0; c < NC; ++c) red[tid][oc * NC + c] = acc[oc][c];
  __syncthreads();
  // run p of output e: lanes 32 p .. 32 p + 31 in lane order
  for (int t = tid; t < RUNS * E; t += LANES) {
    const int e = t % E, p = t / E;
    float v = 0.f;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) v += red[p * 32 + j][e];
    run[p][e] = v;
  }
  __syncthreads();
  if (tid < E) {
    float v = 0.f;
#pragma unroll
    for (int p = 0; p < RUNS; ++p) v += run[p][tid];
    const int oc = tid / NC, c = tid - oc * NC;
    const int row = row0 + oc;
    const long col = col0 + c;
    if (row < Mr && col < ncols) {
      const int b = (int)(col / Tc);
      conv_out(a, row, b, (int)(col - (long)b * Tc), v);
    }
  }
}

// Chained sums: workgroup (thread block, channel block) stages the OC output
// channels' weights in LDS as fp32 [C_in][K][OC]; thread n owns TT
// consecutive columns of those channels for slot n / (column tiles per
// slot) (transposed: TT input positions, S outputs each; strided: S is the
// stride; for the causal form S is the kernel K).  FORM 0 causal,
// 1 strided, 2 transposed.
template <int FORM, int OC, int TT, int S>
__global__ __launch_bounds__(256) void codec_conv_chain_kernel(ConvArgs a) {
  extern __shared__ float wl[];
  constexpr int K = FORM == 0 ? S : 2 * S;
  const int tid = threadIdx.x, o0 = blockIdx.y * OC;
  for (int e = tid; e < a.C_in * K * OC; e += 256) {
    const int oc = e % OC, k = (e / OC) % K, i = e / (OC * K);
    const int o = o0 + oc;
    wl[e] = o < a.C_out ? bf2f(a.w[((long)o * a.C_in + i) * K + k]) : 0.f;
  }
  __syncthreads();
  const int Tc = FORM == 1 ? a.T_in / S : a.T_in;
  const int nt = (Tc + TT - 1) / TT;
  const long n = (long)blockIdx.x * 256 + tid;
  if (n >= (long)a.B * nt) return;
  const int b = (int)(n / nt), t0 = (int)(n - (long)b * nt) * TT;
  // inputs the thread's taps reach, from time tau0
  constexpr int NW = FORM == 0 ? TT + K - 1 : FORM == 1 ? TT * S + S : TT + 1;
  const int tau0 = FORM == 0 ? t0 - (K - 1) : FORM == 1 ? t0 * S - S : t0 - 1;
  constexpr int NO = FORM == 2 ? TT * S : TT;  // outputs per channel
  float acc[OC][NO];
#pragma unroll
  for (int oc = 0; oc < OC; ++oc)
#pragma unroll
    for (int u = 0; u < NO; ++u) acc[oc][u] = 0.f;
  // several channels' loads in flight at once: more for small tiles
  // (a channel holds NW inputs and K x OC weights in registers: about 96 of
  // them over the channels in flight, at most 32 channels)
  constexpr int PER_CH = NW + K * OC;
  constexpr int UNR = PER_CH * 32 <= 96 ? 32 : PER_CH * 16 <= 96 ? 16 : PER_CH * 8 <= 96 ? 8
                      : PER_CH * 4 <= 96 ? 4 : PER_CH * 2 <= 96 ? 2 : 1;
#pragma unroll UNR
  for (int i = 0; i < a.C_in; ++i) {
    float xw[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int tau = tau0 + j;
      // past this call's inputs only for a slot's last tile
      xw[j] = tau < a.T_in ? conv_x(a, b, i, tau) : 0.f;
    }
    const float* wi = wl + (long)i * K * OC;
    if constexpr (FORM == 0) {
#pragma unroll
      for (int k = 0; k < K; ++k)
#pragma unroll
        for (int oc = 0; oc < OC; ++oc) {
          const float w = wi[k * OC + oc];
#pragma unroll
          for (int u = 0; u < TT; ++u) acc[oc][u] = __builtin_fmaf(w, xw[u + k], acc[oc][u]);
        }
    } else if constexpr (FORM == 1) {
#pragma unroll
      for (int k = 0; k < 2 * S; ++k)
#pragma unroll
        for (int oc = 0; oc < OC; ++oc) {
          const float w = wi[k * OC + oc];
#pragma unroll
          for (int u = 0; u < TT; ++u) acc[oc][u] = __builtin_fmaf(w, xw[u * S + k], acc[oc][u]);
        }
    } else {
      // output (u, r): tap r on input t0 + u (xw[u + 1]), then tap r + S on
      // input t0 + u - 1 (xw[u])
#pragma unroll
      for (int r = 0; r < S; ++r)
#pragma unroll
        for (int oc = 0; oc < OC; ++oc) {
          const float w0 = wi[r * OC + oc], w1 = wi[(r + S) * OC + oc];
#pragma unroll
          for (int u = 0; u < TT; ++u) {
            acc[oc][u * S + r] = __builtin_fmaf(w0, xw[u + 1], acc[oc][u * S + r]);
            acc[oc][u * S + r] = __builtin_fmaf(w1, xw[u], acc[oc][u * S + r]);
          }
        }
    }
  }
#pragma unroll
  for (int oc = 0; oc < OC; ++oc) {
    if (o0 + oc >= a.C_out) continue;
#pragma unroll
    for (int u = 0; u < TT; ++u) {
      if (t0 + u >= Tc) continue;
      if constexpr (FORM == 2) {
#pragma unroll
        for (int r = 0; r < S; ++r) conv_out(a, (o0 + oc) * S + r, b, t0 + u, acc[oc][u * S + r]);
      } else {
        conv_out(a, o0 + oc, b, t0 + u, acc[oc][u]);
      }
    }
  }
}

// Threads a chained-sum launch should reach before its tile grows.
constexpr long CONV_THREADS = 1L << 15;

template <int FORM, int OC, int TT, int S>
static void launch_chain(const ConvArgs& a, hipStream_t st, int Tc) {
  const long threads = (long)a.B * ((Tc + TT - 1) / TT);
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)((a.C_out + OC - 1) / OC));
  const size_t lds = (size_t)a.C_in * a.K * OC * 4;
  hipLaunchKernelGGL((codec_conv_chain_kernel<FORM, OC, TT, S>), grid, dim3(256), lds, st, a);
}

// Chained-sum launch shape (the arithmetic does not depend on it): the largest
// tile of OC output channels x TT columns that still gives CONV_THREADS
// threads, else one output channel and one column per thread.
template <int FORM, int S>
static void launch_chain_tile(const ConvArgs& a, hipStream_t st, int Tc) {
  auto threads = [&](int oc, int tt) { return (long)a.B * ((a.C_out + oc - 1) / oc) * ((Tc + tt - 1) / tt); };
  if constexpr (FORM == 0) {  // S = K
    if (a.C_out >= 8 && threads(8, 4) >= CONV_THREADS) launch_chain<0, 8, 4, S>(a, st, Tc);
    else if (a.C_out >= 8 && threads(8, 2) >= CONV_THREADS) launch_chain<0, 8, 2, S>(a, st, Tc);
    else if (a.C_out >= 4 && threads(4, 1) >= CONV_THREADS) launch_chain<0, 4, 1, S>(a, st, Tc);
    else launch_chain<0, 1, 1, S>(a, st, Tc);
  } else if constexpr (FORM == 1) {
    if (a.C_out >= 8 && threads(8, 2) >= CONV_THREADS) launch_chain<1, 8, 2, S>(a, st, Tc);
    else if (a.C_out >= 4 && threads(4, 1) >= CONV_THREADS) launch_chain<1, 4, 1, S>(a, st, Tc);
    else launch_chain<1, 1, 1, S>(a, st, Tc);
  } else {
    constexpr int TT = S >= 8 ? 1 : 8 / S;
    if (a.C_out >= 4 && threads(4, TT) >= CONV_THREADS) launch_chain<2, 4, TT, S>(a, st, Tc);
    else launch_chain<2, 1, 1, S>(a, st, Tc);
  }
}

// FORM 0: by the kernel K; else by the stride
template <int FORM>
static void launch_chain_s(const ConvArgs& a, hipStream_t st, int Tc) {
  switch (FORM == 0 ? a.K : a.stride) {
    case 1: launch_chain_tile<FORM, 1>(a, st, Tc); break;
    case 2: launch_chain_tile<FORM, 2>(a, st, Tc); break;
    case 3: launch_chain_tile<FORM, 3>(a, st, Tc); break;
    case 4: launch_chain_tile<FORM, 4>(a, st, Tc); break;
    case 5: launch_chain_tile<FORM, 5>(a, st, Tc); break;
    case 6: launch_chain_tile<FORM, 6>(a, st, Tc); break;
    case 7: launch_chain_tile<FORM, 7>(a, st, Tc); break;
    default: launch_chain_tile<FORM, 8>(a, st, Tc); break;
  }
}

template <int LANES, int OC, int NC>
static void launch_split_tile(const ConvArgs& a, hipStream_t st, long ncols, int rows) {
  const dim3 grid((unsigned)((ncols + NC - 1) / NC), (unsigned)((rows + OC - 1) / OC));
  hipLaunchKernelGGL((codec_conv_split_kernel<LANES, OC, NC>), grid, dim3(LANES), 0, st, a);
}

// Split-sum tile (launch shape only): with at most 4 columns in the batch,
// one row of those columns per workgroup; else 32 outputs per workgroup, in
// columns when the batch has at least as many columns as rows, while that
// leaves CONV_SPLIT_WGS workgroups; else 8.
constexpr long CONV_SPLIT_WGS = 512;
template <int LANES>
static void launch_split(const ConvArgs& a, hipStream_t st, int Tc) {
  const long ncols = (long)a.B * Tc;
  const int rows = a.transposed ? a.C_out * a.stride : a.C_out;
  auto wgs = [&](int oc, int nc) { return ((rows + oc - 1) / oc) * ((ncols + nc - 1) / nc); };
  const bool wide = ncols >= rows;
  if (ncols == 1) launch_split_tile<LANES, 1, 1>(a, st, ncols, rows);
  else if (ncols == 2) launch_split_tile<LANES, 1, 2>(a, st, ncols, rows);
  else if (ncols <= 4) launch_split_tile<LANES, 1, 4>(a, st, ncols, rows);
  else if (wide && wgs(4, 8) >= CONV_SPLIT_WGS) launch_split_tile<LANES, 4, 8>(a, st, ncols, rows);
  else if (!wide && wgs(8, 4) >= CONV_SPLIT_WGS) launch_split_tile<LANES, 8, 4>(a, st, ncols, rows);
  else if (wide) launch_split_tile<LANES, 2, 4>(a, st, ncols, rows);
  else launch_split_tile<LANES, 4, 2>(a, st, ncols, rows);
}

// The kernel by the layer's shape (input channels, terms per output), the
// tile by the launch.
void launch_codec_conv(const ConvArgs& a, hipStream_t st) {
  const int Tc = a.strided ? a.T_in / a.stride : a.T_in;
  if (a.C_in <= CONV_CHAIN_C) {  // weights of 8 channels in LDS: at most 32 x 16 x 8 floats
    if (a.transposed) launch_chain_s<2>(a, st, Tc);
    else if (a.strided) launch_chain_s<1>(a, st, Tc);
    else launch_chain_s<0>(a, st, Tc);
    return;
  }
  const long kd = (long)a.C_in * (a.transposed ? 2 : a.K);
  if (kd > CONV_WIDE_KD) launch_split<256>(a, st, Tc);
  else launch_split<64>(a, st, Tc);
}

// ---------------------------------------------------------------------------
// Residual vector quantisation.  Stage q is one launch of (codeword tile,
// slot) workgroups: each first finishes stage q - 1 for its slot (the
// minimum over that stage's tile minima, lowest index among equals; the
// residual r_q = r_{q-1} - row), then takes RVQ_ROWS codewords of codebook q
// with 4 lanes per codeword: distance |c|^2 - 2 r.c (the |r|^2 common to
// every row left out), each lane summing a quarter of the features in order
// in fp32, the 4 quarters folded by a fixed butterfly; the tile's minimum
// (lowest index among equals) is written for the next stage.  Tile 0 writes
// the finished code and residual.  A last launch finishes stage n_q - 1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool rvq_better(float v2, int i2, float v, int i) {
  return v2 < v || (v2 == v && i2 < i);
}

// stage q - 1's code for slot b from its tile minima (every thread gets it)
__device__ int rvq_finish(const RvqArgs& a, int q, int b, int* red_i) {
  const int tiles = rvq_tiles(a.card), tid = threadIdx.x;
  const float* pv = a.part_v + ((long)((q - 1) & 1) * a.B + b) * tiles;
  const int* pi = a.part_i + ((long)((q - 1) & 1) * a.B + b) * tiles;
  if (tid < 64) {
    float bv = INFINITY;
    int bi = 0x7fffffff;
    for (int t = tid; t < tiles; t += 64)
      if (rvq_better(pv[t], pi[t], bv, bi)) {
        bv = pv[t];
        bi = pi[t];
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float v2 = __shfl_xor(bv, off);
      const int i2 = __shfl_xor(bi, off);
      if (rvq_better(v2, i2, bv, bi)) {
        bv = v2;
        bi = i2;
      }
    }
    if (tid == 0) red_i[0] = min(bi, a.card - 1);
  }
  __syncthreads();
  return red_i[0];
}

__global__ __launch_bounds__(256) void codec_rvq_stage_kernel(RvqArgs a, int q) {
  extern __shared__ float rr[];  // [d] this stage's residual
  __shared__ float red_v[4];
  __shared__ int red_i[4];
  const int tile = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this stage's residual: z, or the previous stage's residual minus its row
  const float* rin = q == 0 ? a.z + (long)b * a.d : a.res + ((long)((q - 1) & 1) * a.B + b) * a.d;
  int prev = -1;
  if (q > 0) prev = rvq_finish(a, q, b, red_i);
  const bf16_t* prow = q > 0 ? a.codebooks + ((long)(q - 1) * a.card + prev) * a.d : nullptr;
  for (int i = tid; i < a.d; i += 256) rr[i] = q > 0 ? rin[i] - bf2f(prow[i]) : rin[i];
  __syncthreads();
  if (tile == 0 && q > 0) {
    if (tid == 0) a.codes[b * a.n_q + q - 1] = prev;
    for (int i = tid; i < a.d; i += 256) a.res[((long)(q & 1) * a.B + b) * a.d + i] = rr[i];
  } else if (tile == 0) {
    for (int i = tid; i < a.d; i += 256) a.res[((long)(q & 1) * a.B + b) * a.d + i] = rr[i];
  }
  if (q == a.n_q) return;  // the finishing launch
  // 4 lanes per codeword: lane quarter k sums features k*d/4 .. (k+1)*d/4 - 1
  const int cw = tid >> 2, qk = tid & 3;
  const int j = tile * RVQ_ROWS + cw;
  const int n4 = a.d / 4;
  float dot = 0.f, cc = 0.f;
  if (j < a.card) {
    const bf16_t* row = a.codebooks + ((long)q * a.card + j) * a.d;
    for (int i = qk * n4; i < (qk + 1) * n4; i += 8) {
      float f[8];
      unpack8(ld16(row + i), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dot = __builtin_fmaf(f[e], rr[i + e], dot);
        cc = __builtin_fmaf(f[e], f[e], cc);
      }
    }
  }
  dot += __shfl_xor(dot, 1);
  cc += __shfl_xor(cc, 1);
  dot += __shfl_xor(dot, 2);
  cc += __shfl_xor(cc, 2);
  // rows past the codebook's end (the last tile's tail) never win; a NaN
  // distance counts as +inf, so the winner is always a real row
  float bv = j < a.card ? cc - 2.f * dot : INFINITY;
  if (bv != bv) bv = INFINITY;
  int bi = j < a.card ? j : 0x7fffffff;
#pragma unroll
  for (int off = 4; off <= 32; off <<= 1) {
    const float v2 = __shfl_xor(bv, off);
    const int i2 = __shfl_xor(bi, off);
    if (rvq_better(v2, i2, bv, bi)) {
      bv = v2;
      bi = i2;
    }
  }
  if (lane == 0) {
    red_v[wave] = bv;
    red_i[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float v = red_v[0];
    int ix = red_i[0];
    for (int w = 1; w < 4; ++w)
      if (rvq_better(red_v[w], red_i[w], v, ix)) {
        v = red_v[w];
        ix = red_i[w];
      }
    const long o = ((long)(q & 1) * a.B + b) * rvq_tiles(a.card) + tile;
    a.part_v[o] = v;
    a.part_i[o] = ix;
  }
}

void launch_codec_rvq(const RvqArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.d * 4;
  for (int q = 0; q < a.n_q; ++q)
    hipLaunchKernelGGL(codec_rvq_stage_kernel, dim3(rvq_tiles(a.card), a.B), dim3(256), lds, s, a, q);
  hipLaunchKernelGGL(codec_rvq_stage_kernel, dim3(1, a.B), dim3(256), lds, s, a, a.n_q);
}

// ---------------------------------------------------------------------------
// Streaming state: new history[j] = (old history, input)[T + j] for each
// convolution with memory, all of them in one launch (grid-stride).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void codec_hist_kernel(HistArgs a) {
  for (int e = 0; e < a.n; ++e) {
    const HistEntry& h = a.e[e];
    const long n = (long)a.B * h.C * h.H;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
      const int j = (int)(i % h.H);
      const long bc = i / h.H;  // b * C + c
      const int src = h.T + j;  // index into (old history, input)
      h.new_h[i] = src < h.H ? h.old_h[bc * h.H + src] : h.x[bc * h.T + (src - h.H)];
    }
  }
}

void launch_codec_hist(const HistArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(codec_hist_kernel, dim3(64), dim3(256), 0, s, a);
}

}  // namespace pp
