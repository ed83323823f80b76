// Streaming codec decoder (code2wav) kernels for gfx950: the residual-
// quantiser sum, the output norm, the causal and transposed convolutions of
// the upsampling stack, and the streaming-state update.
//
// chenxutan.com PersonaPlex article, section 2.3 on Mimi: a causal codec of
// the SoundStream / EnCodec family that turns 12.5 Hz frames of 8 codebooks
// back into 24 kHz audio; PersonaPlex recipe, "Architecture": 1920 samples
// per 80 ms frame.  The layer structure is this library's reading of that
// family (codec.h).  The work is small and latency-bound (at most a few
// hundred thousand outputs per call, each a sum of 16 to 3584 products), so
// the convolutions are direct sums on the vector ALU in fp32: a group of
// lanes per output splits the (input channel, tap) sum in a fixed order and
// folds it with a fixed butterfly, so each slot's result depends only on its
// own inputs.
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
// Convolutions.  Output (b, o, t) = bias[o] + sum over input channels i and
// taps of w * input (plus the skip), stored raw and/or after ELU; the inputs
// arrive already activated.  A group of LPO lanes owns TT consecutive
// outputs of one (slot, output channel): lane l takes input channels
// l, l + LPO, ... in order, keeps the K + TT - 1 inputs its taps reach in
// registers and the channel's K weights, then the LPO partial sums of each
// output are folded by a fixed butterfly.  The causal form reads time
// t - (K-1-k) at tap k; the transposed form gives each thread the `stride`
// outputs of one input position m (output m s + r reads input m at tap r and
// input m - 1 at tap r + s).  Times before this call's first input come from
// the history.
// ---------------------------------------------------------------------------
constexpr int CONV_KMAX = 8;

__device__ __forceinline__ float elu_f(float v) { return v > 0.f ? v : expm1f(v); }

template <int LPO, int TT>
__device__ __forceinline__ void conv_store(const ConvArgs& a, bool live, int l, int b, int o, int t0, int T_out,
                                           float (&acc)[TT], int n) {
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    if (u < n) {  // n is the same for the whole group (for the whole launch unless ragged)
#pragma unroll
      for (int off = LPO / 2; off >= 1; off >>= 1) acc[u] += __shfl_xor(acc[u], off, LPO);
    }
  }
  if (!live || l != 0) return;
  const long base = ((long)b * a.C_out + o) * T_out + t0;
  const float bo = a.bias[o];
#pragma unroll
  for (int u = 0; u < TT; ++u) {
    if (u < n) {
      float y = bo + acc[u];
      if (a.skip) y += a.skip[base + u];
      if (a.y) a.y[base + u] = y;
      if (a.ya) a.ya[base + u] = elu_f(y);
    }
  }
}

// causal convolution: TT consecutive outputs per group
template <int LPO, int TT>
__global__ __launch_bounds__(256) void codec_conv_kernel(ConvArgs a) {
  const int T = a.T_in, nt = (T + TT - 1) / TT;
  const long n_grp = (long)a.B * a.C_out * nt;
  const long gid = ((long)blockIdx.x * blockDim.x + threadIdx.x) / LPO;
  const int l = threadIdx.x % LPO;
  const bool live = gid < n_grp;
  const long g = live ? gid : 0;
  const int t0 = (int)(g % nt) * TT;
  const int o = (int)((g / nt) % a.C_out);
  const int b = (int)(g / ((long)nt * a.C_out));
  const int K = a.K;
  float acc[TT];
#pragma unroll
  for (int u = 0; u < TT; ++u) acc[u] = 0.f;
#pragma unroll 2
  for (int i = l; i < a.C_in; i += LPO) {
    const float* xi = a.x + ((long)b * a.C_in + i) * T;
    const float* hi = a.hist ? a.hist + ((long)b * a.C_in + i) * a.H : nullptr;
    const bf16_t* wi = a.w + ((long)o * a.C_in + i) * K;
    // inputs t0 - (K-1) .. t0 + TT - 1
    float xv[CONV_KMAX - 1 + TT];
    float wv[CONV_KMAX];
#pragma unroll
    for (int k = 0; k < CONV_KMAX; ++k) wv[k] = k < K ? bf2f(wi[k]) : 0.f;
#pragma unroll
    for (int j = 0; j < CONV_KMAX - 1 + TT; ++j) {
      const int tt = t0 - (K - 1) + j;
      xv[j] = j >= K - 1 + TT ? 0.f : tt >= T ? 0.f : tt >= 0 ? xi[tt] : hi[a.H + tt];
    }
#pragma unroll
    for (int k = 0; k < CONV_KMAX; ++k) {
      if (k < K) {
#pragma unroll
        for (int u = 0; u < TT; ++u) acc[u] = __builtin_fmaf(wv[k], xv[u + k], acc[u]);
      }
    }
  }
  conv_store<LPO, TT>(a, live, l, b, o, t0, T, acc, T - t0);
}

// transposed convolution: the `stride` outputs of one input position per group
template <int LPO>
__global__ __launch_bounds__(256) void codec_convt_kernel(ConvArgs a) {
  const int s = a.stride, T = a.T_in, T_out = T * s;
  const long n_grp = (long)a.B * a.C_out * T;
  const long gid = ((long)blockIdx.x * blockDim.x + threadIdx.x) / LPO;
  const int l = threadIdx.x % LPO;
  const bool live = gid < n_grp;
  const long g = live ? gid : 0;
  const int m = (int)(g % T);
  const int o = (int)((g / T) % a.C_out);
  const int b = (int)(g / ((long)T * a.C_out));
  float acc[CONV_KMAX];
#pragma unroll
  for (int r = 0; r < CONV_KMAX; ++r) acc[r] = 0.f;
#pragma unroll 2
  for (int i = l; i < a.C_in; i += LPO) {
    const float* xi = a.x + ((long)b * a.C_in + i) * T;
    const float x0 = xi[m];
    const float x1 = m > 0 ? xi[m - 1] : a.hist[((long)b * a.C_in + i) * a.H + a.H - 1];
    const bf16_t* wi = a.w + ((long)o * a.C_in + i) * a.K;
#pragma unroll
    for (int r = 0; r < CONV_KMAX; ++r) {
      if (r < s) acc[r] = __builtin_fmaf(bf2f(wi[r + s]), x1, __builtin_fmaf(bf2f(wi[r]), x0, acc[r]));
    }
  }
  conv_store<LPO, CONV_KMAX>(a, live, l, b, o, m * s, T_out, acc, s);
}

// Enough lanes for the part (256 CUs x 4 SIMDs x 2 waves of 64).
constexpr long CONV_LANES = 1L << 17;

// strided convolution: one output per group
template <int LPO>
__global__ __launch_bounds__(256) void codec_convs_kernel(ConvArgs a) {
  const int s = a.stride, T = a.T_in, T_out = T / s;
  const long n_grp = (long)a.B * a.C_out * T_out;
  const long gid = ((long)blockIdx.x * blockDim.x + threadIdx.x) / LPO;
  const int l = threadIdx.x % LPO;
  const bool live = gid < n_grp;
  const long g = live ? gid : 0;
  const int t = (int)(g % T_out);
  const int o = (int)((g / T_out) % a.C_out);
  const int b = (int)(g / ((long)T_out * a.C_out));
  float acc[1] = {0.f};
#pragma unroll 2
  for (int i = l; i < a.C_in; i += LPO) {
    const float* xi = a.x + ((long)b * a.C_in + i) * T;
    const float* hi = a.hist + ((long)b * a.C_in + i) * a.H;
    const bf16_t* wi = a.w + ((long)o * a.C_in + i) * a.K;
#pragma unroll
    for (int k = 0; k < 2 * CONV_KMAX; ++k) {
      if (k < a.K) {
        const int u = t * s - s + k;  // input time, >= -s
        const float v = u >= 0 ? xi[u] : hi[a.H + u];
        acc[0] = __builtin_fmaf(bf2f(wi[k]), v, acc[0]);
      }
    }
  }
  conv_store<LPO, 1>(a, live, l, b, o, t, T_out, acc, 1);
}

template <int LPO>
static void launch_conv_lpo(const ConvArgs& a, hipStream_t s, int tt) {
  const long groups = (long)a.B * a.C_out *
                      (a.transposed ? a.T_in : a.strided ? a.T_in / a.stride : (a.T_in + tt - 1) / tt);
  const dim3 grid((unsigned)((groups * LPO + 255) / 256));
  if (a.transposed) {
    hipLaunchKernelGGL(codec_convt_kernel<LPO>, grid, dim3(256), 0, s, a);
    return;
  }
  if (a.strided) {
    hipLaunchKernelGGL(codec_convs_kernel<LPO>, grid, dim3(256), 0, s, a);
    return;
  }
  switch (tt) {
    case 8: hipLaunchKernelGGL((codec_conv_kernel<LPO, 8>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((codec_conv_kernel<LPO, 4>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((codec_conv_kernel<LPO, 2>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((codec_conv_kernel<LPO, 1>), grid, dim3(256), 0, s, a); break;
  }
}

// Launch shape: the fewest lanes per output group (1, 8 or 64, at most the
// input channels) that still gives CONV_LANES lanes, else the most; then, for
// the causal form, the most outputs per group (8, 4, 2 or 1, at most the
// samples of the call) that keeps CONV_LANES lanes.  Fewer lanes per group
// fold fewer partial sums; more outputs per group re-read fewer inputs.
void launch_codec_conv(const ConvArgs& a, hipStream_t s) {
  // groups of one output (or one input position)
  const long outs = (long)a.B * a.C_out * (a.strided ? a.T_in / a.stride : a.T_in);
  int lpo = 1;
  for (int c : {1, 8, 64}) {
    if (c > 1 && a.C_in < c) break;
    lpo = c;
    if (outs * c >= CONV_LANES) break;
  }
  int tt = 1;
  if (!a.transposed && !a.strided)
    for (int c : {8, 4, 2}) {
      if (c <= a.T_in && (long)a.B * a.C_out * ((a.T_in + c - 1) / c) * lpo >= CONV_LANES) {
        tt = c;
        break;
      }
    }
  if (lpo == 64) launch_conv_lpo<64>(a, s, tt);
  else if (lpo == 8) launch_conv_lpo<8>(a, s, tt);
  else launch_conv_lpo<1>(a, s, tt);
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
