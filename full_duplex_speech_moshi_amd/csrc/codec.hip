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
// Latent: x = sum of the n_q codebooks' rows in codebook order (fp32), with
// x * alpha as a bf16 pair and the per-16 sums of squares for the first
// layer's QKV launch, and the frame's RoPE table.  One thread per 8 features.
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
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int q = 0; q < a.n_q; ++q) {
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
// Convolutions.  Output (b, o, t) = bias[o] + sum over j of w * act(input),
// j running over (input channel i, tap): K taps for the causal form (tap k
// reads time t - (K-1-k)), 2 for the transposed form (m = t / s, r = t % s:
// tap r reads input m, tap r + s reads input m - 1).  Times before this
// call's first input come from the history.  LPO lanes share one output:
// lane l adds j = l, l + LPO, ... in order, then the LPO partial sums are
// folded by a fixed butterfly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float elu_f(float v) { return v > 0.f ? v : expm1f(v); }

template <int LPO>
__global__ __launch_bounds__(256) void codec_conv_kernel(ConvArgs a) {
  const int T_out = a.T_in * a.stride;
  const long n_out = (long)a.B * a.C_out * T_out;
  const long gid = ((long)blockIdx.x * blockDim.x + threadIdx.x) / LPO;
  const int l = threadIdx.x % LPO;
  const bool live = gid < n_out;
  const long g = live ? gid : 0;
  const int t = (int)(g % T_out);
  const int o = (int)((g / T_out) % a.C_out);
  const int b = (int)(g / ((long)T_out * a.C_out));
  const float* xb = a.x + (long)b * a.C_in * a.T_in;
  const float* hb = a.hist + (long)b * a.C_in * a.H;
  const bf16_t* wo = a.w + (long)o * a.C_in * a.K;
  float acc = 0.f;
  if (!a.transposed) {
    const int R = a.C_in * a.K;
    for (int j = l; j < R; j += LPO) {
      const int i = j / a.K, k = j - i * a.K;
      const int u = t - (a.K - 1 - k);  // input time
      float v = u >= 0 ? xb[(long)i * a.T_in + u] : hb[(long)i * a.H + a.H + u];
      if (a.act) v = elu_f(v);
      acc = __builtin_fmaf(bf2f(wo[j]), v, acc);
    }
  } else {
    const int s = a.stride, m = t / s, r = t - m * s;
    const int R = a.C_in * 2;
    for (int j = l; j < R; j += LPO) {
      const int i = j >> 1, e = j & 1;
      const int u = m - e;
      float v = u >= 0 ? xb[(long)i * a.T_in + u] : hb[(long)i * a.H + a.H - 1];
      if (a.act) v = elu_f(v);
      acc = __builtin_fmaf(bf2f(wo[(long)i * a.K + r + e * s]), v, acc);
    }
  }
#pragma unroll
  for (int off = LPO / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPO);
  if (live && l == 0) {
    float y = a.bias[o] + acc;
    const long oi = ((long)b * a.C_out + o) * T_out + t;
    if (a.skip) y += a.skip[oi];
    a.y[oi] = y;
  }
}

void launch_codec_conv(const ConvArgs& a, hipStream_t s) {
  const long n_out = (long)a.B * a.C_out * a.T_in * a.stride;
  const int R = a.C_in * (a.transposed ? 2 : a.K);
  auto blocks = [&](int lpo) { return dim3((unsigned)((n_out * lpo + 255) / 256)); };
  if (R >= 1024) hipLaunchKernelGGL(codec_conv_kernel<64>, blocks(64), dim3(256), 0, s, a);
  else if (R >= 128) hipLaunchKernelGGL(codec_conv_kernel<8>, blocks(8), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(codec_conv_kernel<1>, blocks(1), dim3(256), 0, s, a);
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
