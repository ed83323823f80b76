// Kernels of the streaming codec (codec.hip) and their arguments.  The
// transformer layers of both directions run on the tick's GEMM and
// ring-decode launchers (kernels.h); these are the rest: the codebook sum
// (or the encoder's latent) into the first layer, the output norm, the causal
// (transposed, strided) convolutions, the residual quantiser and the
// streaming-state update.  Layouts: activations fp32 [B][C][T] (T = samples
// of this call at the layer's rate), convolution weights bf16
// [C_out][C_in][K], histories fp32 [B][C][H] (the H inputs before this call,
// as the layer is fed them: after their ELU).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pp {

constexpr int CODEC_MAX_HIST = 24;   // history entries (convolutions with memory)

struct CodecEmbedArgs {
  const float* y;         // [B][d] the transformer's input itself (the encoder), or null: the codebook sum
  const int* codes;       // [B][n_q]
  const int* ti;          // tick-input layout: the slot's frame position at TI_POS
  int B, d, n_q, card;
  const bf16_t* codebooks;  // [n_q][card][d]
  const float* alpha;       // first attention-norm alpha
  float* x;                 // [B][d] residual stream
  bf16_t* xa; long xa_lo;   // [B][d] x * alpha as a bf16 hi/lo pair
  float* part;              // [B][d/16] sums of squares per 16 features
  const double* inv_freq; int head_dim; float* rope;  // RoPE table [B][head_dim] (cos, sin) at the position
};
void launch_codec_embed(const CodecEmbedArgs& a, hipStream_t s);

struct CodecNormArgs {
  const float* x;        // [B][d]
  const float* part;     // [B][d/16] sums of squares of x per 16 features
  const float* alpha;    // [d]
  float eps;
  int B, d;
  float* z;              // [B][d]
};
void launch_codec_norm(const CodecNormArgs& a, hipStream_t s);

// One convolution.  transposed = strided = 0: causal convolution of kernel
// K <= 8 (stride 1); transposed = 1: causal transposed convolution with
// stride `stride` <= 8 and K = 2 stride, T_out = T_in * stride; strided = 1:
// causal strided convolution with stride `stride` <= 8 and K = 2 stride,
// T_out = T_in / stride, output t reading inputs t s - s + k.  Input x
// [B][C_in][T_in] with its history hist [B][C_in][H] (H = K - 1 for the
// causal form, 1 for the transposed form, `stride` for the strided form);
// both already hold the layer's input as it is fed (after its ELU).  Output
// [B][C_out][T_out]: bias + sum, plus skip [B][C_out][T_out] when given,
// stored raw into y and/or after ELU into ya (either may be null).
struct ConvArgs {
  const float* x; int C_in, T_in;
  const float* hist; int H;
  const bf16_t* w; const float* bias; int C_out, K, stride, transposed, strided;
  const float* skip;
  float* y;
  float* ya;
  int B;
};
void launch_codec_conv(const ConvArgs& a, hipStream_t s);

// Residual vector quantisation: per slot, for q = 0..n_q-1, the row of
// codebook q nearest to the residual (squared distance, lowest index on
// ties), then residual -= that row.  z [B][d] fp32 in, codes [B][n_q] out.
struct RvqArgs {
  const float* z; int B, d, n_q, card;
  const bf16_t* codebooks;  // [n_q][card][d]
  int* codes;
  // work buffers: per-tile minima [2][B][card / RVQ_ROWS] (value, index),
  // alternating by stage, and the residual [2][B][d]
  float* part_v; int* part_i;
  float* res;
};
constexpr int RVQ_ROWS = 64;  // codewords per workgroup and stage
inline __host__ __device__ int rvq_tiles(int card) { return (card + RVQ_ROWS - 1) / RVQ_ROWS; }
void launch_codec_rvq(const RvqArgs& a, hipStream_t s);

// The streaming-state update after a call: for each convolution with memory,
// the new history is the last H entries of (old history, this call's input).
struct HistEntry {
  const float* x; int C, T;     // this call's input [B][C][T]
  const float* old_h; float* new_h; int H;  // [B][C][H] each
};
struct HistArgs {
  HistEntry e[CODEC_MAX_HIST];
  int n, B;
};
void launch_codec_hist(const HistArgs& a, hipStream_t s);

}  // namespace pp
