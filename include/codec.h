/*
 * codec.h -- C ABI of the streaming codec (decoder / code2wav, and encoder)
 * in libpp.so for MI355X (gfx950).
 *
 * One call of pp_codec_decode turns one 80 ms frame of 8 codebook indices per
 * session slot into 1920 audio samples at 24 kHz; one call of
 * pp_codec_encode turns 1920 samples of user audio per slot into 8 codebook
 * indices.  Each direction carries each slot's streaming state to its next
 * call.
 *
 *   chenxutan.com PersonaPlex article, section 2.3 on Mimi: a streaming neural
 *   codec of the SoundStream / EnCodec family, 24 kHz audio <-> 12.5 Hz
 *   discrete tokens at 1.1 kbps, fully causal, with transformers in the
 *   encoder and the decoder.  PersonaPlex recipe, "Architecture (Moshi
 *   RQ-Transformer, all native)": 8 active codebooks of 2048 entries, 1920
 *   samples per frame, streaming encode and decode; the agent's audio rows
 *   1-8 of each tick are what the decoder turns into speech.
 *
 * The pages give neither the decoder's layers nor its weights.  The decoder
 * here is this library's reading of that family, fixed by pp_codec_dims:
 *
 *   1. latent x = sum over the n_q codebooks of codebook_q[code_q], in
 *      codebook order (fp32);
 *   2. a causal transformer over frames at the slot's frame position with
 *      the temporal transformer's block (RMSNorm with fp32 alpha, fused QKV,
 *      interleaved RoPE, softmax attention over the `window` most recent
 *      frames whose keys and values are kept as bf16, SiLU-gated MLP), then
 *      an output RMSNorm: z;
 *   3. a causal convolution of kernel conv_k from d to channels[0];
 *   4. per stage i (stride s_i): ELU, causal transposed convolution of kernel
 *      2 s_i from channels[i] to channels[i+1] (upsampling by s_i), then a
 *      residual unit: ELU, causal convolution of kernel res_k to
 *      channels[i+1]/2, ELU, 1 x 1 convolution back to channels[i+1], added
 *      to the stage's upsampled signal;
 *   5. ELU and a causal convolution of kernel conv_k to one channel: the
 *      samples.  The strides multiply to the samples per frame.
 *
 * The encoder mirrors it: a causal convolution of kernel conv_k from one
 * channel to channels[n_stages]; per stage j = 0 .. n_stages-1 (decoder
 * stage i = n_stages-1-j in reverse) a residual unit on channels[i+1] as
 * above, then ELU and a causal strided convolution of kernel 2 s_i and
 * stride s_i to channels[i]; then ELU and a causal convolution of kernel
 * conv_k to d channels (one latent per frame); the transformer block with the
 * encoder's own weights and output norm; then residual vector quantisation
 * against the decoder's codebooks: code_q = the row of codebook q nearest to
 * the residual (squared Euclidean distance, the lowest index on ties),
 * residual -= that row, for q = 0 .. n_q-1.  Causal strided convolution:
 * output t = b + sum_i sum_k w[o][i][k] x[i][t s - s + k].
 *
 * Causal convolution: y[o][t] = b[o] + sum_i sum_k w[o][i][k] x[i][t-(K-1-k)]
 * with zeros before the stream's first frame.  Causal transposed convolution
 * (stride s, K = 2 s): input m adds w[o][i][k] x[i][m] to output m s + k;
 * each call emits the outputs of its own inputs' span, the overhang of its
 * last input being completed by the next call.
 *
 * Conventions are those of pp.h: bf16 as uint16_t bit patterns, caller-owned
 * device buffers and stream, validate-then-commit, PP_E* return codes,
 * PP_EDEVICE poisons the handle, no C++ exception crosses the interface.
 * Slots are isolated: a slot's samples and codes depend only on its own
 * stream, bit for bit the same for every batch size B and every other
 * slot's content.
 */
#ifndef PP_CODEC_H
#define PP_CODEC_H

#include <stddef.h>
#include <stdint.h>

#include "pp.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PP_CODEC_MAX_STAGES 6    /* upsampling stages */
#define PP_CODEC_MAX_BATCH  32   /* slots per handle */
#define PP_CODEC_MAX_WINDOW 256  /* transformer frames (one decode split) */

typedef struct pp_codec_dims {
  int32_t n_q;        /* codebooks per frame (1..16) */
  int32_t card;       /* entries per codebook */
  int32_t d;          /* latent and transformer width (a multiple of 32, at most 8192) */
  int32_t n_layers, n_heads, ffn;   /* transformer; head_dim = d / n_heads in {32, 64, 128}; ffn % 32 == 0 */
  int32_t window;     /* frames the attention sees, 1..PP_CODEC_MAX_WINDOW */
  int32_t conv_k;     /* kernel of the first and the last convolution (1..8) */
  int32_t res_k;      /* kernel of each residual unit's first convolution (1..8) */
  int32_t n_stages;   /* 1..PP_CODEC_MAX_STAGES */
  int32_t strides[PP_CODEC_MAX_STAGES];       /* each 1..8 */
  int32_t channels[PP_CODEC_MAX_STAGES + 1];  /* channels[0] after the first convolution, then after each
                                                 stage; channels[i] for i >= 1 even */
  float norm_eps;
  float rope_base;
} pp_codec_dims;

/* Device pointers, all required.  Transformer matrices are in the tile layout
 * of pp_pack_matrix (pp.h), stacked per layer with pp_packed_elems(M, K)
 * elements each; convolution weights are row-major bf16 [C_out][C_in][K] (the
 * transposed convolutions too); biases and RMSNorm alphas are fp32. */
typedef struct pp_codec_weights {
  const uint16_t* codebooks;  /* [n_q][card][d] row-major */
  const float* attn_norm;     /* [n_layers][d] */
  const uint16_t* wqkv;       /* [n_layers] x [3d][d], rows q; k; v, heads contiguous */
  const uint16_t* wo;         /* [n_layers] x [d][d] */
  const float* mlp_norm;      /* [n_layers][d] */
  const uint16_t* w_in;       /* [n_layers] x [2 ffn][d], rows gate; up */
  const uint16_t* w_out;      /* [n_layers] x [d][ffn] */
  const float* out_norm;      /* [d] */
  const uint16_t* conv_in_w;  /* [channels[0]][d][conv_k] */
  const float* conv_in_b;     /* [channels[0]] */
  const uint16_t* up_w[PP_CODEC_MAX_STAGES];     /* [channels[i+1]][channels[i]][2 strides[i]] */
  const float* up_b[PP_CODEC_MAX_STAGES];        /* [channels[i+1]] */
  const uint16_t* res_a_w[PP_CODEC_MAX_STAGES];  /* [channels[i+1]/2][channels[i+1]][res_k] */
  const float* res_a_b[PP_CODEC_MAX_STAGES];     /* [channels[i+1]/2] */
  const uint16_t* res_b_w[PP_CODEC_MAX_STAGES];  /* [channels[i+1]][channels[i+1]/2][1] */
  const float* res_b_b[PP_CODEC_MAX_STAGES];     /* [channels[i+1]] */
  const uint16_t* conv_out_w; /* [1][channels[n_stages]][conv_k] */
  const float* conv_out_b;    /* [1] */
  /* the encoder (stage j works at decoder stage i = n_stages-1-j's channels and stride) */
  const uint16_t* enc_conv_in_w;  /* [channels[n_stages]][1][conv_k] */
  const float* enc_conv_in_b;     /* [channels[n_stages]] */
  const uint16_t* enc_res_a_w[PP_CODEC_MAX_STAGES];  /* [channels[i+1]/2][channels[i+1]][res_k] */
  const float* enc_res_a_b[PP_CODEC_MAX_STAGES];     /* [channels[i+1]/2] */
  const uint16_t* enc_res_b_w[PP_CODEC_MAX_STAGES];  /* [channels[i+1]][channels[i+1]/2][1] */
  const float* enc_res_b_b[PP_CODEC_MAX_STAGES];     /* [channels[i+1]] */
  const uint16_t* enc_down_w[PP_CODEC_MAX_STAGES];   /* [channels[i]][channels[i+1]][2 strides[i]] */
  const float* enc_down_b[PP_CODEC_MAX_STAGES];      /* [channels[i]] */
  const uint16_t* enc_conv_out_w; /* [d][channels[0]][conv_k] */
  const float* enc_conv_out_b;    /* [d] */
  const float* enc_attn_norm;     /* as the decoder's transformer fields */
  const uint16_t* enc_wqkv;
  const uint16_t* enc_wo;
  const float* enc_mlp_norm;
  const uint16_t* enc_w_in;
  const uint16_t* enc_w_out;
  const float* enc_out_norm;
} pp_codec_weights;

typedef struct pp_codec pp_codec;

/* Samples per frame of `dims` (the product of the strides), or a negative
 * PP_E* code for invalid dims. */
int pp_codec_samples(const pp_codec_dims* dims);

/* Bytes of the device arena a handle of B slots needs (every slot's key and
 * value ring, streaming state and activations).  PP_EINVAL for invalid dims
 * or B outside 1..PP_CODEC_MAX_BATCH. */
int pp_codec_arena_bytes(const pp_codec_dims* dims, int B, size_t* out_bytes);

/* Creates a codec handle (decoder and encoder) for B slots in the caller's arena (256-byte aligned, at
 * least pp_codec_arena_bytes) on the caller's stream, every slot fresh
 * (position 0, zero history).  Captures its graphs.  PP_EINVAL for a NULL or
 * invalid argument, PP_ENOSPC for a small arena, PP_EDEVICE if a HIP call
 * fails; *out is NULL on error. */
int pp_codec_create(const pp_codec_dims* dims, int B, const pp_codec_weights* w, void* arena,
                    size_t arena_bytes, void* stream, pp_codec** out);

/* Decodes one frame for every slot: codes host int32 [B][n_q] (each in
 * [0, card), else PP_EINVAL and nothing runs), pcm host float [B][samples]
 * receives the samples.  Synchronous; advances every slot by one frame. */
int pp_codec_decode(pp_codec* h, const int32_t* codes, float* pcm);

/* Encodes one frame for every slot: pcm host float [B][samples] (finite,
 * else PP_EINVAL and nothing runs), codes host int32 [B][n_q] receives the
 * codebook indices.  Synchronous; advances every slot's encoder by one frame. */
int pp_codec_encode(pp_codec* h, const float* pcm, int32_t* codes);

/* Makes slot a fresh stream in both directions (positions 0, zero
 * histories); the other slots are untouched.  PP_EINVAL for a slot outside
 * [0, B). */
int pp_codec_reset(pp_codec* h, int slot);

/* Measurement hook: average device time of one decode call's graph over
 * `iters` back-to-back launches (HIP events on the handle's stream).  The
 * launches recompute the current frame without advancing any slot, so the
 * slots' state is unchanged. */
int pp_codec_time(pp_codec* h, int iters, float* avg_ms);

/* The same for one encode call's graph. */
int pp_codec_time_encode(pp_codec* h, int iters, float* avg_ms);

/* Device views of the decoder's state after the last call. */
typedef struct pp_codec_taps_t {
  const uint16_t* ring;  /* bf16 [B][n_layers][2][n_heads][window][head_dim]: the transformer's stored keys
                            (index 0) and values (index 1), position p at p mod window */
  const float* z;        /* [B][d]: the last call's transformer output after the output norm */
  const uint16_t* enc_ring;  /* the encoder's, laid out as ring */
  const float* enc_y;    /* [B][d]: the last encode call's latent (the transformer's input) */
  const float* enc_z;    /* [B][d]: the last encode call's transformer output after the output norm */
} pp_codec_taps_t;

/* Test hook: fills *out with device pointers into the arena (valid until
 * the handle is destroyed; the contents are those of the last call in each
 * direction).  Waits for the handle's device work. */
int pp_codec_taps(pp_codec* h, pp_codec_taps_t* out);

/* Waits for the handle's device work, then frees its host resources. */
void pp_codec_destroy(pp_codec* h);

/* Message of the handle's last error, or of the last failed pp_codec_create
 * when h is NULL. */
const char* pp_codec_last_error(const pp_codec* h);

#ifdef __cplusplus
}
#endif

#endif /* PP_CODEC_H */
