// HIP kernels of the lockstep tick, written for gfx950 (CDNA4, 64-lane waves).
//
// Every kernel is batch-invariant: the arithmetic that produces slot b's
// values (instruction sequence, summation order, split points) depends only
// on slot b's own inputs and position, never on B or on other slots, so a
// session computes the same bits alone or in a full batch ("greedy isolation
// is bit-exact", PersonaPlex recipe, Summary / Notes).
#include "kernels.h"
#include "device.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace pp {

// ---------------------------------------------------------------------------
// Skinny GEMM family  Y[b][m] = sum_k W[m][k] * X[b][k],  b < B <= 32.
//
// Arithmetic contract (the same for every B, so a slot's bits never depend on
// the batch): the K/32 k-steps are cut into 8 ranges R_w = [floor(ks*w/8),
// floor(ks*(w+1)/8)); partial p_w accumulates, in increasing k-step order,
// one MFMA on the hi plane then one on the lo plane of the input; the result
// is ((p_0 + p_1) + ...) + p_7 in fp32.
//
// One workgroup = 8 waves owns a 16-row tile (two tiles, gate and up, for the
// gated MLP) over the whole K; the waves split K into 8 contiguous ranges and
// their partial tiles are summed in LDS in wave order.  Each wave streams its
// weight rows with 16-byte loads (4 lanes cover 64 contiguous bytes of a row)
// straight into v_mfma_f32_16x16x32_bf16 as the A operand; the slots are the
// 16 columns of the B operand, zero beyond B.  Activations arrive as a bf16
// hi/lo pair and each k-step issues one MFMA per plane into the same fp32
// accumulator, so the products are exact and the input carries 16 bits.  The MFMA computes every output
// column from that column alone, so a slot's result does not depend on what
// occupies the other columns.  Weight streaming is the bound (HBM); the
// matrix cores are idle most of the time even at B = 32.
//
// Normalised inputs: the producer of x stores bf16(x * alpha) and per-16-row
// sums of squares; the consumer scales its output column b by
// 1/sqrt(mean(x_b^2) + eps) in the epilogue (RMSNorm commutes with the
// projection), so no separate normalisation pass is needed.
// ---------------------------------------------------------------------------

template <int RT, int NT>
struct EpiSmem {
  float fin[RT][ROWS][NT * 16];   // the finished tile(s), [row][slot]
  float inv_rms[NT * 16];
};

template <int RT, int NT>
struct GemmSmem {
  float red[GEMM_WAVES][RT * NT][256];
  EpiSmem<RT, NT> e;
};

// Inverse RMS of each slot's input from the per-16-feature sums of squares.
// The loads are issued early (rms_preload, before the weight stream) and the
// sums formed later (rms_finish); lane sums run over i = lane, lane+64, ...
// and then a fixed butterfly, whichever way the loads were issued.
constexpr int RMS_PRE = 4;  // partials per lane held in registers
template <int NT>
struct RmsPre {
  float v[(NT * 16 + GEMM_WAVES - 1) / GEMM_WAVES][RMS_PRE];
};

template <int NT>
__device__ __forceinline__ void rms_preload(const GemmArgs& a, RmsPre<NT>& rp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // every lane loads (from a clamped, valid address) and then selects: no
  // branch per load, so the loads stay in flight together
#pragma unroll
  for (int k = 0; k < (NT * 16 + GEMM_WAVES - 1) / GEMM_WAVES; ++k) {
    const int c = wave + k * GEMM_WAVES;
#pragma unroll
    for (int q = 0; q < RMS_PRE; ++q) {
      const int i = lane + 64 * q;
      const bool ok = c < a.B && i < a.n_part;
      const float v = a.part_in[ok ? (long)c * a.n_part + i : 0];
      rp.v[k][q] = ok ? v : 0.f;
    }
  }
}

template <int NT>
__device__ __forceinline__ void rms_finish(const GemmArgs& a, const RmsPre<NT>& rp, float* inv_rms) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < (NT * 16 + GEMM_WAVES - 1) / GEMM_WAVES; ++k) {
    const int c = wave + k * GEMM_WAVES;
    if (c >= a.B) continue;  // wave-uniform: no slot here
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < RMS_PRE; ++q)
      if (lane + 64 * q < a.n_part) s += rp.v[k][q];
    for (int i = lane + 64 * RMS_PRE; i < a.n_part; i += 64) s += a.part_in[(long)c * a.n_part + i];
    s = wave_sum_rows(s);
    if (lane == 0 && c < NT * 16) inv_rms[c] = 1.0f / sqrtf(s / (float)a.feat + a.eps);
  }
}

// Per-thread epilogue inputs loaded before the weight stream: for EPI_RESID
// the old residual value and the next norm's alpha of item (row tid%16, slot
// tid/16).
struct EpiPre {
  float x0, x1;  // EPI_RESID: old residual value, next norm's alpha
  float cs, sn;  // EPI_QKV: rotation of the item's frequency at the slot's position
  int pos;       // EPI_QKV: the slot's position
};

template <int EPI, int NT>
__device__ __forceinline__ EpiPre epi_preload(const GemmArgs& a, const int tile) {
  EpiPre p{0.f, 0.f, 1.f, 0.f, 0};
  const int tid = threadIdx.x, row0 = tile * ROWS;
  if constexpr (EPI == EPI_QKV) {
    // item idx == tid of the epilogue: pair pr of rows, slot c
    const int pr = tid & 7, c = tid >> 3;
    const int cc = (c < a.B && c < NT * 16) ? c : 0;  // a valid slot for the loads
    p.pos = a.ti ? a.ti[cc * TI_STRIDE + TI_POS] : a.pos_const;
    const int d = a.n_heads * a.head_dim;
    const int r = row0 + 2 * pr;
    const int rr = r % d, dd = rr % a.head_dim;  // even: the pair's first feature
    if (a.rope && r < 2 * d) {
      p.cs = a.rope[(long)cc * a.head_dim + dd];
      p.sn = a.rope[(long)cc * a.head_dim + dd + 1];
    }
  }
  if constexpr (EPI == EPI_RESID) {
    const int r = tid & 15, c = tid >> 4;
    const bool ok = c < a.B && c < NT * 16;
    const float x0 = a.x[(long)(ok ? c : 0) * a.ldres + row0 + r];  // valid address either way
    const float x1 = a.alpha_next[row0 + r];
    p.x0 = ok ? x0 : 0.f;
    p.x1 = ok ? x1 : 0.f;
  }
  return p;
}


// Epilogue of one finished tile (rows 16*tile..): e.fin holds W x for the
// tile's rows and every slot, e.inv_rms the slots' inverse RMS where needed.
template <int EPI, int NT>
__device__ void gemm_epilogue(const GemmArgs& a, const int tile, EpiSmem<(EPI == EPI_GATED) ? 2 : 1, NT>& e,
                              const EpiPre& pre) {
  const int tid = threadIdx.x;
  const int row0 = tile * ROWS;
  if constexpr (EPI == EPI_QKV) {
    const int d = a.n_heads * a.head_dim;
    for (int idx = tid; idx < 8 * NT * 16; idx += 512) {
      const int pr = idx & 7, c = idx >> 3;
      if (c >= a.B) continue;
      const int r = row0 + 2 * pr;
      if (r >= a.M) continue;
      const int which = r / d;  // 0 q, 1 k, 2 v
      const int rr = r - which * d;
      const int h = rr / a.head_dim, dd = rr - h * a.head_dim;
      // workgroup: item idx == tid, pre holds its position and rotation
      const int pos = pre.pos;
      const bool rot = which < 2 && a.inv_freq;
      float cs = pre.cs, sn = pre.sn;
      if (rot && !a.rope) {
        const double th = (double)pos * a.inv_freq[dd >> 1];
        cs = (float)cos(th);
        sn = (float)sin(th);
      }
      float y0, y1;
      qkv_pair(e.fin[0][2 * pr][c], e.fin[0][2 * pr + 1][c], e.inv_rms[c], rot, cs, sn, y0, y1);
      if (which == 0) {
        a.q_out[(long)c * a.ldq + rr] = y0;
        a.q_out[(long)c * a.ldq + rr + 1] = y1;
      } else {
        bf16_t* dst = a.kv + (long)c * a.kv_slot_stride + (which == 2 ? a.kv_v_off : 0) +
                      ((long)h * a.window + (pos % a.window)) * a.head_dim + dd;
        dst[0] = f2bf(y0);
        dst[1] = f2bf(y1);
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    for (int idx = tid; idx < ROWS * NT * 16; idx += 512) {
      const int r = idx & 15, c = idx >> 4;
      if (c >= a.B) continue;
      const int m = row0 + r;
      const long o = (long)c * a.ldres + m;
      const float xn = pre.x0 + e.fin[0][r][c];  // item idx == tid: pre holds x[o], alpha_next[m]
      a.x[o] = xn;
      store_split(a.xa_out + o, a.xa_lo, xn * pre.x1);
      if (a.tap) a.tap[o] = xn;
      e.fin[0][r][c] = xn;
    }
    __syncthreads();
    if (tid < a.B) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < ROWS; ++r) s += e.fin[0][r][tid] * e.fin[0][r][tid];
      a.part_out[(long)tid * (a.M / ROWS) + tile] = s;
    }
  } else if constexpr (EPI == EPI_GATED) {
    for (int idx = tid; idx < ROWS * NT * 16; idx += 512) {
      const int r = idx & 15, c = idx >> 4;
      if (c >= a.B) continue;
      const int m = row0 + r;
      if (m >= a.M) continue;
      const float gt = e.fin[0][r][c] * e.inv_rms[c];
      const float up = e.fin[1][r][c] * e.inv_rms[c];
      store_split(a.m_out + (long)c * a.ldm + m, a.m_lo, gt / (1.0f + expf(-gt)) * up);
    }
  } else if constexpr (EPI == EPI_STORE) {
    for (int idx = tid; idx < ROWS * NT * 16; idx += 512) {
      const int r = idx & 15, c = idx >> 4;
      if (c >= a.B) continue;
      const int m = row0 + r;
      if (m >= a.M) continue;
      a.f_out[(long)c * a.ldf + m] = e.fin[0][r][c] * e.inv_rms[c];
    }
  } else {  // EPI_LOGITS
    for (int idx = tid; idx < ROWS * NT * 16; idx += 512) {
      const int r = idx & 15, c = idx >> 4;
      if (c >= a.B) continue;
      const int m = row0 + r;
      if (m >= a.M) continue;
      const float v = e.fin[0][r][c] * e.inv_rms[c];
      a.f_out[(long)c * a.ldf + m] = v;
      e.fin[0][r][c] = v;
    }
    __syncthreads();
    if (tid < a.B) {
      // strict '>' in row order: the lowest index wins a tie
      float best = e.fin[0][0][tid];
      int bi = row0;
      for (int r = 1; r < ROWS && row0 + r < a.M; ++r) {
        const float v = e.fin[0][r][tid];
        if (v > best) { best = v; bi = row0 + r; }
      }
      a.amax_v[(long)tid * a.ld_amax + tile] = best;
      a.amax_i[(long)tid * a.ld_amax + tile] = bi;
    }
  }
}


template <int DH>
__global__ __launch_bounds__(256) void dep_attn_kernel(DepAttnArgs d) {
  constexpr int PPW = 128 / DH;
  const DepAttnOut r = dep_attend<DH>(d, (blockIdx.x * 4 + (threadIdx.x >> 6)) * PPW);
  if (!r.ok) return;
  const int b = r.pair / d.n_heads, h = r.pair - b * d.n_heads;
  bf16_t* o = d.o + (long)b * d.ldo + h * DH + r.feat;
  store_split(o, d.o_lo, r.o0);
  store_split(o + 1, d.o_lo, r.o1);
}

void launch_dep_attention(const DepAttnArgs& d, hipStream_t s) {
  const int waves = (d.B * d.n_heads * d.head_dim + 127) / 128;  // 128/head_dim pairs per wave
  const dim3 grid((waves + 3) / 4);
  switch (d.head_dim) {
    case 32: hipLaunchKernelGGL(dep_attn_kernel<32>, grid, dim3(256), 0, s, d); break;
    case 64: hipLaunchKernelGGL(dep_attn_kernel<64>, grid, dim3(256), 0, s, d); break;
    default: hipLaunchKernelGGL(dep_attn_kernel<128>, grid, dim3(256), 0, s, d); break;
  }
}


// The greedy finisher of the previous depformer step (or of the text head),
// computed by every workgroup of the next step's first QKV projection for
// its B <= DEP_FUSE_B slots: the same choice as finish_unit (the argmax
// winner does not depend on the reduction order), the same y = u + table
// row, and the same x * alpha (hi/lo, into `olds`) and per-16-feature sums
// of squares (into `fparts`).  Workgroup 0 also writes the tokens and y.
__device__ void fin_into_lds(const FinishArgs& f, const int B, bf16_t* olds, float* fparts) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
  constexpr long OPL = (long)DEP_FUSE_B * DEP_FUSE_D;
  constexpr int PB = 8;  // partials per thread requested in one batch
  __shared__ float fsv[GEMM_WAVES];
  __shared__ int fsi[GEMM_WAVES];
  __shared__ int tok_s[DEP_FUSE_B];
  const int nk = f.step + 1, ng = f.dd / 16;
  // requests that do not depend on the choice go out first: this thread's
  // item (slot, 16-feature group) of u and alpha, and every slot's partials
  const bool item = tid < B * ng;
  const int ib = item ? tid / ng : 0, ig = item ? tid - ib * ng : 0;
  float uu[16], al[16];
  {
    const float* u = f.u + ((long)ib * f.dep_q + nk) * f.dd + ig * 16;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uu[i] = item ? u[i] : 0.f;
      al[i] = item ? f.alpha[ig * 16 + i] : 0.f;
    }
  }
  const int per = (f.n_part + nt - 1) / nt, t0 = tid * per, t1 = min(f.n_part, t0 + per);
  float vv[DEP_FUSE_B][PB];
  int ii[DEP_FUSE_B][PB];
#pragma unroll
  for (int b = 0; b < DEP_FUSE_B; ++b)
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const bool ok = b < B && t0 + j < t1;
      vv[b][j] = ok ? f.amax_v[(long)b * f.ld_amax + t0 + j] : 0.f;
      ii[b][j] = ok ? f.amax_i[(long)b * f.ld_amax + t0 + j] : 0x7fffffff;
    }
  for (int b = 0; b < B; ++b) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (amax_better(vv[b][j], ii[b][j], bv, bi)) { bv = vv[b][j]; bi = ii[b][j]; }
    for (int t = t0 + PB; t < t1; ++t) {  // more than PB partials per thread (n_part > PB * nt)
      const float v = f.amax_v[(long)b * f.ld_amax + t];
      const int i = f.amax_i[(long)b * f.ld_amax + t];
      if (amax_better(v, i, bv, bi)) { bv = v; bi = i; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float v2 = __shfl_xor(bv, off);
      const int i2 = __shfl_xor(bi, off);
      if (amax_better(v2, i2, bv, bi)) { bv = v2; bi = i2; }
    }
    if (lane == 0) {
      fsv[wave] = bv;
      fsi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < nt / 64; ++w)
        if (amax_better(fsv[w], fsi[w], bv, bi)) { bv = fsv[w]; bi = fsi[w]; }
      const int forced = f.step < 8 ? f.ti[b * TI_STRIDE + TI_FORCE + 1 + f.step] : -1;
      const int chosen = forced >= 0 ? forced : bi;
      if (blockIdx.x == 0) {
        int* to = f.to + b * TO_STRIDE;
        if (f.step < 8) {
          to[TO_PRED + 1 + f.step] = bi;
          to[TO_CHOSEN + 1 + f.step] = chosen;
        } else {
          to[TO_USER + f.step - 8] = bi;
        }
      }
      tok_s[b] = chosen;
    }
    __syncthreads();
  }
  if (item) {
    const bf16_t* e = f.table + (long)tok_s[ib] * f.dd + ig * 16;
    float fe[16];
    unpack8(ld16(e), fe);
    unpack8(ld16(e + 8), fe + 8);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = ig * 16 + i;
      const float v = uu[i] + fe[i];
      if (blockIdx.x == 0) f.y[(long)ib * f.dd + m] = v;
      store_split(olds + (long)ib * DEP_FUSE_D + m, OPL, v * al[i]);
      ss += v * v;
    }
    fparts[ib * (DEP_FUSE_D / 16) + ig] = ss;
  }
  __syncthreads();
}

// One 16-row tile (gate+up pair for EPI_GATED) of the GEMM, computed by a
// 512-thread workgroup; `smem` holds a GemmSmem<RT, NT>.  XS: where the
// input X comes from: 0 global memory; 1 the depformer attention, computed
// here (ATT); 2 the previous step's finisher, computed here (FIN).
template <int EPI, int NT, bool NTL, int XS = 0, int UB = 0>
__device__ void gemm_unit(const GemmArgs& a, const int tile, char* smem, bf16_t* olds = nullptr,
                          float* fparts = nullptr) {
  constexpr int RT = (EPI == EPI_GATED) ? 2 : 1;
  // k-steps per load batch (UB: a larger batch, so that a wave's whole
  // k-range is requested at once)
  constexpr int U = UB > 0 ? UB : (RT * NT > 1) ? 4 : 8;
  GemmSmem<RT, NT>& sm = *reinterpret_cast<GemmSmem<RT, NT>*>(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int ksteps = a.K >> 5;
  const int s0 = (ksteps * wave) / GEMM_WAVES;
  const int s1 = (ksteps * (wave + 1)) / GEMM_WAVES;

  // Weights in the tile layout: block (row tile T, k-step s) is 1 KB at
  // (T * ksteps + s) * 512 elements, lane l's 8 elements at l * 8.  Rows past
  // M are zero in that layout, so the loads need no row mask.
  const bf16_t* arow[RT];
  arow[0] = a.W + (long)tile * ksteps * 512 + lane * 8;
  if (RT == 2) arow[RT - 1] = a.W + ((long)tile + a.gate_off / ROWS) * ksteps * 512 + lane * 8;
  const bf16_t* xrow[NT];
  bool b_ok[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int c = ct * 16 + r16;
    b_ok[ct] = c < a.B;
    xrow[ct] = a.X + (long)(b_ok[ct] ? c : 0) * a.ldx + g * 8;
  }
  // With more than a few slots the activation rows are loaded in row order
  // (lane 4c + p takes 16-byte piece p of slot c's 64 bytes, so each group
  // of 4 lanes reads one contiguous piece instead of 4 rows 2 KB apart) and
  // moved into the MFMA operand order (lane 16p + c) by a lane permute
  // before use; the operand values are the same either way.
  const bool xperm = XS == 0 && a.B > 4;
  const int xsrc = ((lane & 15) * 4 + (lane >> 4)) * 4;  // permute source (bytes) of this lane
  if (xperm) {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      const int c = ct * 16 + (lane >> 2);
      b_ok[ct] = c < a.B;
      xrow[ct] = a.X + (long)(b_ok[ct] ? c : 0) * a.ldx + (lane & 3) * 8;
    }
  }
  auto xop = [&](const u32x4& v) -> bf16x8 {
    if (!xperm) return __builtin_bit_cast(bf16x8, v);
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc, (int)v[i]);
    return __builtin_bit_cast(bf16x8, r);
  };

  f32x4 acc[RT][NT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[rt][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // epilogue inputs requested now, consumed after the weight stream
  const EpiPre pre = epi_preload<EPI, NT>(a, tile);
  RmsPre<NT> rp;
  if (EPI != EPI_RESID && XS != 2) rms_preload<NT>(a, rp);

  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  // XS 1 / 2: the input is the depformer attention output / the previous
  // step's finisher output, computed here into LDS ([plane][slot][DEP_FUSE_D])
  // while the first weight batch is in flight.
  u32x4 pf[RT][U];
  constexpr long OPL = (long)DEP_FUSE_B * DEP_FUSE_D;  // LDS plane stride
  if constexpr (XS != 0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) pf[rt][u] = (s0 + u < s1) ? ldw16<NTL>(arow[rt] + (long)(s0 + u) * 512) : zero;
  }
  if constexpr (XS == 2) {
    fin_into_lds(a.fin, a.B, olds, fparts);
    // the slots' norm partials, in the lanes rms_preload would have used
    const int lane_ = tid & 63;
#pragma unroll
    for (int k = 0; k < (NT * 16 + GEMM_WAVES - 1) / GEMM_WAVES; ++k) {
      const int c = wave + k * GEMM_WAVES;
#pragma unroll
      for (int q = 0; q < RMS_PRE; ++q) {
        const int i = lane_ + 64 * q;
        rp.v[k][q] = (c < a.B && i < a.n_part) ? fparts[c * (DEP_FUSE_D / 16) + i] : 0.f;
      }
    }
  }
  if constexpr (XS == 1) {
    const int ppw = 128 / a.att.head_dim;
    for (int pp = wave * ppw; pp < a.B * a.att.n_heads; pp += GEMM_WAVES * ppw) {
      const DepAttnOut r = a.att.head_dim == 32   ? dep_attend<32>(a.att, pp)
                           : a.att.head_dim == 64 ? dep_attend<64>(a.att, pp)
                                                  : dep_attend<128>(a.att, pp);
      if (r.ok) {
        const int b = r.pair / a.att.n_heads, h = r.pair - b * a.att.n_heads;
        bf16_t* o = olds + (long)b * DEP_FUSE_D + h * a.att.head_dim + r.feat;
        store_split(o, OPL, r.o0);
        store_split(o + 1, OPL, r.o1);
      }
    }
    __syncthreads();
  }
  for (int s = s0; s < s1; s += U) {
    u32x4 av[RT][U], bh[NT][U], bl[NT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = (s + u) < s1;
      const int k = (s + u) * 32;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        av[rt][u] = (XS != 0 && s == s0) ? pf[rt][u] : ok ? ldw16<NTL>(arow[rt] + (long)(s + u) * 512) : zero;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        if constexpr (XS != 0) {
          const bf16_t* xo = olds + (long)(ct * 16 + r16) * DEP_FUSE_D + g * 8 + k;
          bh[ct][u] = (ok && b_ok[ct]) ? *reinterpret_cast<const u32x4*>(xo) : zero;
          bl[ct][u] = (ok && b_ok[ct]) ? *reinterpret_cast<const u32x4*>(xo + OPL) : zero;
        } else {
          bh[ct][u] = (ok && b_ok[ct]) ? ld16(xrow[ct] + k) : zero;
          bl[ct][u] = (ok && b_ok[ct]) ? ld16(xrow[ct] + a.x_lo + k) : zero;
        }
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const bf16x8 w8 = __builtin_bit_cast(bf16x8, av[rt][u]);
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, xop(bh[ct][u]), acc[rt][ct], 0, 0, 0);
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, xop(bl[ct][u]), acc[rt][ct], 0, 0, 0);
        }
  }

  // Partial tiles to LDS, then a fixed-order sum over the 8 waves.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) sm.red[wave][rt * NT + ct][j * 64 + lane] = acc[rt][ct][j];
  if (EPI != EPI_RESID) rms_finish<NT>(a, rp, sm.e.inv_rms);
  __syncthreads();
  for (int idx = tid; idx < RT * NT * 256; idx += 512) {
    const int t = idx >> 8, e = idx & 255;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < GEMM_WAVES; ++w) s += sm.red[w][t][e];
    const int rt = t / NT, ct = t % NT, j = e >> 6, ln = e & 63;
    sm.e.fin[rt][4 * (ln >> 4) + j][ct * 16 + (ln & 15)] = s;
  }
  __syncthreads();
  gemm_epilogue<EPI, NT>(a, tile, sm.e, pre);
  __syncthreads();  // LDS is reused by the next unit
}

constexpr size_t GEMM_SMEM_BYTES = sizeof(GemmSmem<2, 2>);

template <int EPI, int NT, bool NTL, int UB = 0>
__global__ __launch_bounds__(512) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GEMM_SMEM_BYTES];
  gemm_unit<EPI, NT, NTL, 0, UB>(a, blockIdx.x, smem);
}

// The arguments seen by slots s0 .. s0+n-1 only: every per-slot pointer
// advanced by s0 slots and B = n.  Lets the 16-column kernel serve slots
// 16..31 of a larger batch (blockIdx.y = slot half) with each slot's
// arithmetic unchanged.
__device__ __forceinline__ GemmArgs slot_view(const GemmArgs& a, const int s0, const int n) {
  GemmArgs v = a;
  v.B = n;
  v.X = a.X + (long)s0 * a.ldx;
  if (a.part_in) v.part_in = a.part_in + (long)s0 * a.n_part;
  if (a.q_out) v.q_out = a.q_out + (long)s0 * a.ldq;
  if (a.rope) v.rope = a.rope + (long)s0 * a.head_dim;
  if (a.kv) v.kv = a.kv + (long)s0 * a.kv_slot_stride;
  if (a.ti) v.ti = a.ti + (long)s0 * TI_STRIDE;
  if (a.x) v.x = a.x + (long)s0 * a.ldres;
  if (a.xa_out) v.xa_out = a.xa_out + (long)s0 * a.ldres;
  if (a.part_out) v.part_out = a.part_out + (long)s0 * (a.M / ROWS);
  if (a.tap) v.tap = a.tap + (long)s0 * a.ldres;
  if (a.m_out) v.m_out = a.m_out + (long)s0 * a.ldm;
  if (a.f_out) v.f_out = a.f_out + (long)s0 * a.ldf;
  if (a.amax_v) v.amax_v = a.amax_v + (long)s0 * a.ld_amax;
  if (a.amax_i) v.amax_i = a.amax_i + (long)s0 * a.ld_amax;
  return v;
}

// Slot groups: blockIdx.y takes slots G*y .. G*y+G-1 (G = a.slot_grp <= 16),
// each group the 16-column kernel; the weights are read once per group, so
// this serves cache-resident weights.  It trades weight re-reads for fewer
// activation bytes per workgroup, which is what bounds these launches once
// the batch is large.
template <int EPI, bool NTL, int UB = 0>
__global__ __launch_bounds__(512) void gemm_group_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GEMM_SMEM_BYTES];
  const int s0 = blockIdx.y * a.slot_grp;
  const GemmArgs v = slot_view(a, s0, min(a.slot_grp, a.B - s0));
  gemm_unit<EPI, 1, NTL, 0, UB>(v, blockIdx.x, smem);
}

// Slot groups with two row tiles per workgroup, for the cache-resident
// (depformer) GEMMs once the batch spans two slot groups: blockIdx.y takes
// slots G*y .. G*y+G-1 as gemm_group_kernel does, and workgroup x the TT
// output tiles TT*x .. TT*x+TT-1 (for the gated MLP each output tile is a
// gate and an up weight tile) over the whole K.  Wave w owns k-range
// R_(w+x) mod 8 of every one of them and accumulates it in k-step order, hi
// then lo, as the one-tile kernel's wave w accumulates R_w; the 8 range
// partials of a tile are summed in range order in LDS and the common epilogue
// runs per tile, so the bits are the contract's.  Each k-step's activation
// operand (16 slots) is loaded once for RT*TT weight tiles, halving the
// activation reads that bound these launches at large batch; the range
// rotation keeps neighbouring workgroups on different activation lines.
template <int EPI, int TT>
__global__ __launch_bounds__(512) void gemm_tiles_kernel(GemmArgs a0) {
  constexpr int NT = 1;
  const int gs0 = blockIdx.y * a0.slot_grp;
  const GemmArgs a = slot_view(a0, gs0, min(a0.slot_grp, a0.B - gs0));
  constexpr int RT = (EPI == EPI_GATED) ? 2 : 1, NW = RT * TT, U = 2;
  __shared__ float red[GEMM_WAVES][NW * NT][256];  // [range][weight tile * NT + column tile][element]
  __shared__ EpiSmem<RT, NT> e;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = (wave + (int)blockIdx.x) & (GEMM_WAVES - 1);  // this wave's k-range
  const int ksteps = a.K >> 5;
  const int s0 = (ksteps * rg) / GEMM_WAVES, s1 = (ksteps * (rg + 1)) / GEMM_WAVES;
  const int n_out = (a.M + ROWS - 1) / ROWS;
  const int tile0 = (int)blockIdx.x * TT;
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};

  // weight tile w = rt * TT + tt: output tile tile0 + tt (a tile past the
  // last loads the last one's weights again; its results are not stored)
  const bf16_t* arow[NW];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const long t = min(tile0 + tt, n_out - 1) + (rt ? a.gate_off / ROWS : 0);
      arow[rt * TT + tt] = a.W + t * ksteps * 512 + lane * 8;
    }
  // activation rows in row order (lane 4c + p: 16-byte piece p of slot c),
  // moved into the MFMA operand order (lane 16p + c) by a lane permute
  const int xsrc = ((lane & 15) * 4 + (lane >> 4)) * 4;
  const bf16_t* xrow[NT];
  bool b_ok[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int c = ct * 16 + (lane >> 2);
    b_ok[ct] = c < a.B;
    xrow[ct] = a.X + (long)(b_ok[ct] ? c : 0) * a.ldx + (lane & 3) * 8;
  }
  auto xop = [&](const u32x4& v) -> bf16x8 {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(xsrc, (int)v[i]);
    return __builtin_bit_cast(bf16x8, r);
  };

  EpiPre pre[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) pre[tt] = epi_preload<EPI, NT>(a, min(tile0 + tt, n_out - 1));
  RmsPre<NT> rp;
  if (EPI != EPI_RESID) rms_preload<NT>(a, rp);

  f32x4 acc[NW][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[w][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; s += U) {
    u32x4 av[NW][U], bh[NT][U], bl[NT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = (s + u) < s1;
      const int k = (s + u) * 32;
#pragma unroll
      for (int w = 0; w < NW; ++w) av[w][u] = ok ? ldw16<false>(arow[w] + (long)(s + u) * 512) : zero;
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        bh[ct][u] = (ok && b_ok[ct]) ? ld16(xrow[ct] + k) : zero;
        bl[ct][u] = (ok && b_ok[ct]) ? ld16(xrow[ct] + a.x_lo + k) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        const bf16x8 xh = xop(bh[ct][u]), xl = xop(bl[ct][u]);
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const bf16x8 w8 = __builtin_bit_cast(bf16x8, av[w][u]);
          acc[w][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, xh, acc[w][ct], 0, 0, 0);
          acc[w][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, xl, acc[w][ct], 0, 0, 0);
        }
      }
  }

#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[rg][w * NT + ct][j * 64 + lane] = acc[w][ct][j];
  if (EPI != EPI_RESID) rms_finish<NT>(a, rp, e.inv_rms);
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int tile = tile0 + tt;
    if (tile >= n_out) break;  // the same in every thread
    for (int idx = tid; idx < RT * NT * 256; idx += 512) {
      const int b = idx >> 8, el = idx & 255;
      const int rt = b / NT, ct = b % NT, j = el >> 6, ln = el & 63;
      const int blk = (rt * TT + tt) * NT + ct;
      float sum = 0.f;
#pragma unroll
      for (int r = 0; r < GEMM_WAVES; ++r) sum += red[r][blk][el];
      e.fin[rt][4 * (ln >> 4) + j][ct * 16 + (ln & 15)] = sum;
    }
    __syncthreads();
    gemm_epilogue<EPI, NT>(a, tile, e, pre[tt]);
    __syncthreads();
  }
}

// Depformer out-projection that computes its input, the attention output,
// itself (B <= DEP_FUSE_B): saves the attention launch of every layer-step.
__global__ __launch_bounds__(512) void gemm_att_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GEMM_SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) bf16_t olds[2 * DEP_FUSE_B * DEP_FUSE_D];
  gemm_unit<EPI_RESID, 1, false, 1>(a, blockIdx.x, smem, olds);
}

// Depformer first QKV projection of a codebook step that computes its input,
// the previous step's greedy finisher, itself (B <= DEP_FUSE_B): saves the
// finisher launch of every step.
__global__ __launch_bounds__(512) void gemm_fin_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[GEMM_SMEM_BYTES];
  __shared__ __attribute__((aligned(16))) bf16_t olds[2 * DEP_FUSE_B * DEP_FUSE_D];
  __shared__ float fparts[DEP_FUSE_B * (DEP_FUSE_D / 16)];
  gemm_unit<EPI_QKV, 1, false, 2>(a, blockIdx.x, smem, olds, fparts);
}

// ---------------------------------------------------------------------------
// The same GEMM for large batches (B >= WIDE_MIN_B, K >= 4096).  The per-slot
// arithmetic is the contract above, computed in another order of work.  At
// B = 32 the activation operand is 4x the weight bytes per k-step, so it is
// staged in LDS and shared by 8 weight tiles:
//
//   * gemm_wide_kernel: workgroup (g, j), j = blockIdx % 8, takes k-range R_j
//     of the 8 weight tiles 8g..8g+7, one per wave (for the gated MLP the
//     gate tiles come first, then the up tiles).  Consecutive workgroups are
//     spread over the XCDs round-robin, so all workgroups of range j share
//     one XCD's L2 for their activation slice.  Each wave streams its tile's
//     weights (non-temporal) through the staged slice and stores p_j;
//   * gemm_wide_reduce: one workgroup per output tile sums p_0..p_7 in order
//     and runs the common epilogue.
//
// Up to B = 16 every kernel of the path carries one 16-column MFMA tile
// (NT = 1): half the activation slice, half the partials and half the MFMAs
// of the 32-column form, whose second tile would hold only padding.
// ---------------------------------------------------------------------------

// k-steps per stage (activations in LDS, weights in registers).  Measured
// on the 7B device tick against 8: stages of 12 k-steps were neutral
// (-0.01 ms at B = 16, +0.01 at B = 32), of 16 slower (+0.01, +0.04).
constexpr int WIDE_SK = 8;

// Store p_j of weight tile t for NT column tiles (NT * 16 slots, NT * 256
// floats).  Default layout [t][j][ct][q][lane] (the reduce kernel reads it
// with one thread per element); with qkv_to_attn, slot-major
// [t][j][slot][16 rows], so that the decode pass reads one slot's 16 rows as
// 64 contiguous bytes.  MFMA accumulator q of lane l holds row
// 4 * (l >> 4) + q of column (slot) ct * 16 + (l & 15).
template <int NT>
__device__ __forceinline__ void store_partial(const GemmArgs& a, long t, int j, const f32x4 (&acc)[NT], int lane) {
  if (a.qkv_to_attn) {
    float* P = a.split_part + (t * GEMM_WAVES + j) * (NT * 256) + (lane & 15) * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) *reinterpret_cast<f32x4*>(P + ct * 256) = acc[ct];
  } else {
    float* P = a.split_part + (t * GEMM_WAVES + j) * (NT * 256) + lane;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q) P[ct * 256 + q * 64] = acc[ct][q];
  }
}

// LDS rows of the activation slice are 64 bytes (32 bf16 of one column);
// the 16-byte chunk `part` of column c is stored at chunk part ^ ((c >> 1) & 3),
// so the 8 lanes of a 128-bit read (8 consecutive columns, one chunk) hit 8
// different bank groups instead of 2.
__device__ __forceinline__ int xs_chunk(int c, int part) { return part ^ ((c >> 1) & 3); }

// Stage st of the k-range is software-pipelined: while the waves multiply
// stage st (weights in registers, activations in LDS buffer st & 1), the
// weights and activations of stage st + 1 are in flight; one barrier per
// stage.  Every wave still accumulates its k-range in k-step order, hi then
// lo, as the contract requires.
template <int RT, int NT>
__global__ __launch_bounds__(512) void gemm_wide_kernel(GemmArgs a) {
  constexpr int NTC = NT * 16, CS = NT == 2 ? 5 : 4;     // columns held, log2 of it
  constexpr int WIDE_XL = 2 * WIDE_SK * NTC * 4 / 512;  // 16-byte activation pieces per thread per stage
  static_assert(WIDE_XL * 512 == 2 * WIDE_SK * NTC * 4, "a stage's pieces must split evenly over 512 threads");
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][2][WIDE_SK][NTC][32];  // [buffer][hi/lo][k-step][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int j = blockIdx.x % GEMM_WAVES, grp = blockIdx.x / GEMM_WAVES;
  const int ks = a.K >> 5;
  const int s0 = (ks * j) / GEMM_WAVES, s1 = (ks * (j + 1)) / GEMM_WAVES;
  const int n_out = (a.M + ROWS - 1) / ROWS;
  const int t = grp * GEMM_WAVES + wave;  // this wave's weight tile
  const bool t_ok = t < RT * n_out;
  const long wt = (RT == 2 && t >= n_out) ? (long)(t - n_out) + a.gate_off / ROWS : (long)t;
  const bf16_t* w = a.W + (t_ok ? wt : 0) * ks * 512 + lane * 8;
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};

  // workgroup 0 also forms the slots' inverse RMS for the reduce kernel (the
  // same functions and order as every other path)
  if (a.wide_rms && blockIdx.x == 0) {
    __shared__ float inv[NTC];
    RmsPre<NT> rp;
    rms_preload<NT>(a, rp);
    rms_finish<NT>(a, rp, inv);
    __syncthreads();
    if (tid < NTC) a.wide_rms[tid] = inv[tid];
  }

  // activation piece i of a stage (i = tid + 512 u): 16 bytes of row
  // r = i >> (2 + CS), i.e. plane r / WIDE_SK and k-step r % WIDE_SK, column
  // (i >> 2) % NTC, part i & 3
  auto load_x = [&](int c0, int nsub, u32x4 (&xr)[WIDE_XL]) {
#pragma unroll
    for (int u = 0; u < WIDE_XL; ++u) {
      const int i = tid + 512 * u, r = i >> (2 + CS);
      const int part = i & 3, c = (i >> 2) & (NTC - 1), q = r % WIDE_SK, pl = r / WIDE_SK;
      xr[u] = (q < nsub && c < a.B) ? ld16(a.X + (pl ? a.x_lo : 0) + (long)c * a.ldx + (c0 + q) * 32 + part * 8) : zero;
    }
  };
  auto store_x = [&](int buf, const u32x4 (&xr)[WIDE_XL]) {
#pragma unroll
    for (int u = 0; u < WIDE_XL; ++u) {
      const int i = tid + 512 * u, r = i >> (2 + CS);
      const int part = i & 3, c = (i >> 2) & (NTC - 1), q = r % WIDE_SK, pl = r / WIDE_SK;
      *reinterpret_cast<u32x4*>(&xs[buf][pl][q][c][xs_chunk(c, part) * 8]) = xr[u];
    }
  };
  auto load_w = [&](int c0, int nsub, u32x4 (&wr)[WIDE_SK]) {
#pragma unroll
    for (int u = 0; u < WIDE_SK; ++u) wr[u] = (t_ok && u < nsub) ? ldw16<true>(w + (long)(c0 + u) * 512) : zero;
  };

  f32x4 acc[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) acc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};

  u32x4 xr[WIDE_XL], wr[WIDE_SK];
  load_x(s0, min(WIDE_SK, s1 - s0), xr);
  load_w(s0, min(WIDE_SK, s1 - s0), wr);
  store_x(0, xr);
  __syncthreads();
  for (int st = 0;; ++st) {
    const int c0 = s0 + st * WIDE_SK, nsub = min(WIDE_SK, s1 - c0);
    const int cn = c0 + WIDE_SK, nn = min(WIDE_SK, s1 - cn);
    const int buf = st & 1;
    u32x4 wn[WIDE_SK];
    if (nn > 0) {
      load_w(cn, nn, wn);
      load_x(cn, nn, xr);
    }
#pragma unroll
    for (int u = 0; u < WIDE_SK; ++u) {
      if (u < nsub) {
        const bf16x8 w8 = __builtin_bit_cast(bf16x8, wr[u]);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const u32x4 bh = *reinterpret_cast<const u32x4*>(&xs[buf][0][u][ct * 16 + r16][xs_chunk(r16, g4) * 8]);
          const u32x4 bl = *reinterpret_cast<const u32x4*>(&xs[buf][1][u][ct * 16 + r16][xs_chunk(r16, g4) * 8]);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, __builtin_bit_cast(bf16x8, bh), acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, __builtin_bit_cast(bf16x8, bl), acc[ct], 0, 0, 0);
        }
      }
    }
    if (nn <= 0) break;
    // buffer buf ^ 1 was last read in stage st - 1, before the barrier that
    // ended it
    store_x(buf ^ 1, xr);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < WIDE_SK; ++u) wr[u] = wn[u];
  }
  if (t_ok) store_partial<NT>(a, t, j, acc, lane);
}

// The same partials for k-ranges of exactly WIDE_RES k-steps (K = 4096):
// workgroup (p, j), j = blockIdx % 8, loads the activation slice of range
// R_j into LDS once, then each wave streams the weights of its TPW tiles
// p * 8 + wave + i * 8P (P = gridDim / 8, i < TPW) through it, the tiles side
// by side: each k-step's activation fragment is read from LDS once for all of
// them (a wave reading it once per tile was bound by LDS bandwidth at large
// B).  No barrier after the slice is loaded.  Per tile, a wave's accumulation
// is the contract's k-step order, hi then lo.
constexpr int WIDE_RES = 16;  // k-steps of one range held in LDS
constexpr int WIDE_RES_WGS = 512;  // workgroups: two per compute unit

inline int wide_res_tpw(long tiles) { return (int)((tiles + 8L * (WIDE_RES_WGS / 8) - 1) / (8L * (WIDE_RES_WGS / 8))); }

template <int RT, int NT, int TPW>
__global__ __launch_bounds__(512) void gemm_wide_res_kernel(GemmArgs a) {
  constexpr int NTC = NT * 16, CS = NT == 2 ? 5 : 4;  // columns held, log2 of it
  __shared__ __attribute__((aligned(16))) bf16_t xs[2][WIDE_RES][NTC][32];  // [hi/lo][k-step][column]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const int j = blockIdx.x % GEMM_WAVES, p = blockIdx.x / GEMM_WAVES, P = gridDim.x / GEMM_WAVES;
  const int ks = a.K >> 5;  // = GEMM_WAVES * WIDE_RES
  const int s0 = j * WIDE_RES;
  const int n_out = (a.M + ROWS - 1) / ROWS;
  const long T = (long)RT * n_out;
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};

  if (a.wide_rms && blockIdx.x == 0) {
    __shared__ float inv[NTC];
    RmsPre<NT> rp;
    rms_preload<NT>(a, rp);
    rms_finish<NT>(a, rp, inv);
    __syncthreads();
    if (tid < NTC) a.wide_rms[tid] = inv[tid];
  }

  // the wave's i-th tile: its weights at k-step s0 (nullptr past the last tile)
  auto tile_w = [&](int i) -> const bf16_t* {
    const long t = (long)p * GEMM_WAVES + wave + (long)i * 8 * P;
    if (t >= T) return nullptr;
    const long wt = (RT == 2 && t >= n_out) ? t - n_out + a.gate_off / ROWS : t;
    return a.W + (wt * ks + s0) * 512 + lane * 8;
  };

  // The wave's tiles advance side by side: at k-step q the activation
  // fragment is read from LDS once and multiplied into every tile's
  // accumulator; the weights of k-step q + D of every tile are requested as
  // k-step q is consumed.  Per tile the accumulation is the contract's k-step
  // order, hi then lo.
  // k-steps of each tile in flight: 8 with up to two tiles per wave (QKV at
  // B = 16 19.7 -> 19.0 us and at B = 32 22.5 -> 22.1 us against 4; 16 for
  // the one-tile out-projection was slower), fewer with more tiles, where
  // more registers would leave one workgroup per compute unit.
  constexpr int D = TPW <= 2 ? 8 : TPW == 3 ? 4 : 2;
  const bf16_t* wp[TPW];
  bool wv[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    wp[i] = tile_w(i);
    wv[i] = wp[i] != nullptr;
  }
  u32x4 wr[TPW][D];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int q = 0; q < D; ++q) wr[i][q] = wv[i] ? ldw16<true>(wp[i] + (long)q * 512) : zero;
  // the range's activation slice: piece i = tid + 512 u is 16 bytes of plane
  // i >> (6 + CS), k-step (i >> (2 + CS)) & 15, column (i >> 2) % NTC, part i & 3
#pragma unroll
  for (int u = 0; u < 2 * WIDE_RES * NTC * 4 / 512; ++u) {
    const int i = tid + 512 * u;
    const int part = i & 3, c = (i >> 2) & (NTC - 1), q = (i >> (2 + CS)) & 15, pl = i >> (6 + CS);
    const u32x4 v = ld16(a.X + (pl ? a.x_lo : 0) + (long)min(c, a.B - 1) * a.ldx + (s0 + q) * 32 + part * 8);
    *reinterpret_cast<u32x4*>(&xs[pl][q][c][xs_chunk(c, part) * 8]) = c < a.B ? v : zero;
  }
  __syncthreads();

  f32x4 acc[TPW][NT];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[i][ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < WIDE_RES; ++q) {
    u32x4 bh[NT], bl[NT];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      bh[ct] = *reinterpret_cast<const u32x4*>(&xs[0][q][ct * 16 + r16][xs_chunk(r16, g4) * 8]);
      bl[ct] = *reinterpret_cast<const u32x4*>(&xs[1][q][ct * 16 + r16][xs_chunk(r16, g4) * 8]);
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const bf16x8 w8 = __builtin_bit_cast(bf16x8, wr[i][q % D]);
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        acc[i][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, __builtin_bit_cast(bf16x8, bh[ct]), acc[i][ct], 0, 0, 0);
        acc[i][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, __builtin_bit_cast(bf16x8, bl[ct]), acc[i][ct], 0, 0, 0);
      }
      if (q + D < WIDE_RES) wr[i][q % D] = wv[i] ? ldw16<true>(wp[i] + (long)(q + D) * 512) : zero;
    }
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const long t = (long)p * GEMM_WAVES + wave + (long)i * 8 * P;
    if (wv[i]) store_partial<NT>(a, t, j, acc[i], lane);
  }
}

template <int EPI, int NT>
__global__ __launch_bounds__(512) void gemm_wide_reduce(GemmArgs a) {
  constexpr int RT = (EPI == EPI_GATED) ? 2 : 1;
  __shared__ EpiSmem<RT, NT> e;
  const int tile = blockIdx.x, tid = threadIdx.x;
  const int n_out = (a.M + ROWS - 1) / ROWS;
  // element tid (< NT * 256) of the partial tile: column tile ct,
  // accumulator q, lane ln
  const bool el = tid < NT * 256;
  float v[RT][GEMM_WAVES];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const long tt = rt ? (long)tile + n_out : (long)tile;
#pragma unroll
    for (int jj = 0; jj < GEMM_WAVES; ++jj)
      v[rt][jj] = el ? a.split_part[(tt * GEMM_WAVES + jj) * (NT * 256) + tid] : 0.f;
  }
  // inverse RMS: from the main kernel, or formed here when no buffer is given
  RmsPre<NT> rp;
  if (EPI != EPI_RESID) {
    if (a.wide_rms) {
      if (tid < NT * 16) e.inv_rms[tid] = a.wide_rms[tid];
    } else {
      rms_preload<NT>(a, rp);
    }
  }
  const EpiPre pre = epi_preload<EPI, NT>(a, tile);
  const int ct = tid >> 8, q = (tid >> 6) & 3, ln = tid & 63;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float s = 0.f;
#pragma unroll
    for (int jj = 0; jj < GEMM_WAVES; ++jj) s += v[rt][jj];
    if (el) e.fin[rt][4 * (ln >> 4) + q][ct * 16 + (ln & 15)] = s;
  }
  if (EPI != EPI_RESID && !a.wide_rms) rms_finish<NT>(a, rp, e.inv_rms);
  __syncthreads();
  gemm_epilogue<EPI, NT>(a, tile, e, pre);
}

// Row-major [M][K] bf16 -> tile layout (see gemm_unit); one thread moves the
// 16 bytes of one lane of one (tile, k-step) block; rows past M become zero.
__global__ __launch_bounds__(256) void pack_kernel(const bf16_t* src, int M, int K, bf16_t* dst) {
  const int ks = K >> 5;
  const long nblk = (long)((M + ROWS - 1) / ROWS) * ks;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;  // (block, lane)
  if (i >= nblk * 64) return;
  const long blk = i >> 6;
  const int lane = (int)(i & 63);
  const long T = blk / ks;
  const int s = (int)(blk - T * ks);
  const long row = T * ROWS + (lane & 15);
  u32x4 v = (u32x4){0u, 0u, 0u, 0u};
  if (row < M) v = ld16(src + row * K + s * 32 + (lane >> 4) * 8);
  *reinterpret_cast<u32x4*>(dst + i * 8) = v;
}

void launch_pack(const bf16_t* src, int M, int K, bf16_t* dst, hipStream_t s) {
  const long n = (long)((M + ROWS - 1) / ROWS) * (K >> 5) * 64;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, M, K, dst);
}

// Path choice per launch: both paths compute the same bits (the contract),
// so the choice only moves time.  The k-range split pays off once the
// activation operand outweighs the weights and the k-ranges are long enough
// to amortise staging and the partial exchange (K >= 4096).  Where that
// happens depends on the GEMM; each threshold below is the batch from which
// the large-batch form measured faster on the 7B device tick (the other
// GEMMs held fixed):
//   * QKV from B = 9 (-0.04 ms at B = 9, neutral at 8): its partials go
//     straight to the decode, with no reduce launch;
//   * down-projection, text head and input projections from B = 10 (neutral
//     at 9);
//   * gate/up from B = 14: its small-batch kernel, two tiles per workgroup,
//     was faster by 0.12 ms at B = 10, 0.07 at 12 and 0.025 at 13, slower by
//     0.015 at 14 and 0.11 at 16;
//   * the square out-projection (K = M) from B = 17: its 256 tiles give each
//     wave of the large-batch form a single tile, and the reduce launch costs
//     more than the activation reads it saves while one column tile holds
//     every slot (-0.07 ms at B = 10, -0.007 at 16, +0.21 at 32 on the
//     small-batch kernel).
constexpr int WIDE_B_QKV = 9, WIDE_B_DOWN_HEADS = 10, WIDE_B_GATED = 14, WIDE_B_OUT = 17;
static_assert(WIDE_MIN_B == WIDE_B_QKV && WIDE_B_DOWN_HEADS >= WIDE_MIN_B && WIDE_B_GATED >= WIDE_MIN_B &&
                  WIDE_B_OUT >= WIDE_MIN_B,
              "WIDE_MIN_B sizes the partial buffer: it must be the smallest per-GEMM threshold");
static int wide_min_b(int epi, const GemmArgs& a) {
  if (epi == EPI_QKV) return WIDE_B_QKV;
  if (epi == EPI_GATED) return WIDE_B_GATED;
  if (epi == EPI_RESID && a.K == a.M) return WIDE_B_OUT;
  return WIDE_B_DOWN_HEADS;
}

// The large-batch path needs the partial buffer: a launch given none (the
// depformer layers and heads, whose user-stream half runs on a second stream
// beside other phases of the tick) always takes the other paths.
static bool use_wide(int epi, const GemmArgs& a) {
  return a.split_part != nullptr && a.B >= wide_min_b(epi, a) && a.K >= 4096;
}

// Slots per workgroup for the other paths: 32 (both column tiles in one
// workgroup) or a group size G <= 16 (gemm_group_kernel, blockIdx.y = slot
// group).  Weights streamed from HBM once per tick are never split: every
// group would stream them again.  Cache-resident weights may be: each group
// re-reads them from the cache and carries G/B of the activation bytes.
// That pays for the depformer down-projection (K = 2816 > M = 1024, the
// largest activation row): four groups took 0.18 ms off the 7B device tick
// at B = 16 and 0.04 ms at B = 8, and were neutral at B = 32 and B = 4,
// while splitting the other depformer GEMMs further was neutral or slower.
// A wave's k-range of 9..12 k-steps (the depformer down-projection, K = 2816)
// in one load batch instead of two: these launches are latency-bound.  Only
// without slot groups: the batch's registers leave one workgroup per compute
// unit, which costs more than the saved round trip once there are groups.
// Measured on the 7B device tick: -0.029 ms at B = 1, -0.033 ms at B = 2;
// with groups +0.10 ms at B = 8 and +0.11 ms at B = 32.
static bool deep_batch(const GemmArgs& a) {
  const int per_wave = ((a.K >> 5) + GEMM_WAVES - 1) / GEMM_WAVES;
  return per_wave > 8 && per_wave <= 12;
}

static int slot_group(int epi, const GemmArgs& a) {
  if (a.w_keep && epi == EPI_RESID && a.K > a.M && a.B >= 8) return (a.B + 3) / 4;
  if (a.B <= 16) return 16;
  return a.w_keep ? 16 : 32;
}

template <int EPI>
static void launch_gemm_nt(const GemmArgs& a, hipStream_t s) {
  const int tiles = (a.M + ROWS - 1) / ROWS;
  constexpr bool TILES2 = EPI == EPI_QKV || EPI == EPI_GATED || EPI == EPI_RESID;  // epilogues with a two-tile form
  if (EPI == EPI_RESID && a.fuse_att) {  // caller guarantees B <= DEP_FUSE_B, K <= DEP_FUSE_D
    hipLaunchKernelGGL(gemm_att_kernel, dim3(tiles), dim3(512), 0, s, a);
    return;
  }
  if (EPI == EPI_QKV && a.fuse_fin) {  // caller guarantees B <= DEP_FUSE_B, K <= DEP_FUSE_D, greedy choice
    hipLaunchKernelGGL(gemm_fin_kernel, dim3(tiles), dim3(512), 0, s, a);
    return;
  }
  if (use_wide(EPI, a)) {
    const long groups = (wide_tiles(EPI, a.M) + GEMM_WAVES - 1) / GEMM_WAVES;
    GemmArgs w = a;
    if (EPI == EPI_RESID) w.wide_rms = nullptr;  // no normalised input
    constexpr int RT = EPI == EPI_GATED ? 2 : 1;
    const bool one = gemm_wide_cols(a) == 16;  // one 16-column tile holds every slot
    if ((a.K >> 5) == GEMM_WAVES * WIDE_RES) {
      const long T = wide_tiles(EPI, a.M);
      const long P = (T + 8L * wide_res_tpw(T) - 1) / (8L * wide_res_tpw(T));
      // the wave's tiles side by side (TPW in registers).  Measured on the 7B
      // device tick with every ring full, against one tile after another:
      // -0.19 to -0.30 ms at B = 32, -0.14 ms at B = 16 (gate/up 4.16 -> 4.33
      // TB/s and QKV 4.34 -> 4.54 TB/s at B = 32)
      const int tpw = wide_res_tpw(T);
      auto go = [&](auto tp) {
        constexpr int TP = decltype(tp)::value;
        if (one) hipLaunchKernelGGL((gemm_wide_res_kernel<RT, 1, TP>), dim3(P * GEMM_WAVES), dim3(512), 0, s, w);
        else hipLaunchKernelGGL((gemm_wide_res_kernel<RT, 2, TP>), dim3(P * GEMM_WAVES), dim3(512), 0, s, w);
      };
      if (tpw <= 1) go(std::integral_constant<int, 1>{});
      else if (tpw == 2) go(std::integral_constant<int, 2>{});
      else if (tpw == 3) go(std::integral_constant<int, 3>{});
      else go(std::integral_constant<int, 4>{});
    } else {
      if (one) hipLaunchKernelGGL((gemm_wide_kernel<RT, 1>), dim3(groups * GEMM_WAVES), dim3(512), 0, s, w);
      else hipLaunchKernelGGL((gemm_wide_kernel<RT, 2>), dim3(groups * GEMM_WAVES), dim3(512), 0, s, w);
    }
    if (!(EPI == EPI_QKV && a.qkv_to_attn)) {
      if (one) hipLaunchKernelGGL((gemm_wide_reduce<EPI, 1>), dim3(tiles), dim3(512), 0, s, w);
      else hipLaunchKernelGGL((gemm_wide_reduce<EPI, 2>), dim3(tiles), dim3(512), 0, s, w);
    }
  } else {
    const int G = slot_group(EPI, a);
    GemmArgs v = a;
    v.slot_grp = G;
    const unsigned groups = (unsigned)((a.B + G - 1) / G);
    if (G > 16) {
      if (a.w_keep) hipLaunchKernelGGL((gemm_kernel<EPI, 2, false>), dim3(tiles), dim3(512), 0, s, v);
      else hipLaunchKernelGGL((gemm_kernel<EPI, 2, true>), dim3(tiles), dim3(512), 0, s, v);
    } else if (EPI == EPI_RESID && a.w_keep && groups == 1 && deep_batch(a)) {
      // cache-resident weights, 9..12 k-steps per wave, one workgroup per
      // tile: the whole k-range in one load batch
      hipLaunchKernelGGL((gemm_kernel<EPI_RESID, 1, false, 12>), dim3(tiles), dim3(512), 0, s, v);
    } else if (EPI == EPI_RESID && !a.w_keep && groups == 1 && a.K > a.M) {
      // streamed down-projection (K = 11264: 44 k-steps per wave) in load
      // batches of 4 k-steps: 72 registers instead of 120.  Measured on the
      // 7B device tick: -0.03 ms at B = 1, -0.04 at B = 4, -0.06 at B = 8;
      // batches of 2, 3, 6 and 16 were slower than 4.
      hipLaunchKernelGGL((gemm_kernel<EPI_RESID, 1, true, 4>), dim3(tiles), dim3(512), 0, s, v);
    } else if (TILES2 && a.w_keep && groups > 1 && (EPI != EPI_RESID || a.K == a.M)) {
      // cache-resident weights, two slot groups or more: two row tiles per
      // workgroup.  Measured on the 7B device tick with every ring full, for
      // the QKV, gate/up and out-projection GEMMs of the depformer: -0.16 ms
      // at B = 24, -0.22 ms at B = 32.  With one group it lost (+0.04 ms at
      // B = 8, 12 and 16); at B = 32, against two tiles, so did 4 tiles
      // (+0.27 ms), 3 tiles for QKV (+0.03 ms) and the down-projection in
      // two-tile groups of 16 slots (+0.08 ms)
      if constexpr (TILES2) hipLaunchKernelGGL((gemm_tiles_kernel<EPI, 2>), dim3((tiles + 1) / 2, groups), dim3(512), 0, s, v);
    } else if (EPI == EPI_RESID && a.w_keep && G >= 8 && deep_batch(a)) {
      // the depformer down-projection in slot groups of 8 or more: the whole
      // k-range in one load batch (256 workgroups, one per compute unit).
      // Measured on the 7B device tick with every ring full: -0.05 to -0.10
      // ms at B = 32 (groups of 8); with groups of 4 and 2 (B = 16 and 8) it
      // was slower, +0.12 and +0.10 ms
      hipLaunchKernelGGL((gemm_group_kernel<EPI_RESID, false, 12>), dim3(tiles, groups), dim3(512), 0, s, v);
    } else if (groups > 1) {
      if (a.w_keep) hipLaunchKernelGGL((gemm_group_kernel<EPI, false>), dim3(tiles, groups), dim3(512), 0, s, v);
      else hipLaunchKernelGGL((gemm_group_kernel<EPI, true>), dim3(tiles, groups), dim3(512), 0, s, v);
    } else {
      if (a.w_keep) hipLaunchKernelGGL((gemm_kernel<EPI, 1, false>), dim3(tiles), dim3(512), 0, s, v);
      else hipLaunchKernelGGL((gemm_kernel<EPI, 1, true>), dim3(tiles), dim3(512), 0, s, v);
    }
  }
}

int gemm_wide_cols(const GemmArgs& a) { return a.B <= 16 ? 16 : 32; }

bool gemm_splits_k(Epi epi, const GemmArgs& a) {
  return !(epi == EPI_RESID && a.fuse_att) && !(epi == EPI_QKV && a.fuse_fin) && use_wide(epi, a);
}

void launch_gemm(Epi epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_QKV: launch_gemm_nt<EPI_QKV>(a, s); break;
    case EPI_RESID: launch_gemm_nt<EPI_RESID>(a, s); break;
    case EPI_GATED: launch_gemm_nt<EPI_GATED>(a, s); break;
    case EPI_LOGITS: launch_gemm_nt<EPI_LOGITS>(a, s); break;
    case EPI_STORE: launch_gemm_nt<EPI_STORE>(a, s); break;
  }
}

// ---------------------------------------------------------------------------
// Split-K flash-decoding over the ring.
//
// Slot b at absolute position pos attends to the n = min(pos+1, W) most
// recent positions p = pos-n+1 .. pos, stored at ring index p mod W (guide,
// "架构": fixed-capacity ring KV; recipe: sliding window 3000 frames).  The
// keys are visited in position order in fixed splits of ATT_CHUNK keys; one
// workgroup (4 waves x 64 keys) per (head, slot, split) produces the split's
// running max, sum of exponentials and unnormalised output; the last split to
// finish combines all of them in split order.  With a single split the
// workgroup writes the normalised output itself.  Lanes: head_dim/8 lanes share one key
// (16 bytes each, coalesced 256-byte rows for head_dim 128).
// ---------------------------------------------------------------------------

struct AttnPos {
  int pos, n, lo, nc;
};

__device__ __forceinline__ AttnPos attn_pos(const AttnArgs& a, int b) {
  AttnPos p;
  p.pos = a.ti ? a.ti[b * TI_STRIDE + TI_POS] : a.pos_const;
  p.n = min(p.pos + 1, a.window);
  p.lo = p.pos + 1 - p.n;
  p.nc = (p.n + ATT_CHUNK - 1) / ATT_CHUNK;
  return p;
}

// One (head, slot, split) of the decode pass, computed by waves 0..3 of the
// workgroup.  Keys and values of the split are requested together up front
// (the values do not depend on the scores).  With several splits, each
// writes (max, sum of exponentials, unnormalised output) through
// device-coherent stores and takes an integer ticket; the last split of the
// (slot, head) combines all splits in split order and writes the output.
template <int DH>
__device__ void attn_unit(const AttnArgs& a, const int h, const int b, const int c) {
  constexpr int LPK = DH / 8;
  constexpr int KPI = 64 / LPK;
  constexpr int ITER = 64 / KPI;
  const AttnPos P = attn_pos(a, b);
  if (c >= P.nc) return;
  const bool active = threadIdx.x < 256;
  const int k0 = c * ATT_CHUNK;
  const int kn = min(ATT_CHUNK, P.n - k0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPK, kg = lane / LPK;
  const float scale = 1.0f / sqrtf((float)DH);

  const bool fused = a.qkv_part != nullptr;
  const bool last = c == P.nc - 1;  // the split that holds the current position (its last key)
  float qv[8];
  if (!fused) {
    const float* qp = a.q + (long)b * a.ldq + h * DH + sub * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qp[i];
  }

  // Ring row of key j: (r0 + j) mod W, with r0 < W and j < W.  The head's
  // key and value bases are uniform; one 32-bit lane offset serves both.
  const int r0 = (P.lo + k0) % a.window;
  const char* kbase = reinterpret_cast<const char*>(a.kv + (long)b * a.kv_slot_stride + (long)h * a.window * DH);
  const char* vbase = kbase + a.kv_v_off * (long)sizeof(bf16_t);
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
  u32x4 kr[ITER], vr[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = active ? wave * 64 + it * KPI + kg : ATT_CHUNK;
    kr[it] = zero;
    vr[it] = zero;
    if (j < kn) {
      int row = r0 + j;
      row -= row >= a.window ? a.window : 0;
      const uint32_t off = (uint32_t)(row * DH + sub * 8) * (uint32_t)sizeof(bf16_t);
      kr[it] = ldw16<true>(reinterpret_cast<const bf16_t*>(kbase + off));  // read once per tick: non-temporal
      vr[it] = ldw16<true>(reinterpret_cast<const bf16_t*>(vbase + off));
    }
  }

  // Large-batch path: finish this head's q (and, in the last split, k and v)
  // from the QKV partials while the keys and values are in flight.  Row r of
  // vector `which` (0 q, 1 k, 2 v) is GEMM row which * d + h * DH + r, in
  // tile T = row / 16; the 8 range partials of (T, slot b) are 16 contiguous
  // rows.  Sums in range order, then qkv_pair: the bits of the reduce kernel.
  __shared__ float qp_s[3][DH][GEMM_WAVES + 1];
  __shared__ float q_s[DH];
  __shared__ __attribute__((aligned(16))) bf16_t kv_s[2][DH];
  if (fused) {
    const int nvec = last ? 3 : 1;
    const int tiles_d = a.n_heads * DH / ROWS;
    // piece i: vector i / (2 DH), tile (i / 32) % (DH / 16), range (i / 4) % 8,
    // rows 4 (i % 4) .. +3 (16 bytes)
#pragma unroll 1
    for (int i = threadIdx.x; i < nvec * 2 * DH; i += blockDim.x) {
      const int which = i / (2 * DH), ii = i - which * 2 * DH;
      const int ti = ii >> 5, jj = (ii >> 2) & 7, qq = ii & 3;
      const long T = (long)which * tiles_d + h * (DH / ROWS) + ti;
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.qkv_part + ((T * GEMM_WAVES + jj) * a.qkv_cols + b) * 16 + 4 * qq);
#pragma unroll
      for (int r = 0; r < 4; ++r) qp_s[which][ti * 16 + 4 * qq + r][jj] = v[r];
    }
    __syncthreads();
    const int pos = P.pos;
    if ((int)threadIdx.x < nvec * (DH / 2)) {
      const int which = threadIdx.x / (DH / 2), pr = threadIdx.x - which * (DH / 2);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int jj = 0; jj < GEMM_WAVES; ++jj) s0 += qp_s[which][2 * pr][jj];
#pragma unroll
      for (int jj = 0; jj < GEMM_WAVES; ++jj) s1 += qp_s[which][2 * pr + 1][jj];
      const float cs = a.rope[(long)b * DH + 2 * pr], sn = a.rope[(long)b * DH + 2 * pr + 1];
      float y0, y1;
      qkv_pair(s0, s1, a.qkv_rms[b], which < 2, cs, sn, y0, y1);
      if (which == 0) {
        q_s[2 * pr] = y0;
        q_s[2 * pr + 1] = y1;
      } else {
        const bf16_t e0 = f2bf(y0), e1 = f2bf(y1);
        kv_s[which - 1][2 * pr] = e0;
        kv_s[which - 1][2 * pr + 1] = e1;
        bf16_t* dst = a.kv + (long)b * a.kv_slot_stride + (which == 2 ? a.kv_v_off : 0) +
                      ((long)h * a.window + (pos % a.window)) * DH + 2 * pr;
        dst[0] = e0;
        dst[1] = e1;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = q_s[sub * 8 + i];
  }
  // the current key and value (last key of the last split) from LDS: the
  // ring row loaded above still holds the position W ticks back
  auto key_at = [&](int it, int j) -> u32x4 {
    return (fused && last && j == kn - 1) ? *reinterpret_cast<const u32x4*>(&kv_s[0][sub * 8]) : kr[it];
  };
  auto val_at = [&](int it, int j) -> u32x4 {
    return (fused && last && j == kn - 1) ? *reinterpret_cast<const u32x4*>(&kv_s[1][sub * 8]) : vr[it];
  };

  float s[ITER];
  float mloc = -INFINITY;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = active ? wave * 64 + it * KPI + kg : ATT_CHUNK;
    float kf[8];
    unpack8(key_at(it, j), kf);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dot += qv[i] * kf[i];
    dot = group_sum<LPK>(dot);
    s[it] = (j < kn) ? dot * scale : -INFINITY;
    mloc = fmaxf(mloc, s[it]);
  }
  mloc = group_max<64>(mloc);

  float lsum = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int j = active ? wave * 64 + it * KPI + kg : ATT_CHUNK;
    if (j < kn) {
      const float p = expf(s[it] - mloc);
      if (sub == 0) lsum += p;
      float vf[8];
      unpack8(val_at(it, j), vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] += p * vf[i];
    }
  }
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] += __shfl_xor(o[i], off);
  lsum = group_sum<64>(lsum);

  __shared__ float sm_m[4], sm_l[4], sm_o[4][DH];
  __shared__ int is_last;
  if (active && lane == 0) {
    sm_m[wave] = mloc;
    sm_l[wave] = lsum;
  }
  if (active && kg == 0)
#pragma unroll
    for (int i = 0; i < 8; ++i) sm_o[wave][sub * 8 + i] = o[i];
  __syncthreads();
  const int e = threadIdx.x;
  float M = 0.f, L = 0.f, O = 0.f;
  if (e < DH) {
    M = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (sm_m[w] == -INFINITY) ? 0.f : expf(sm_m[w] - M);
      L += sm_l[w] * f;
      O += sm_o[w][e] * f;
    }
  }
  if (P.nc == 1) {
    if (e < DH) store_split(a.o + (long)b * a.ldo + h * DH + e, a.o_lo, O / L);
    __syncthreads();  // LDS is reused by the next unit
    return;
  }
  float* base = a.part + ((long)b * a.n_heads + h) * a.max_chunks * (DH + 2);
  if (e < DH) {
    float* pp = base + c * (DH + 2);
    __hip_atomic_store(pp + 2 + e, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e == 0) {
      __hip_atomic_store(pp, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pp + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* cnt = a.cnt + (long)b * a.n_heads + h;
    const unsigned prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev == (unsigned)P.nc - 1;
    if (is_last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (is_last && e < DH) {
    // every split's (max, sum, output) requested before any is used
    float mv[ATT_MAX_SPLITS], lv[ATT_MAX_SPLITS], ov[ATT_MAX_SPLITS];
#pragma unroll
    for (int cc = 0; cc < ATT_MAX_SPLITS; ++cc) {
      const float* pp = base + cc * (DH + 2);
      const bool ok = cc < P.nc;
      mv[cc] = ok ? __hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -INFINITY;
      lv[cc] = ok ? __hip_atomic_load(pp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
      ov[cc] = ok ? __hip_atomic_load(pp + 2 + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
    }
    float Mx = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < ATT_MAX_SPLITS; ++cc)
      if (cc < P.nc) Mx = fmaxf(Mx, mv[cc]);
    float Lx = 0.f, Ox = 0.f;
#pragma unroll
    for (int cc = 0; cc < ATT_MAX_SPLITS; ++cc) {
      if (cc < P.nc) {
        const float f = expf(mv[cc] - Mx);
        Lx += lv[cc] * f;
        Ox += ov[cc] * f;
      }
    }
    store_split(a.o + (long)b * a.ldo + h * DH + e, a.o_lo, Ox / Lx);
  }
  __syncthreads();  // LDS is reused by the next unit
}

template <int DH>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  attn_unit<DH>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

template <int DH>
static void launch_attn_dh(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_kernel<DH>), dim3(a.n_heads, a.B, a.max_chunks), dim3(256), 0, s, a);
}

void launch_attention(const AttnArgs& a, hipStream_t s) {
  switch (a.head_dim) {
    case 32: launch_attn_dh<32>(a, s); break;
    case 64: launch_attn_dh<64>(a, s); break;
    default: launch_attn_dh<128>(a, s); break;
  }
}


// ---------------------------------------------------------------------------
// 17-way embedding gather-sum: x_b = sum over rows r of table_r[col_b[r]], in
// row order in fp32 (column layout: recipe, "Architecture").  Also stores
// bf16(x * alpha) for the first QKV projection, the per-16 sums of squares
// and the hidden-state tap.
// ---------------------------------------------------------------------------

// One thread per 8 features of one slot: the 17 row indices are read first,
// then all 17 row segments are requested before any is summed, so the gather
// costs one memory round trip.  Rows are summed in row order r = 0..16.
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int b = blockIdx.y;
  // the tick's RoPE table for this slot: angle pos * base^(-2i/head_dim) in
  // fp64, cos and sin rounded to fp32 (every layer's QKV epilogue reads it)
  if (a.rope && blockIdx.x == 0) {
    const int pos = a.ti[b * TI_STRIDE + TI_POS];
    for (int i = threadIdx.x; i < a.head_dim / 2; i += blockDim.x) {
      const double th = (double)pos * a.inv_freq[i];
      a.rope[(long)b * a.head_dim + 2 * i] = (float)cos(th);
      a.rope[(long)b * a.head_dim + 2 * i + 1] = (float)sin(th);
    }
  }
  const int g8 = blockIdx.x * blockDim.x + threadIdx.x;  // 8-feature group
  if (g8 >= a.d / 8) return;                              // d % 16 == 0: pairs stay whole
  const int* t = a.ti + b * TI_STRIDE + TI_COL;
  const long off = (long)b * a.d + g8 * 8;
  float acc[8];
  if (a.xin && a.ti[b * TI_STRIDE + TI_XIN]) {
    // embedding-form prefill frame: the given input replaces the gather-sum
    // (the flag is per slot, so the branch is uniform over the workgroup)
    const float4 x0 = *reinterpret_cast<const float4*>(a.xin + off);
    const float4 x1 = *reinterpret_cast<const float4*>(a.xin + off + 4);
    acc[0] = x0.x; acc[1] = x0.y; acc[2] = x0.z; acc[3] = x0.w;
    acc[4] = x1.x; acc[5] = x1.y; acc[6] = x1.z; acc[7] = x1.w;
  } else {
    u32x4 v[17];
#pragma unroll
    for (int r = 0; r < 17; ++r) {
      const bf16_t* e = (r == 0) ? a.emb_text + (long)t[0] * a.d
                                 : a.emb_audio + ((long)(r - 1) * a.audio_rows + t[r]) * a.d;
      v[r] = ld16(e + g8 * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int r = 0; r < 17; ++r) {
      float f[8];
      unpack8(v[r], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a.x[off + i] = acc[i];
    a.tap[off + i] = acc[i];
    store_split(a.xa + off + i, a.xa_lo, acc[i] * a.alpha[g8 * 8 + i]);
    ss += acc[i] * acc[i];
  }
  ss += __shfl_xor(ss, 1);  // the two halves of a 16-feature group are adjacent lanes
  if ((g8 & 1) == 0) a.part[(long)b * (a.d / 16) + g8 / 2] = ss;
}

void launch_embed(const EmbedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3((a.d / 8 + 255) / 256, a.B), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// Head finisher: greedy token of one head (text or depformer codebook `step`)
// from the per-workgroup (max, argmax) partials, forced choice applied
// (recipe: voice forces the agent stream, persona the text stream), and the
// next depformer step's input e = P_{k+1} z + table_{k+1}[chosen] with its
// normalisation partials.
// ---------------------------------------------------------------------------

// Slot b of the finisher, computed by the whole workgroup (up to 512
// threads).  The argmax selection (largest value, then lowest index) does not
// depend on the reduction tree, so the block size does not change results.

// ---------------------------------------------------------------------------
// Sampling variant of the token choice (the guides' deployment knobs:
// temperature, top-p, repetition penalty; top-k).  For one logits row, in
// this order: the repetition penalty on the text row (a positive logit of a
// recently chosen token divided by rho, a negative one multiplied; each
// distinct token once); z = logit / T (T = 0: the argmax of the penalised
// logits, lowest index on ties); top-k = the k first entries of the order
// (z descending, index ascending); p = exp(z - max) over the kept entries;
// top-p = the shortest prefix of the order (p descending, index ascending)
// whose sum reaches top_p times the total; then the inverse CDF over the
// kept entries in index order at u times their sum.  u = Philox4x32-10
// (Salmon, Moraes, Dror and Shaw, SC 2011) of counter (tick since the slot's
// reset, row, 0) and key (the slot's seed), first word >> 8, times 2^-24;
// row 0 is the text token, 1 + k codebook k.
//
// One 256-thread workgroup per decision; the row lives in LDS; thread t owns
// the contiguous entries [t * per, (t + 1) * per).  The k-th largest z and
// the top-p threshold are found by bisection over order-preserving 32-bit
// keys (32 counting passes each), ties resolved in index order with a scan.
// ---------------------------------------------------------------------------

constexpr int SAMPLE_NT = 256;

__device__ __forceinline__ void philox4x32_10(unsigned c[4], unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const unsigned lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const unsigned n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// larger float -> larger key (for -0 canonicalised to +0 beforehand)
__device__ __forceinline__ unsigned order_key(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct SampleSmem {
  int i[SAMPLE_NT];
  float red[4];
  int redi[4];
  float red3[3][4];
};

__device__ __forceinline__ float blk_sum(float v, SampleSmem& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) sh.red[wave] = v;
  __syncthreads();
  return ((sh.red[0] + sh.red[1]) + sh.red[2]) + sh.red[3];
}

// three sums at once (the 4-way threshold search)
__device__ __forceinline__ void blk_sum3(float (&v)[3], SampleSmem& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v[j] += __shfl_xor(v[j], off);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int j = 0; j < 3; ++j) sh.red3[j][wave] = v[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 3; ++j) v[j] = ((sh.red3[j][0] + sh.red3[j][1]) + sh.red3[j][2]) + sh.red3[j][3];
}

__device__ __forceinline__ int blk_isum(int v, SampleSmem& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) sh.redi[wave] = v;
  __syncthreads();
  return sh.redi[0] + sh.redi[1] + sh.redi[2] + sh.redi[3];
}

__device__ __forceinline__ float blk_max(float v, SampleSmem& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sh.red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh.red[0], sh.red[1]), fmaxf(sh.red[2], sh.red[3]));
}

__device__ __forceinline__ int blk_imin(int v, SampleSmem& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) sh.redi[wave] = v;
  __syncthreads();
  return min(min(sh.redi[0], sh.redi[1]), min(sh.redi[2], sh.redi[3]));
}

// exclusive prefix of the threads' values in thread order (a fixed
// shuffle-up scan within each wave, then the wave totals in order); returns
// this thread's prefix, *total the sum of all
__device__ __forceinline__ float blk_scan(float v, SampleSmem& sh, float* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == 63) sh.red[wave] = inc;
  __syncthreads();
  float base = 0.f;
  for (int w = 0; w < wave; ++w) base += sh.red[w];
  *total = ((sh.red[0] + sh.red[1]) + sh.red[2]) + sh.red[3];
  return base + (inc - v);
}

__device__ __forceinline__ int blk_iscan(int v, SampleSmem& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == 63) sh.redi[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += sh.redi[w];
  return base + inc - v;
}

// The sampled token of slot b for the finisher's row; z: LDS of n floats.
__device__ int sample_row(const FinishArgs& a, const int b, const unsigned* ctx, float* z, SampleSmem& sh) {
  const SampleParams sp = *a.sp;
  const int n = a.n_logits, tid = threadIdx.x;
  const int per = (n + SAMPLE_NT - 1) / SAMPLE_NT, i0 = min(n, tid * per), i1 = min(n, i0 + per);
  const float* lg = a.logits + (long)b * a.ld_logits;
  // the row into LDS, 16 loads in flight per thread
  for (int i0b = 0; i0b < n; i0b += 16 * SAMPLE_NT) {
    float v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = i0b + q * SAMPLE_NT + tid;
      v[q] = lg[min(i, n - 1)];
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int i = i0b + q * SAMPLE_NT + tid;
      if (i < n) z[i] = v[q];
    }
  }
  if (a.step < 0 && sp.rho != 1.f) {
    if (tid < SAMPLE_REP) sh.i[tid] = a.rep[(long)b * SAMPLE_REP + tid];
    __syncthreads();
    if (tid < SAMPLE_REP) {
      const int v = sh.i[tid];
      bool first = v >= 0 && v < n;
      for (int j = 0; j < tid; ++j) first = first && sh.i[j] != v;
      if (first) {
        const float x = z[v];
        z[v] = x > 0.f ? x / sp.rho : x * sp.rho;
      }
    }
  }
  __syncthreads();
  const float T = a.step < 0 ? sp.t_text : sp.t_audio;
  if (T == 0.f) {  // argmax of the penalised logits, lowest index on ties
    float bv = -INFINITY;
    int bi = n;
#pragma unroll 8
    for (int i = i0; i < i1; ++i)
      if (z[i] > bv || bi == n) { bv = z[i]; bi = i; }
    const float m = blk_max(bv, sh);
    return blk_imin(bv == m ? bi : n, sh);
  }
#pragma unroll 8
  for (int i = i0; i < i1; ++i) z[i] = z[i] / T + 0.0f;  // + 0 turns -0 into +0
  __syncthreads();
  if (sp.top_k > 0 && sp.top_k < n) {
    // res = the largest key t with count(key >= t) >= k (the k-th largest),
    // two bits per pass: the counts of the three candidates go out together
    unsigned res = 0;
    for (int sh2 = 30; sh2 >= 0; sh2 -= 2) {
      float c[3] = {0.f, 0.f, 0.f};  // counts below 2^24: exact in fp32
#pragma unroll 8
      for (int i = i0; i < i1; ++i) {
        const unsigned k = order_key(z[i]);
#pragma unroll
        for (int d = 1; d <= 3; ++d) c[d - 1] += k >= (res | ((unsigned)d << sh2)) ? 1.f : 0.f;
      }
      blk_sum3(c, sh);
      int dd = 0;
#pragma unroll
      for (int d = 1; d <= 3; ++d)
        if (c[d - 1] >= (float)sp.top_k) dd = d;
      res |= (unsigned)dd << sh2;
    }
    int gt = 0, eq = 0;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
      const unsigned k = order_key(z[i]);
      gt += k > res;
      eq += k == res;
    }
    const int need = sp.top_k - blk_isum(gt, sh);
    int rank = blk_iscan(eq, sh);
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
      const unsigned k = order_key(z[i]);
      bool keep = k > res;
      if (k == res) keep = rank++ < need;
      if (!keep) z[i] = -INFINITY;
    }
    __syncthreads();
  }
  float mx = -INFINITY;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) mx = fmaxf(mx, z[i]);
  const float m = blk_max(mx, sh);
  float cs = 0.f;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) {
    const float p = z[i] == -INFINITY ? 0.f : expf(z[i] - m);
    z[i] = p;
    cs += p;
  }
  __syncthreads();
  if (sp.top_p < 1.f) {
    const float target = sp.top_p * blk_sum(cs, sh);
    // res = the largest t with the sum of p over bits(p) >= t reaching the
    // target (0 <= p <= 1: its bits order like its value and stay below
    // 2^30); two bits per pass, three candidate sums together
    unsigned res = 0;
    for (int sh2 = 28; sh2 >= 0; sh2 -= 2) {
      float sm[3] = {0.f, 0.f, 0.f};
#pragma unroll 8
      for (int i = i0; i < i1; ++i) {
        const unsigned k = __float_as_uint(z[i]);
#pragma unroll
        for (int d = 1; d <= 3; ++d) sm[d - 1] += k >= (res | ((unsigned)d << sh2)) ? z[i] : 0.f;
      }
      blk_sum3(sm, sh);
      int dd = 0;
#pragma unroll
      for (int d = 1; d <= 3; ++d)
        if (sm[d - 1] >= target) dd = d;
      res |= (unsigned)dd << sh2;
    }
    float g = 0.f, eq = 0.f;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
      const unsigned k = __float_as_uint(z[i]);
      g += k > res ? z[i] : 0.f;
      eq += k == res ? z[i] : 0.f;
    }
    const float G = blk_sum(g, sh);
    float tot;
    float run = blk_scan(eq, sh, &tot);
    cs = 0.f;
#pragma unroll 8
    for (int i = i0; i < i1; ++i) {
      const unsigned k = __float_as_uint(z[i]);
      bool keep = k > res;
      if (k == res) {
        keep = G + run < target;
        run += z[i];
      }
      if (!keep) z[i] = 0.f;
      cs += z[i];
    }
    __syncthreads();
  }
  unsigned c[4] = {ctx[2], ctx[3], (unsigned)(a.step + 1), 0u};
  philox4x32_10(c, ctx[0], ctx[1]);
  const float u = (float)(c[0] >> 8) * 5.9604644775390625e-8f;  // 2^-24
  float total;
  float run = blk_scan(cs, sh, &total);
  const float target = u * total;
  int pick = n, last = -1;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) {
    if (z[i] > 0.f) {
      last = i;
      run += z[i];
      if (pick == n && run > target) pick = i;
    }
  }
  pick = blk_imin(pick, sh);
  if (pick == n) pick = -blk_imin(-last, sh);  // rounding left the target at the total: the last kept entry
  return pick;
}

__device__ void finish_unit(const FinishArgs& a, const int b, float* zrow) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sv[8];
  __shared__ int si[8];
  __shared__ int chosen_s;
  const int nk = a.step + 1;
  const bool next = nk < a.dep_q;
  // Requests that do not depend on the choice go out first: the forced
  // token, and this thread's first 16-feature group of u_{k+1} and alpha.
  const int forced = (tid == 0 && a.step < 8) ? a.ti[b * TI_STRIDE + TI_FORCE + 1 + a.step] : -1;
  const float* u = a.u + ((long)b * a.dep_q + nk) * a.dd;
  float u0[16], al0[16];
  const bool has0 = next && tid < a.dd / 16;
  if (has0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      u0[i] = u[tid * 16 + i];
      al0[i] = a.alpha[tid * 16 + i];
    }
  }
  // per-thread contiguous range, strict '>' so the lowest index wins ties;
  // the range is read 8 entries at a time, all 8 requested before any is used
  const int per = (a.n_part + nt - 1) / nt;
  const int t0 = tid * per, t1 = min(a.n_part, t0 + per);
  const float* pv = a.amax_v + (long)b * a.ld_amax;
  const int* pi = a.amax_i + (long)b * a.ld_amax;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int t = t0; t < t1; t += 8) {
    float vv[8];
    int ii[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = t + j < t1;
      vv[j] = ok ? pv[t + j] : 0.f;
      ii[j] = ok ? pi[t + j] : 0x7fffffff;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (ii[j] != 0x7fffffff && (vv[j] > bv || bi == 0x7fffffff)) { bv = vv[j]; bi = ii[j]; }
  }
  // wave butterfly, then the waves' winners in LDS (the winner does not
  // depend on the reduction order)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float v2 = __shfl_xor(bv, off);
    const int i2 = __shfl_xor(bi, off);
    if (amax_better(v2, i2, bv, bi)) { bv = v2; bi = i2; }
  }
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  // sampling: the slot's (seed, tick) travel from the tick input (text
  // finisher) to the codebook finishers through a.sctx
  __shared__ SampleSmem ssm;
  __shared__ int spred;
  const bool samp = a.sp && a.sp->enabled;
  if (samp) {
    unsigned* ctx = a.sctx + (long)b * 4;
    if (a.step < 0) {
      __shared__ unsigned tctx[4];
      if (tid < 4) tctx[tid] = (unsigned)a.ti[b * TI_STRIDE + TI_SEED + tid];
      __syncthreads();
      if (tid < 4) ctx[tid] = tctx[tid];
      const int p = sample_row(a, b, tctx, zrow, ssm);
      if (tid == 0) spred = p;
    } else {
      __shared__ unsigned uctx[4];
      if (tid < 4) uctx[tid] = ctx[tid];
      __syncthreads();
      const int p = sample_row(a, b, uctx, zrow, ssm);
      if (tid == 0) spred = p;
    }
    __syncthreads();
  }
  if (tid == 0) {
    for (int w = 1; w < nt / 64; ++w)
      if (amax_better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    const int pred = samp ? spred : bi;
    int* to = a.to + b * TO_STRIDE;
    const int chosen = forced >= 0 ? forced : pred;  // step -1 -> text force
    if (a.step < 8) {
      to[TO_PRED + 1 + a.step] = pred;
      to[TO_CHOSEN + 1 + a.step] = chosen;
    } else {
      to[TO_USER + a.step - 8] = pred;
    }
    chosen_s = chosen;
  }
  __syncthreads();
  const int tok = chosen_s;
  const bf16_t* e = a.table + (long)tok * a.dd;
  for (int grp = tid; next && grp < a.dd / 16; grp += nt) {
    float f[16];
    unpack8(ld16(e + grp * 16), f);
    unpack8(ld16(e + grp * 16 + 8), f + 8);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = grp * 16 + i;
      const float um = grp == tid ? u0[i] : u[m];
      const float am = grp == tid ? al0[i] : a.alpha[m];
      const float v = um + f[i];
      a.y[(long)b * a.dd + m] = v;
      store_split(a.ya + (long)b * a.dd + m, a.ya_lo, v * am);
      ss += v * v;
    }
    a.part[(long)b * (a.dd / 16) + grp] = ss;
  }
}

__global__ __launch_bounds__(256) void finish_kernel(FinishArgs a) {
  extern __shared__ float zrow[];  // the logits row when sampling (n_logits floats, at most SAMPLE_MAX_N)
  finish_unit(a, blockIdx.x, zrow);
}

void finish_prepare() {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(finish_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            SAMPLE_MAX_N * 4);
}

void launch_finish(const FinishArgs& a, hipStream_t s) {
  // room for the row only where it can be sampled (pp_set_sampling refuses wider rows)
  const size_t lds = (a.sp && a.n_logits <= SAMPLE_MAX_N) ? (size_t)a.n_logits * 4 : 0;
  hipLaunchKernelGGL(finish_kernel, dim3(a.B), dim3(256), lds, s, a);
}

// ---------------------------------------------------------------------------
// Work buffers held by the library for callers that cannot allocate device
// memory.  In host code `scratch` names a host-side stand-in, not the device
// array: kernels are only ever given the address hipGetSymbolAddress returns
// for the current device, kept per device below.
// ---------------------------------------------------------------------------

static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_u32_kernel(unsigned* p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

void launch_zero_u32(unsigned* p, long n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
}

}  // namespace pp
