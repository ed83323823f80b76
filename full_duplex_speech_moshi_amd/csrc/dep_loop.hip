// Fused depformer loop for gfx950: one persistent launch runs 8 codebook
// steps (6 layers each, then the codebook's head and greedy choice) for a few
// columns, in place of about 200 dependent kernel launches.
//
// The depformer (PersonaPlex recipe, "Architecture (Moshi RQ-Transformer,
// all native)": 1024-d, 6 layers, 16 heads, autoregressive over 16
// codebooks, reset each frame) is latency-bound at small batch: each GEMM
// reads a few MB from the last-level cache and every step depends on the one
// before.  Here the tick's GEMM arithmetic contract (8 fixed k-ranges, each
// accumulated in k-step order, hi then lo, summed in range order) is mapped
// onto the part's 8 XCDs:
//
//   * XCD x owns the depformer heads whose columns form k-range x of the
//     out-projection (heads 2x, 2x+1 at the 7B shape), and the FFN slice that
//     forms k-range x of the down-projection (352 of 2816 rows);
//   * per layer: QKV tiles of those heads (XCD x) -> attention of those heads
//     and the out-projection's range-x partial (XCD x) -> every workgroup sums
//     the 8 partials in range order and adds the residual -> gate/up tiles of
//     the FFN slice (XCD x) -> the down-projection's range-x partial (XCD x)
//     -> every workgroup sums them again;
//   * then the codebook's head (one 16-row tile per workgroup) and the greedy
//     choice, which every workgroup makes from the tiles' (max, argmax).
//
// Only the two residual updates per layer and the head cross XCDs; QKV ->
// attention and gate/up -> down stay within one XCD.  Every workgroup keeps
// the columns' residual stream in LDS and applies each update itself, so the
// sums are taken in the same order as the per-launch kernels' and a slot's
// bits do not depend on which path ran it.
//
// Exchanges go through 8-byte words (value, launch tag) written with
// device-scope stores.  Small ones (queries, keys and values, FFN slice, head
// argmax) are polled directly until every tag matches; the partial sums are
// read after their producers' done words carry the tag, with cacheable loads
// (one fetch per XCD), and any word whose tag does not match is re-read with
// device-scope loads.  Every wait is bounded: past ctl.spin_limit polls, or
// once any workgroup has raised an error, a workgroup stops and leaves the
// error in the control block for the host.  A workgroup takes its XCD from
// the hardware register and its rank within the XCD from a per-XCD arrival
// counter; the part deals the DL_GRID workgroups to its 8 XCDs in turn, so
// each XCD holds DL_GRID / 8 of them (else DL_ERR_PLACEMENT).
//
// Every pointer carries its address space (LDS or global), so that LDS
// accesses compile to ds_* instructions and do not wait for the weight loads
// issued ahead of each job.
#include "kernels.h"
#include "device.h"
#include "../../include/pp.h"

namespace pp {

namespace {

constexpr int DL_MAX_HT = DL_GRID / 2;  // head tiles per codebook (A / 16)

typedef __attribute__((address_space(1))) const bf16_t gcbf16;
typedef __attribute__((address_space(1))) const float gcfloat;
typedef __attribute__((address_space(1))) const int gcint;
typedef __attribute__((address_space(1))) const uint64_t gcu64;
typedef __attribute__((address_space(1))) const u32x4 gcu32x4;
typedef __attribute__((address_space(3))) const u32x4 lcu32x4;

__device__ __forceinline__ uint64_t xld(const gu64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void xst(gu64* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t cld(const gu32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void cst(gu32* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tw(uint32_t payload, uint32_t tag) { return ((uint64_t)tag << 32) | payload; }
__device__ __forceinline__ uint32_t wtag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float wval(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & 0xfu; }

// Dimensions and derived counts, the same in every workgroup.
struct Dims {
  int dd, dH, dhd, dF, Ld, A, dep_q;
  int ks, ksF;     // k-steps of K = dd and K = dF
  int HX;          // heads per XCD
  int T1;          // QKV tiles per XCD
  int NO;          // workgroups per XCD for the range partials (one output tile per wave)
  int FX, T3;      // FFN rows per XCD, gate/up tile pairs per XCD
  int HT;          // head tiles (A / 16)
};

struct Lds {
  lfloat* ys;      // [C][DL_MAX_DD] residual stream of each column
  lbf16* xin;      // [2][C][DL_MAX_DD] normalised GEMM input, hi plane then lo plane
  lfloat* red;     // [8 waves][2][256] partial tiles
  lfloat* fin;     // [2][16][16] finished tile(s): [rt][row][col]
  lfloat* inv;     // [DL_MAX_COLS] inverse RMS
  lfloat* part;    // [C][DL_MAX_DD / 16] sums of squares per 16 features
  lfloat* q;       // [C][DL_MAX_DD / 8] queries of this XCD's heads
  lbf16* kvs;      // [C][2][HX][16][dhd] keys and values of this XCD's heads
  lbf16* oatt;     // [2][C][DL_MAX_DD / 8] attention output (hi, lo) of this XCD's heads
  lbf16* msl;      // [2][C][DL_MAX_KW * 32] this XCD's FFN slice (hi, lo)
  lint* tok;       // [DL_MAX_COLS] chosen tokens
  lint* flag;      // [4] wait status
  lfloat* hv;      // [C][A / 16] head tiles' maxima
  lint* hi;        // [C][A / 16] head tiles' argmax
  lint* nk;        // [DL_MAX_COLS] key counts of this step's attention
  lint* ck0;       // [DL_MAX_COLS] each column's first codebook (0 agent, n_q user)
  lint* cset;      // [DL_MAX_COLS] each column's buffer set
  lint* cslot;     // [DL_MAX_COLS] each column's slot
};

// The launch's global buffers, with their address space.
struct Glb {
  const gcbf16 *wqkv, *wo, *w_in, *w_out, *heads, *emb_text, *emb_audio;
  const gcfloat *attn_norm, *mlp_norm, *out_norm;
  const gcfloat* u[2];   // input projections of z per buffer set, [B][dep_q][dd]
  gfloat* y[2];          // user half's first input per buffer set, [B][dd]
  gfloat* logits;        // [B][dep_q][A]
  const gcfloat* tamax_v;
  const gcint* tamax_i;
  const gcint* ti;
  gint* to;
  gu64 *xq, *xo, *xm, *xd, *xh, *kv;
  gu32 *kvtag, *ctl;
};

// The attention function's arguments, pointing into LDS (the fields of
// DepAttnArgs it reads), with each column's own key count.
struct DepAttnLds {
  const lfloat* q;
  int ldq;
  const lbf16* kv;
  long slot_stride, v_off;
  int n_heads, head_dim, window, B;
  const lint* n_keys_b;
};

struct Ctl {
  gu32* ctl;
  long limit;
  uint32_t tag;
  gint* err_out;   // the tick output's error word (read by the host after the tick)
};

// Raise an error for the whole launch: every wait gives up once it sees it.
__device__ __forceinline__ void raise_error(const Ctl& cx, uint32_t code) {
  cst(cx.ctl + 2, code);
  __hip_atomic_store(cx.err_out, (int)code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0 polls n (<= 64) done words at p until all carry the tag; false if
// the wait gave up (timeout or an error raised elsewhere).
__device__ __forceinline__ bool wait_done(const gu64* p, int n, const Ctl& cx, const Lds& L) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    long spins = 0;
    for (;;) {
      const bool ok = tid >= n || wtag(xld(p + tid)) == cx.tag;
      if (__all(ok)) {
        if (tid == 0) L.flag[0] = 1;
        break;
      }
      ++spins;
      if (spins > cx.limit || ((spins & 31) == 0 && cld(cx.ctl + 2) != 0)) {
        if (tid == 0) {
          L.flag[0] = 0;
          if (spins > cx.limit) raise_error(cx, DL_ERR_TIMEOUT);
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  const bool ok = L.flag[0] == 1;
  __syncthreads();
  return ok;
}

// Every thread polls its words of a tagged array until all carry the tag;
// get(i) gives the address of word i < n.  On success, put(i, word) is called
// for each.  False if the wait gave up.
template <class Get, class Put>
__device__ __forceinline__ bool poll_words(int n, Get get, Put put, const Ctl& cx) {
  long spins = 0;
  for (;;) {
    int bad = 0;
    constexpr int U = 8;
    for (int i0 = threadIdx.x; i0 < n; i0 += U * 512) {
      uint64_t w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * 512;
        w[u] = i < n ? xld(get(i)) : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * 512;
        if (i < n) {
          if (wtag(w[u]) != cx.tag) bad = 1;
          else put(i, w[u]);
        }
      }
    }
    if (!__syncthreads_or(bad)) return true;
    ++spins;
    if (spins > cx.limit || ((spins & 31) == 0 && cld(cx.ctl + 2) != 0)) {
      if (spins > cx.limit && threadIdx.x == 0) raise_error(cx, DL_ERR_TIMEOUT);
      __syncthreads();
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// RMSNorm input of the next GEMM from the residual stream ys: per column the
// sums of squares per 16 features (in feature order), then the inverse RMS
// (rms_finish's order: lane i holds partial i, i + 64, ...; then the fixed
// butterfly), and xin = bf16 pair of ys * alpha.
template <int C>
__device__ __forceinline__ void make_input(const Dims& D, const Lds& L, const gcfloat* alpha, float eps) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ng = D.dd / 16;
  const long PL = (long)C * DL_MAX_DD;
  for (int it = tid; it < C * ng; it += 512) {
    const int c = it / ng, g = it - c * ng;
    const lfloat* y = L.ys + c * DL_MAX_DD + g * 16;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = y[i];
      store_split(L.xin + c * DL_MAX_DD + g * 16 + i, PL, v * alpha[g * 16 + i]);
      ss += v * v;
    }
    L.part[c * (DL_MAX_DD / 16) + g] = ss;
  }
  __syncthreads();
  if (wave < C) {
    float s = 0.f;
    for (int i = lane; i < ng; i += 64) s += L.part[wave * (DL_MAX_DD / 16) + i];
    s = wave_sum_rows(s);
    if (lane == 0) L.inv[wave] = 1.0f / sqrtf(s / (float)D.dd + eps);
  }
  __syncthreads();
}

// Weights of one wave's share of a job, requested ahead of its inputs.
struct WBuf {
  u32x4 w[DL_MAX_KW];
};

__device__ __forceinline__ void load_w(WBuf& b, int off, const gcbf16* W, long tile, int ks, int s0, int n) {
  const int lane = threadIdx.x & 63;
  const gcbf16* p = W + (tile * ks + s0) * 512 + lane * 8;
#pragma unroll
  for (int u = 0; u < DL_MAX_KW; ++u)
    if (u >= off && u < off + n) b.w[u] = *reinterpret_cast<const gcu32x4*>(p + (long)(u - off) * 512);
}

// MFMA over k-steps [s0, s0 + n) with weights b.w[off ..] and the B operand
// from an LDS plane pair (x: [C][ldx] hi at x, lo at x + pl), columns >= C
// zero.  Accumulates in k-step order, hi then lo (the contract's order).
template <int C>
__device__ __forceinline__ f32x4 mfma_range(const WBuf& b, int off, int n, int s0, const lbf16* x, int ldx, long pl,
                                            int kbase, f32x4 acc) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const u32x4 zero = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < DL_MAX_KW; ++u) {
    if (u < n) {
      const int k = (s0 + u) * 32 - kbase;
      const lbf16* xo = x + r16 * ldx + g * 8 + k;
      const u32x4 bh = r16 < C ? *reinterpret_cast<const lcu32x4*>(xo) : zero;
      const u32x4 bl = r16 < C ? *reinterpret_cast<const lcu32x4*>(xo + pl) : zero;
      const bf16x8 w8 = __builtin_bit_cast(bf16x8, b.w[off + u]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, __builtin_bit_cast(bf16x8, bh), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w8, __builtin_bit_cast(bf16x8, bl), acc, 0, 0, 0);
    }
  }
  return acc;
}

// A whole 16-row tile (RT tiles for gate/up) over K = dd: wave w covers
// k-range w, the partial tiles are summed in wave order into L.fin.  Tile rt's
// weights sit at b.w[rt * DL_MAX_KW / 2 ..] (a fixed offset, so the buffer
// stays in registers; a range has at most DL_MAX_KW / 2 k-steps here).
template <int C, int RT>
__device__ __forceinline__ void tile_gemm(const Dims& D, const Lds& L, const WBuf& b) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = (D.ks * wave) / 8, s1 = (D.ks * (wave + 1)) / 8;
  const long PL = (long)C * DL_MAX_DD;
  f32x4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    acc[rt] = mfma_range<C>(b, rt * (DL_MAX_KW / 2), s1 - s0, s0, L.xin, DL_MAX_DD, PL, 0, (f32x4){0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j = 0; j < 4; ++j) L.red[(wave * 2 + rt) * 256 + j * 64 + lane] = acc[rt][j];
  }
  __syncthreads();
  if (tid < RT * 256) {
    const int t = tid >> 8, e = tid & 255;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) s += L.red[(w * 2 + t) * 256 + e];
    const int j = e >> 6, ln = e & 63;
    L.fin[(t * 16 + 4 * (ln >> 4) + j) * 16 + (ln & 15)] = s;
  }
  __syncthreads();
}

// Residual update from 8 range partials (words [8][C][dd] at P, done words
// [8 * NO] at P + 8 C dd): fin = ((0 + p_0) + p_1) ... + p_7, ys += fin.
template <int C>
__device__ __forceinline__ bool apply_partials(const Dims& D, const Lds& L, const gu64* P, const Ctl& cx) {
  const long n = (long)C * D.dd;
  if (!wait_done(P + 8 * n, 8 * D.NO, cx, L)) return false;
  // each thread: element e of [C][dd], all 8 partials requested at once
  long spins = 0;  // one budget for this thread's reloads
  for (long e0 = threadIdx.x; e0 < n; e0 += 512) {
    uint64_t w[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) w[x] = P[x * n + e0];  // cacheable: one fetch per XCD
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      while (wtag(w[x]) != cx.tag) {  // not yet visible through the cache: device-scope reload
        ++spins;
        if (spins > cx.limit || ((spins & 31) == 0 && cld(cx.ctl + 2) != 0)) {
          if (spins > cx.limit) raise_error(cx, DL_ERR_TIMEOUT);
          break;
        }
        w[x] = xld(P + x * n + e0);
      }
      s += wval(w[x]);
    }
    const int c = (int)(e0 / D.dd), m = (int)(e0 - (long)c * D.dd);
    L.ys[c * DL_MAX_DD + m] += s;
  }
  __syncthreads();
  return cld(cx.ctl + 2) == 0;
}

// The argmax over n (value, index) pairs read by get(i) -> (v, idx), lanes of
// one wave; the larger value wins, then the lower index (any order gives the
// same winner).
template <class Get>
__device__ __forceinline__ int wave_argmax(int n, Get get) {
  const int lane = threadIdx.x & 63;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = lane; i < n; i += 64) {
    float v;
    int ix;
    get(i, v, ix);
    if (amax_better(v, ix, bv, bi)) {
      bv = v;
      bi = ix;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float v2 = __shfl_xor(bv, off);
    const int i2 = __shfl_xor(bi, off);
    if (amax_better(v2, i2, bv, bi)) {
      bv = v2;
      bi = i2;
    }
  }
  return bi;
}

// The greedy choice of every column at step sp from the head tiles' (max,
// argmax) words: all of them polled into LDS, then one wave per column takes
// the winner (the same winner as the launches' finisher), applies a forced
// choice (agent codebooks) and, in workgroup 0, writes the tokens.
template <int C>
__device__ __forceinline__ bool choose(const Glb& G, const Dims& D, const Lds& L, const gu64* H, int sp, const Ctl& cx) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = 2 * D.HT;  // words per column
  auto addr = [&](int i) {
    const int c = i / per, rem = i - c * per;
    const int g = L.ck0[c] == 0 ? 0 : 1;
    return H + (((long)g * D.HT + (rem >> 1)) * C + c) * 2 + (rem & 1);
  };
  const bool ok = poll_words(C * per, addr,
                             [&](int i, uint64_t w) {
                               const int c = i / per, rem = i - c * per;
                               if (rem & 1) L.hi[c * DL_MAX_HT + (rem >> 1)] = (int)(uint32_t)w;
                               else L.hv[c * DL_MAX_HT + (rem >> 1)] = wval(w);
                             },
                             cx);
  if (!ok) return false;
  if (wave < C) {
    const int k0 = L.ck0[wave], slot = L.cslot[wave];
    const int kq = k0 + sp;
    const int pred = wave_argmax(D.HT, [&](int i, float& v, int& ix) {
      v = L.hv[wave * DL_MAX_HT + i];
      ix = L.hi[wave * DL_MAX_HT + i];
    });
    const int forced = (k0 == 0 && kq < 8) ? G.ti[slot * TI_STRIDE + TI_FORCE + 1 + kq] : -1;
    const int chosen = forced >= 0 ? forced : pred;
    if (lane == 0) {
      L.tok[wave] = chosen;
      if (blockIdx.x == 0) {
        gint* to = G.to + slot * TO_STRIDE;
        if (kq < 8) {
          to[TO_PRED + 1 + kq] = pred;
          to[TO_CHOSEN + 1 + kq] = chosen;
        } else {
          to[TO_USER + kq - 8] = pred;
        }
      }
    }
  }
  __syncthreads();
  return true;
}

}  // namespace

// The LDS arrays of the kernel for C columns, in the order it takes them.
static size_t dep_loop_lds_bytes(int C) {
  auto r16 = [](size_t b) { return (b + 15) / 16 * 16; };
  return r16((size_t)C * DL_MAX_DD * 4) + r16((size_t)2 * C * DL_MAX_DD * 2) + r16(8 * 2 * 256 * 4) +
         r16(2 * 16 * 16 * 4) + r16(DL_MAX_COLS * 4) + r16((size_t)C * (DL_MAX_DD / 16) * 4) +
         r16((size_t)C * (DL_MAX_DD / 8) * 4) + r16((size_t)C * 2 * (DL_MAX_DD / 8) * 16 * 2) +
         r16((size_t)2 * C * (DL_MAX_DD / 8) * 2) + r16((size_t)2 * C * DL_MAX_KW * 32 * 2) + r16(DL_MAX_COLS * 4) +
         r16(4 * 4) + 2 * r16((size_t)C * DL_MAX_HT * 4) + 4 * r16(DL_MAX_COLS * 4);
}

template <int C>
__global__ __launch_bounds__(512) void dep_loop_kernel(DepLoopArgs a) {
  extern __shared__ __attribute__((aligned(16))) char dsm[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  Glb G;
  G.wqkv = (const gcbf16*)a.wqkv;
  G.wo = (const gcbf16*)a.wo;
  G.w_in = (const gcbf16*)a.w_in;
  G.w_out = (const gcbf16*)a.w_out;
  G.heads = (const gcbf16*)a.heads;
  G.emb_text = (const gcbf16*)a.emb_text;
  G.emb_audio = (const gcbf16*)a.emb_audio;
  G.attn_norm = (const gcfloat*)a.attn_norm;
  G.mlp_norm = (const gcfloat*)a.mlp_norm;
  G.out_norm = (const gcfloat*)a.out_norm;
  G.u[0] = (const gcfloat*)a.u[0];
  G.u[1] = (const gcfloat*)a.u[1];
  G.y[0] = (gfloat*)a.y[0];
  G.y[1] = (gfloat*)a.y[1];
  G.logits = (gfloat*)a.logits;
  G.tamax_v = (const gcfloat*)a.tamax_v;
  G.tamax_i = (const gcint*)a.tamax_i;
  G.ti = (const gcint*)a.ti;
  G.to = (gint*)a.to;
  G.xq = (gu64*)a.xq;
  G.xo = (gu64*)a.xo;
  G.xm = (gu64*)a.xm;
  G.xd = (gu64*)a.xd;
  G.xh = (gu64*)a.xh;
  G.kv = (gu64*)a.kv;
  G.kvtag = (gu32*)a.kvtag;
  G.ctl = (gu32*)a.ctl;

  Lds L;
  {
    lchar* p = (lchar*)dsm;
    auto take = [&](size_t bytes) {
      lchar* q = p;
      p += (bytes + 15) / 16 * 16;
      return q;
    };
    L.ys = (lfloat*)take((size_t)C * DL_MAX_DD * 4);
    L.xin = (lbf16*)take((size_t)2 * C * DL_MAX_DD * 2);
    L.red = (lfloat*)take(8 * 2 * 256 * 4);
    L.fin = (lfloat*)take(2 * 16 * 16 * 4);
    L.inv = (lfloat*)take(DL_MAX_COLS * 4);
    L.part = (lfloat*)take((size_t)C * (DL_MAX_DD / 16) * 4);
    L.q = (lfloat*)take((size_t)C * (DL_MAX_DD / 8) * 4);
    L.kvs = (lbf16*)take((size_t)C * 2 * (DL_MAX_DD / 8) * 16 * 2);
    L.oatt = (lbf16*)take((size_t)2 * C * (DL_MAX_DD / 8) * 2);
    L.msl = (lbf16*)take((size_t)2 * C * DL_MAX_KW * 32 * 2);
    L.tok = (lint*)take(DL_MAX_COLS * 4);
    L.flag = (lint*)take(4 * 4);
    L.hv = (lfloat*)take((size_t)C * DL_MAX_HT * 4);
    L.hi = (lint*)take((size_t)C * DL_MAX_HT * 4);
    L.nk = (lint*)take(DL_MAX_COLS * 4);
    L.ck0 = (lint*)take(DL_MAX_COLS * 4);
    L.cset = (lint*)take(DL_MAX_COLS * 4);
    L.cslot = (lint*)take(DL_MAX_COLS * 4);
  }

  // This workgroup's XCD, from the hardware, and its rank among the
  // workgroups of that XCD, in order of arrival (the dispatcher deals
  // workgroups to the XCDs in turn, but a launch need not start at XCD 0).
  // The columns' descriptors go to LDS alongside, so that no later access
  // picks a kernel argument by a runtime index.
  if (tid == 0) {
    const unsigned xc = xcc_id();
    L.flag[2] = (int)xc;
    L.flag[3] = xc < DL_XCDS ? (int)__hip_atomic_fetch_add(G.ctl + 4 + xc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                             : DL_GRID;
  }
  if (tid < 64) {
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (tid == c) {
        L.ck0[c] = a.col[c].k0;
        L.cset[c] = a.col[c].set;
        L.cslot[c] = a.col[c].slot;
      }
  }
  __syncthreads();
  const int xraw = L.flag[2], r = L.flag[3];
  const int x = xraw & (DL_XCDS - 1);

  Dims D;
  D.dd = a.dd; D.dH = a.dH; D.dhd = a.dhd; D.dF = a.dF; D.Ld = a.Ld; D.A = a.A; D.dep_q = a.dep_q;
  D.ks = a.dd / 32; D.ksF = a.dF / 32;
  D.HX = a.dH / DL_XCDS;
  D.T1 = 3 * (a.dd / DL_XCDS) / 16;
  D.NO = a.dd / 16 / 8;
  D.FX = a.dF / DL_XCDS;
  D.T3 = D.FX / 16;
  D.HT = a.A / 16;

  Ctl cx;
  cx.ctl = G.ctl;
  cx.limit = a.spin_limit;
  cx.err_out = G.to + TO_ERR;
  // this launch's tag: one more than the last launch's (0, the value of
  // never-written memory, is skipped)
  cx.tag = cld(G.ctl) + 1;
  if (cx.tag == 0) cx.tag = 1;

  // every XCD must hold exactly DL_GRID / DL_XCDS of the workgroups
  bool ok = true;
  if (xraw >= DL_XCDS || r >= DL_GRID / DL_XCDS) {
    if (tid == 0) raise_error(cx, DL_ERR_PLACEMENT);
    ok = false;
  }

  // the column set's head groups: 0 agent (k0 == 0), 1 user
  bool has_group[2] = {false, false};
#pragma unroll
  for (int c = 0; c < C; ++c) has_group[a.col[c].k0 == 0 ? 0 : 1] = true;

  const int kx0 = (D.ks * x) / 8, kx1 = (D.ks * (x + 1)) / 8;     // out-projection k-range of this XCD
  const int fx0 = (D.ksF * x) / 8, fx1 = (D.ksF * (x + 1)) / 8;   // down-projection k-range of this XCD
  const int hx0 = x * D.HX;                                        // first head of this XCD
  const int j_head = blockIdx.x;                                   // head job: group j / HT, tile j % HT
  const int hg = j_head / D.HT, ht = j_head - hg * D.HT;
  const bool head_job = j_head < 2 * D.HT && has_group[hg < 2 ? hg : 0] && hg < 2;
  const int npair = a.dhd / 2;

  WBuf wb;
  // weights of one job, requested before its inputs are ready
  auto prefetch = [&](int l, int ph, int kq) {
    if (ph == 0) {  // QKV tile r of this XCD: block which = r / (T1 / 3), local tile
      const int tq = D.T1 / 3, which = r / tq, lt = r - which * tq;
      const long tile = (long)(which * a.dd + x * (a.dd / DL_XCDS)) / 16 + lt;
      const int s0 = (D.ks * wave) / 8, s1 = (D.ks * (wave + 1)) / 8;
      load_w(wb, 0, G.wqkv + (long)l * 3 * a.dd * a.dd, tile, D.ks, s0, s1 - s0);
    } else if (ph == 1) {  // out-projection tile r * 8 + wave, k-range x
      load_w(wb, 0, G.wo + (long)l * a.dd * a.dd, r * 8 + wave, D.ks, kx0, kx1 - kx0);
    } else if (ph == 2) {  // gate / up tile pair r of this XCD's FFN slice
      const long gt = (long)x * D.FX / 16 + r;
      const int s0 = (D.ks * wave) / 8, s1 = (D.ks * (wave + 1)) / 8;
      const gcbf16* W = G.w_in + (long)l * 2 * a.dF * a.dd;
      load_w(wb, 0, W, gt, D.ks, s0, s1 - s0);
      load_w(wb, DL_MAX_KW / 2, W, gt + a.dF / 16, D.ks, s0, s1 - s0);  // the up tile in the buffer's second half
    } else if (ph == 3) {  // down-projection tile r * 8 + wave, k-range x of the FFN
      load_w(wb, 0, G.w_out + (long)l * a.dd * a.dF, r * 8 + wave, D.ksF, fx0, fx1 - fx0);
    } else {  // head tile ht of the group's codebook kq
      const int s0 = (D.ks * wave) / 8, s1 = (D.ks * (wave + 1)) / 8;
      load_w(wb, 0, G.heads + (long)kq * a.A * a.dd, ht, D.ks, s0, s1 - s0);
    }
  };
  auto active = [&](int ph) {
    return ph == 0 ? r < D.T1 : ph == 1 ? r < D.NO : ph == 2 ? r < D.T3 : ph == 3 ? r < D.NO : head_job;
  };
  // the next job after (l, ph) in this workgroup's order, prefetched
  auto prefetch_next = [&](int s, int l, int ph) {
    for (;;) {
      if (++ph == 4) {
        ph = 0;
        if (++l == a.Ld) {
          if (head_job) prefetch(0, 4, (hg == 0 ? 0 : a.n_q) + s);
          return;
        }
      }
      if (active(ph)) {
        prefetch(l, ph, 0);
        return;
      }
    }
  };

  for (int s = 0; ok && s < 8; ++s) {
    // ------------------------------------------------------------- step input
    if (r < D.T1) prefetch(0, 0, 0);
    else prefetch_next(s, 0, 0);
    if (s == 0) {
      // agent columns: the text head's choice (forced where forced); user
      // columns: the input the agent half left
      if (wave < C) {
        const int slot = L.cslot[wave];
        if (L.ck0[wave] == 0) {
          const gcfloat* pv = G.tamax_v + (long)slot * a.ld_amax;
          const gcint* pi = G.tamax_i + (long)slot * a.ld_amax;
          const int pred = wave_argmax(a.n_tpart, [&](int i, float& v, int& ix) {
            v = pv[i];
            ix = pi[i];
          });
          const int forced = G.ti[slot * TI_STRIDE + TI_FORCE];
          const int chosen = forced >= 0 ? forced : pred;
          if (lane == 0) {
            L.tok[wave] = chosen;
            if (blockIdx.x == 0) {
              G.to[slot * TO_STRIDE + TO_PRED] = pred;
              G.to[slot * TO_STRIDE + TO_CHOSEN] = chosen;
            }
          }
        }
      }
      __syncthreads();
      for (int it = tid; it < C * a.dd; it += 512) {
        const int c = it / a.dd, i = it - c * a.dd;
        const int set = L.cset[c], slot = L.cslot[c];
        float v;
        if (L.ck0[c] == 0) {
          const gcfloat* u = G.u[set] + (long)slot * a.dep_q * a.dd;
          v = u[i] + bf2f(G.emb_text[(long)L.tok[c] * a.dd + i]);
        } else {
          v = G.y[set][(long)slot * a.dd + i];
        }
        L.ys[c * DL_MAX_DD + i] = v;
      }
      __syncthreads();
    } else {
      // the previous step's greedy choice from its head tiles
      ok = choose<C>(G, D, L, G.xh + (long)(s - 1) * 2 * D.HT * C * 2, s - 1, cx);
      if (!ok) break;
      for (int it = tid; it < C * a.dd; it += 512) {
        const int c = it / a.dd, i = it - c * a.dd;
        const int k = L.ck0[c] + s;  // this step's codebook
        const int set = L.cset[c], slot = L.cslot[c];
        const gcfloat* u = G.u[set] + (long)slot * a.dep_q * a.dd;
        const gcbf16* tab = G.emb_audio + ((long)(k - 1) * (a.A + 1) + L.tok[c]) * a.dd;
        L.ys[c * DL_MAX_DD + i] = u[(long)k * a.dd + i] + bf2f(tab[i]);
      }
      __syncthreads();
    }

    // ------------------------------------------------------------- layers
    for (int l = 0; ok && l < a.Ld; ++l) {
      const long sl = (long)s * a.Ld + l;
      gu64* Q = G.xq + sl * C * a.dd;
      gu64* O = G.xo + sl * (8L * C * a.dd + 64);
      gu64* M = G.xm + sl * C * a.dF;
      gu64* Dn = G.xd + sl * (8L * C * a.dd + 64);

      // A: QKV tile of this XCD's heads; q to Q, k and v to the cache
      if (r < D.T1) {
        make_input<C>(D, L, G.attn_norm + (long)l * a.dd, a.eps);
        tile_gemm<C, 1>(D, L, wb);
        const int tq = D.T1 / 3, which = r / tq, lt = r - which * tq;
        const int row0 = which * a.dd + x * (a.dd / DL_XCDS) + lt * 16;  // GEMM row of the tile
        prefetch_next(s, l, 0);
        if (tid < 8 * C) {  // pair pr of rows, column c
          const int pr = tid & 7, c = tid >> 3;
          float y0, y1;
          qkv_pair(L.fin[(2 * pr) * 16 + c], L.fin[(2 * pr + 1) * 16 + c], L.inv[c], false, 1.f, 0.f, y0, y1);
          const int rr = row0 + 2 * pr - which * a.dd;  // row within q, k or v
          if (which == 0) {
            xst(Q + (long)c * a.dd + rr, tw(__float_as_uint(y0), cx.tag));
            xst(Q + (long)c * a.dd + rr + 1, tw(__float_as_uint(y1), cx.tag));
          } else {
            const int h = rr / a.dhd, dh = rr - h * a.dhd;
            gu64* kv = G.kv + L.cset[c] * a.kv_set_words + L.cslot[c] * a.kv_slot_words +
                       ((((long)l * 2 + (which - 1)) * a.dH + h) * 16 + (L.ck0[c] + s)) * npair + dh / 2;
            const uint32_t pair = (uint32_t)f2bf(y0) | ((uint32_t)f2bf(y1) << 16);
            xst(kv, tw(pair, cx.tag));
          }
        }
      }

      // B: attention of this XCD's heads, then the out-projection's k-range x
      if (r < D.NO) {
        const int nq = D.HX * a.dhd;  // query features of this XCD
        // queries (this step) and keys / values of codebooks k0 .. k0 + s:
        // entries before k0 come from an earlier launch (tag kvtag)
        ok = poll_words(C * nq, [&](int i) { return Q + (long)(i / nq) * a.dd + x * nq + (i % nq); },
                        [&](int i, uint64_t w) { L.q[(i / nq) * (DL_MAX_DD / 8) + i % nq] = wval(w); }, cx);
        if (!ok) break;
        lu32* kvs32 = (lu32*)L.kvs;
        for (int c = 0; c < C; ++c) {
          const int k0 = L.ck0[c], set = L.cset[c], slot = L.cslot[c];
          const int nk = k0 + s + 1;
          const gu64* kvb = G.kv + set * a.kv_set_words + slot * a.kv_slot_words;
          const int nw = 2 * D.HX * nk * npair;
          const uint32_t old_tag = k0 > 0 ? G.kvtag[set * PP_MAX_BATCH + slot] : cx.tag;
          // old entries (from the agent half's launch): plain loads, checked against its tag
          for (int i = tid; i < nw; i += 512) {
            const int kvw = i / (D.HX * nk * npair), rem = i - kvw * (D.HX * nk * npair);
            const int hh = rem / (nk * npair), rem2 = rem - hh * (nk * npair);
            const int kk = rem2 / npair, p = rem2 - kk * npair;
            if (kk >= k0) continue;
            const uint64_t w = kvb[(((long)l * 2 + kvw) * a.dH + hx0 + hh) * 16 * npair + kk * npair + p];
            if (wtag(w) != old_tag) raise_error(cx, DL_ERR_TIMEOUT);
            kvs32[(((c * 2 + kvw) * D.HX + hh) * 16 + kk) * npair + p] = (uint32_t)w;
          }
          const int nn = nk - k0;
          ok = poll_words(
              2 * D.HX * nn * npair,
              [&](int i) {
                const int kvw = i / (D.HX * nn * npair), rem = i - kvw * (D.HX * nn * npair);
                const int hh = rem / (nn * npair), rem2 = rem - hh * (nn * npair);
                const int kk = k0 + rem2 / npair, p = rem2 % npair;
                return kvb + (((long)l * 2 + kvw) * a.dH + hx0 + hh) * 16 * npair + kk * npair + p;
              },
              [&](int i, uint64_t w) {
                const int kvw = i / (D.HX * nn * npair), rem = i - kvw * (D.HX * nn * npair);
                const int hh = rem / (nn * npair), rem2 = rem - hh * (nn * npair);
                const int kk = k0 + rem2 / npair, p = rem2 % npair;
                kvs32[(((c * 2 + kvw) * D.HX + hh) * 16 + kk) * npair + p] = (uint32_t)w;
              },
              cx);
          if (!ok) break;
        }
        if (!ok) break;
        if (tid < C) L.nk[tid] = L.ck0[tid] + s + 1;
        __syncthreads();
        // attention of the (column, head) pairs of this XCD, each column over
        // its own codebooks 0 .. k0 + s (the same function as the launches)
        {
          DepAttnLds da;
          da.q = L.q;
          da.ldq = DL_MAX_DD / 8;
          da.kv = L.kvs;
          da.slot_stride = 2L * D.HX * 16 * a.dhd;
          da.v_off = (long)D.HX * 16 * a.dhd;
          da.n_heads = D.HX;
          da.head_dim = a.dhd;
          da.window = 16;
          da.B = C;
          da.n_keys_b = L.nk;
          const int ppw = 128 / a.dhd;
          for (int pp0 = wave * ppw; pp0 < C * D.HX; pp0 += 8 * ppw) {
            DepAttnOut o;
            [[clang::always_inline]] o = a.dhd == 32 ? dep_attend<32>(da, pp0)
                                       : a.dhd == 64 ? dep_attend<64>(da, pp0)
                                                     : dep_attend<128>(da, pp0);
            if (o.ok) {
              const int c = o.pair / D.HX, hh = o.pair - c * D.HX;
              lbf16* op = L.oatt + c * (DL_MAX_DD / 8) + hh * a.dhd + o.feat;
              store_split(op, (long)C * (DL_MAX_DD / 8), o.o0);
              store_split(op + 1, (long)C * (DL_MAX_DD / 8), o.o1);
            }
          }
        }
        __syncthreads();
        // out-projection: tile r * 8 + wave over k-range x (this XCD's heads)
        f32x4 acc = mfma_range<C>(wb, 0, kx1 - kx0, kx0, L.oatt, DL_MAX_DD / 8, (long)C * (DL_MAX_DD / 8), kx0 * 32,
                                  (f32x4){0.f, 0.f, 0.f, 0.f});
        prefetch_next(s, l, 1);
        const int c = lane & 15, t = r * 8 + wave;
        if (c < C) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xst(O + ((long)x * C + c) * a.dd + t * 16 + 4 * (lane >> 4) + j, tw(__float_as_uint(acc[j]), cx.tag));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) xst(O + 8L * C * a.dd + x * D.NO + r, tw(0u, cx.tag));
      }

      // every workgroup: y += the out-projection (range partials in order)
      ok = apply_partials<C>(D, L, O, cx);
      if (!ok) break;

      // C: gate / up tile pair r of this XCD's FFN slice
      if (r < D.T3) {
        make_input<C>(D, L, G.mlp_norm + (long)l * a.dd, a.eps);
        tile_gemm<C, 2>(D, L, wb);
        prefetch_next(s, l, 2);
        if (tid < 16 * C) {
          const int rr = tid & 15, c = tid >> 4;
          const float gt = L.fin[(0 * 16 + rr) * 16 + c] * L.inv[c];
          const float up = L.fin[(1 * 16 + rr) * 16 + c] * L.inv[c];
          const float m = gt / (1.0f + expf(-gt)) * up;
          xst(M + (long)c * a.dF + x * D.FX + r * 16 + rr, tw(__float_as_uint(m), cx.tag));
        }
      }

      // D: down-projection tile r * 8 + wave over k-range x of the FFN
      if (r < D.NO) {
        const int nf = (fx1 - fx0) * 32;  // this XCD's FFN rows (its k-range)
        const long mpl = (long)C * DL_MAX_KW * 32;
        ok = poll_words(C * nf, [&](int i) { return M + (long)(i / nf) * a.dF + fx0 * 32 + (i % nf); },
                        [&](int i, uint64_t w) {
                          store_split(L.msl + (i / nf) * (DL_MAX_KW * 32) + (i % nf), mpl, wval(w));
                        },
                        cx);
        if (!ok) break;
        __syncthreads();
        f32x4 acc = mfma_range<C>(wb, 0, fx1 - fx0, fx0, L.msl, DL_MAX_KW * 32, mpl, fx0 * 32,
                                  (f32x4){0.f, 0.f, 0.f, 0.f});
        prefetch_next(s, l, 3);
        const int c = lane & 15, t = r * 8 + wave;
        if (c < C) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xst(Dn + ((long)x * C + c) * a.dd + t * 16 + 4 * (lane >> 4) + j, tw(__float_as_uint(acc[j]), cx.tag));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) xst(Dn + 8L * C * a.dd + x * D.NO + r, tw(0u, cx.tag));
      }

      // every workgroup: y += the down-projection
      ok = apply_partials<C>(D, L, Dn, cx);
    }
    if (!ok) break;

    // ------------------------------------------------------------- head
    if (head_job) {
      make_input<C>(D, L, G.out_norm, a.eps);
      tile_gemm<C, 1>(D, L, wb);
      gu64* H = G.xh + (long)s * 2 * D.HT * C * 2;
      if (tid < C) {
        const int c = tid;
        const int k0 = L.ck0[c], slot = L.cslot[c];
        if ((k0 == 0 ? 0 : 1) == hg) {
          const int kq = k0 + s;
          gfloat* lg = G.logits + ((long)slot * a.dep_q + kq) * a.A + ht * 16;
          float best = -INFINITY;
          int bi = 0;
          for (int rr = 0; rr < 16; ++rr) {
            const float v = L.fin[rr * 16 + c] * L.inv[c];
            lg[rr] = v;
            if (rr == 0 || v > best) {  // strict '>' in row order: the lowest index wins a tie
              best = v;
              bi = ht * 16 + rr;
            }
          }
          gu64* w = H + (((long)hg * D.HT + ht) * C + c) * 2;
          xst(w, tw(__float_as_uint(best), cx.tag));
          xst(w + 1, tw((uint32_t)bi, cx.tag));
        }
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------- last choice
  if (ok) ok = choose<C>(G, D, L, G.xh + 7L * 2 * D.HT * C * 2, 7, cx);
  if (ok) {
    // the agent half leaves the user half's first input, y = u_8 + table_8[chosen]
    if (blockIdx.x == 0) {
      for (int it = tid; it < C * a.dd; it += 512) {
        const int c = it / a.dd, i = it - c * a.dd;
        if (L.ck0[c] != 0) continue;
        const int set = L.cset[c], slot = L.cslot[c];
        const int k = a.n_q;
        const gcfloat* u = G.u[set] + (long)slot * a.dep_q * a.dd;
        const gcbf16* tab = G.emb_audio + ((long)(k - 1) * (a.A + 1) + L.tok[c]) * a.dd;
        G.y[set][(long)slot * a.dd + i] = u[(long)k * a.dd + i] + bf2f(tab[i]);
      }
      if (tid < C && L.ck0[tid] == 0) G.kvtag[L.cset[tid] * PP_MAX_BATCH + L.cslot[tid]] = cx.tag;
    }
  }

  // ------------------------------------------------------------- exit
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(G.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {  // the last workgroup out: counters back to zero, the next launch takes the next tag
      for (int i = 0; i < DL_XCDS; ++i) cst(G.ctl + 4 + i, 0u);
      cst(G.ctl + 1, 0u);
      cst(G.ctl, cx.tag);
    }
  }
}

void dep_loop_prepare() {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dep_loop_kernel<1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dep_loop_lds_bytes(1));
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dep_loop_kernel<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dep_loop_lds_bytes(2));
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dep_loop_kernel<3>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dep_loop_lds_bytes(3));
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(dep_loop_kernel<4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)dep_loop_lds_bytes(4));
}

// DL_GRID workgroups of 512 threads: every workgroup must be resident at
// once (one per compute unit), which holds while no other kernel occupies
// the part's compute units for good.
void launch_dep_loop(const DepLoopArgs& a, hipStream_t s) {
  const size_t lds = dep_loop_lds_bytes(a.ncols);
  switch (a.ncols) {
    case 1: hipLaunchKernelGGL(dep_loop_kernel<1>, dim3(DL_GRID), dim3(512), lds, s, a); break;
    case 2: hipLaunchKernelGGL(dep_loop_kernel<2>, dim3(DL_GRID), dim3(512), lds, s, a); break;
    case 3: hipLaunchKernelGGL(dep_loop_kernel<3>, dim3(DL_GRID), dim3(512), lds, s, a); break;
    default: hipLaunchKernelGGL(dep_loop_kernel<4>, dim3(DL_GRID), dim3(512), lds, s, a); break;
  }
}

}  // namespace pp
