// Device helpers shared by the tick's kernel files (gfx950, 64-lane waves):
// bf16 conversions, fixed-order cross-lane reductions, and the pieces of
// per-slot arithmetic that every path computing the same value goes through
// (so that a slot's bits do not depend on which kernel produced them).
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace pp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (bf16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Store v as a bf16 pair (hi, lo) with hi = bf16(v), lo = bf16(v - hi):
// hi + lo carries 16 significant bits, so a GEMM fed both planes sees its
// input to within 2^-17 relative while the weights stay plain bf16.
__device__ __forceinline__ void store_split(bf16_t* p, long lo, float v) {
  const bf16_t h = f2bf(v);
  p[0] = h;
  p[lo] = f2bf(v - bf2f(h));
}

__device__ __forceinline__ u32x4 ld16(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Pointers with their address space spelled out (LDS: 3, global: 1), for
// code whose pointers travel through structures: accesses through them
// compile to ds_* and global_* instructions, not flat ones (which would make
// every LDS read wait for all global loads in flight).
typedef __attribute__((address_space(3))) float lfloat;
typedef __attribute__((address_space(3))) bf16_t lbf16;
typedef __attribute__((address_space(3))) int lint;
typedef __attribute__((address_space(3))) uint32_t lu32;
typedef __attribute__((address_space(3))) char lchar;
typedef __attribute__((address_space(1))) float gfloat;
typedef __attribute__((address_space(1))) bf16_t gbf16;
typedef __attribute__((address_space(1))) int gint;
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint64_t gu64;
typedef __attribute__((address_space(1))) u32x4 gu32x4;

__device__ __forceinline__ const uint32_t* as_u32(const bf16_t* p) { return reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ const lu32* as_u32(const lbf16* p) { return reinterpret_cast<const lu32*>(p); }
__device__ __forceinline__ void store_split(lbf16* p, long lo, float v) {
  const bf16_t h = f2bf(v);
  p[0] = h;
  p[lo] = f2bf(v - bf2f(h));
}
// Weight loads.  Weights read once per tick (temporal stack, heads, input
// projections: far larger than the caches) carry the non-temporal hint; the
// depformer layers, re-read at every codebook step, are loaded normally so
// that they stay in the last-level cache.
template <bool NTL>
__device__ __forceinline__ u32x4 ldw16(const bf16_t* p) {
  if constexpr (NTL) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return ld16(p);
}
__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(v[i]);
    f[2 * i + 1] = bf_hi(v[i]);
  }
}

// Fixed butterfly over the 64 lanes of a wave (same order on every call).
// Reductions over aligned groups of G lanes (G a power of two up to 64), the
// same result in every lane of the group and a fixed order: within 16-lane
// rows by DPP (swap neighbours, swap pairs, mirror within half-rows, mirror
// within rows), then across rows by exchanges.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if (G >= 2) v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
  if (G >= 4) v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
  if (G >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if (G >= 16) v += dpp_f<0x140>(v); // row_mirror
  if (G >= 32) v += __shfl_xor(v, 16);
  if (G >= 64) v += __shfl_xor(v, 32);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if (G >= 2) v = fmaxf(v, dpp_f<0xb1>(v));
  if (G >= 4) v = fmaxf(v, dpp_f<0x4e>(v));
  if (G >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if (G >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  if (G >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if (G >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum_rows(float v) { return group_sum<64>(v); }

// The QKV epilogue's arithmetic for rows (2i, 2i+1) of one slot: the ordered
// sums s0, s1 scaled by the slot's inverse RMS, then, for q and k, rotated by
// the pair's (cos, sin) at the slot's position (interleaved RoPE).  Every
// path that finishes q, k or v goes through this function.
__device__ __forceinline__ void qkv_pair(float s0, float s1, float inv, bool rot, float cs, float sn, float& y0,
                                         float& y1) {
  y0 = s0 * inv;
  y1 = s1 * inv;
  if (rot) {
    const float r0 = y0 * cs - y1 * sn;
    const float r1 = y0 * sn + y1 * cs;
    y0 = r0;
    y1 = r1;
  }
}

// ---------------------------------------------------------------------------
// Depformer attention (one codebook step, keys of steps 0..n-1 of this
// frame, scale 1/sqrt(head_dim), softmax with max subtraction, keys in step
// order).  One wave takes 128/head_dim consecutive (slot, head) pairs,
// head_dim/2 lanes per pair and two features per lane; the dot products are
// summed over the pair's lanes with a fixed butterfly.  The same function
// serves the standalone kernel and the out-projection that computes its own
// input, so a slot's result does not depend on which of them ran.
// ---------------------------------------------------------------------------

struct DepAttnOut {
  float o0, o1;  // features feat, feat + 1 of pair `pair`
  int pair, feat;
  bool ok;
};

// Argument types with a key count per slot (member n_keys_b) in place of
// DepAttnArgs' one count for every slot.
template <class T, class = void>
struct per_slot_keys : std::false_type {};
template <class T>
struct per_slot_keys<T, std::void_t<decltype(T::n_keys_b)>> : std::true_type {};

// Args: DepAttnArgs (global memory), or a structure with the same fields
// pointing into LDS; the arithmetic is the same either way.
template <int DH, class Args>
__device__ DepAttnOut dep_attend(const Args& d, const int pair0) {
  constexpr int LP = DH / 2;  // lanes per pair
  const int lane = threadIdx.x & 63;
  const int pair = pair0 + lane / LP, f = 2 * (lane % LP);
  const bool ok = pair < d.B * d.n_heads;
  const int b = ok ? pair / d.n_heads : 0, h = ok ? pair - b * d.n_heads : 0;
  const auto qp = d.q + (long)b * d.ldq + h * DH + f;
  const float q0 = ok ? qp[0] : 0.f, q1 = ok ? qp[1] : 0.f;
  const auto kb = d.kv + (long)b * d.slot_stride + (long)h * d.window * DH + f;
  const auto kw = as_u32(kb);
  const auto vw = as_u32(kb + d.v_off);
  int n;
  if constexpr (per_slot_keys<Args>::value) n = d.n_keys_b[b];
  else n = d.n_keys;
  uint32_t kk[DEP_MAX_KEYS], vv[DEP_MAX_KEYS];
#pragma unroll
  for (int p = 0; p < DEP_MAX_KEYS; ++p) {
    kk[p] = (ok && p < n) ? kw[p * LP] : 0u;
    vv[p] = (ok && p < n) ? vw[p * LP] : 0u;
  }
  // all keys' partial dots first, then their butterflies side by side
  float sc[DEP_MAX_KEYS];
#pragma unroll
  for (int p = 0; p < DEP_MAX_KEYS; ++p) sc[p] = __builtin_fmaf(q1, bf_hi(kk[p]), q0 * bf_lo(kk[p]));
#pragma unroll
  for (int p = 0; p < DEP_MAX_KEYS; ++p) sc[p] = group_sum<LP>(sc[p]);
  const float scale = 1.0f / sqrtf((float)DH);
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < DEP_MAX_KEYS; ++p) {
    sc[p] *= scale;
    if (p < n) mx = fmaxf(mx, sc[p]);
  }
  float l = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int p = 0; p < DEP_MAX_KEYS; ++p) {
    if (p < n) {
      const float e = expf(sc[p] - mx);
      l += e;
      o0 = __builtin_fmaf(e, bf_lo(vv[p]), o0);
      o1 = __builtin_fmaf(e, bf_hi(vv[p]), o1);
    }
  }
  return DepAttnOut{o0 / l, o1 / l, pair, f, ok};
}

// (value, index) pairs: larger value wins, then the lower index; index
// 0x7fffffff marks an empty pair.
__device__ __forceinline__ bool amax_better(float v2, int i2, float v, int i) {
  return i2 != 0x7fffffff && (i == 0x7fffffff || v2 > v || (v2 == v && i2 < i));
}

}  // namespace pp
