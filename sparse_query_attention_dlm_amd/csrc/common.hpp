// Device-side helpers shared by the gfx950 kernels of libdlm.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlm {

typedef unsigned short u16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(u16 v) { return __uint_as_float(uint32_t(v) << 16); }

// float -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// unpack 8 bf16 held in a 16-byte vector
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 32x32x16 bf16 MFMA: a = 8 bf16 of row (lane%32), k = 8*(lane/32)..+7;
// b = 8 bf16 of column (lane%32), same k; c/d: lane holds column lane%32,
// register i holds row 8*(i/4) + 4*(lane/32) + (i%4).
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3):
// loads past the end return zeros without touching memory.  Callers keep
// `bytes` below 2^31 wherever they rely on that, put the per-lane part of an
// offset in the VGPR (voff) and a wave-uniform part in soff, and mark a lane
// out of range with voff >= 2^31: then voff alone and voff + soff (< 2^32)
// are both past the end, whichever of the two the range check uses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Reductions over the lane pair (l, l^32) with v_permlane32_swap.  With both
// operands equal, lanes < 32 receive (own, partner) and lanes >= 32 receive
// (partner, own): in both the low-half value comes first, so the two lanes
// compute bit-identical results.
__device__ __forceinline__ float pair_max(float v) {
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  unsigned u = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row -> batch lookup: the batch row b with offsets[b] <= r < offsets[b+1].
__device__ __forceinline__ int batch_of(const int32_t* offsets, int B, int r) {
  int lo = 0, hi = B;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// Merge two softmax partials (max m, sum of exp(z - m), argmax a) of disjoint
// logit sets.  Ties in the max keep the lower index.  s*exp(m-M) + s2*exp(m2-M)
// is commutative, so merge(x, y) and merge(y, x) give identical bits.
// Second-largest value of the union of two sets given each set's largest (m,
// c1) and second-largest (t2, c2) values: the smaller of the two maxima or
// either set's second value, whichever is larger.  Call before the maxima are
// merged.
__device__ __forceinline__ float merge_second(float m, float t2, float c1, float c2) {
  return fmaxf(fminf(m, c1), fmaxf(t2, c2));
}

__device__ __forceinline__ void merge_part(float& m, float& s, int& a, float m2, float s2, int a2) {
  if (m2 == -INFINITY) return;  // empty partner (lane without tiles)
  if (m == -INFINITY) {
    m = m2; s = s2; a = a2;
    return;
  }
  const float M = fmaxf(m, m2);
  const int A = (m > m2) ? a : ((m2 > m) ? a2 : min(a, a2));
  s = s * exp2f((m - M) * kLog2e) + s2 * exp2f((m2 - M) * kLog2e);
  m = M;
  a = A;
}

// merge_part for partials that also carry a sum w of exp(z - m) times a
// per-logit weight (rescaled like s)
__device__ __forceinline__ void merge_part_w(float& m, float& s, float& w, int& a, float m2, float s2,
                                             float w2, int a2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2; s = s2; w = w2; a = a2;
    return;
  }
  const float M = fmaxf(m, m2);
  const int A = (m > m2) ? a : ((m2 > m) ? a2 : min(a, a2));
  const float f1 = exp2f((m - M) * kLog2e), f2 = exp2f((m2 - M) * kLog2e);
  s = s * f1 + s2 * f2;
  w = w * f1 + w2 * f2;
  m = M;
  a = A;
}

}  // namespace dlm
