// Attention column sums and top-k decode order.
//
// Attention-Based Sampler for Diffusion Language Models, Methodologie 1-2:
// tokens are decoded in descending order of the column sums of the attention
// matrix (total attention a key receives), aggregated over all heads.
//
// Pass 1 (matrix cores): a workgroup owns 128 keys of one KV head of one
// sequence (each wave 32 keys, its K rows held in registers as the MFMA
// A-operand for the whole pass) and streams every selected query vector of
// that KV head through LDS in tiles of 32.  S^T = K . Q^T puts one query per
// lane column, so p = exp2(s*scale*log2e - lse*log2e) is accumulated into the
// lane's own 16 key sums with no cross-lane traffic inside the loop; one
// 32-lane reduction at the end.  Results go to a [Hkv][B][S] partial array.
// Pass 2: per sequence, sums the Hkv partials in a fixed order (no float
// atomics: reruns are bit-identical) and selects the top-k keys of
// [key_lo,key_hi) with a bitonic sort of (colsum bits, ~key) 64-bit keys in
// LDS: descending sums, equal sums ordered by the lower position.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

template <int HD>
__global__ __launch_bounds__(256, 2) void colsum_bf16_kernel(const u16* __restrict__ q,
                                                             const int32_t* __restrict__ offsets,
                                                             const u16* __restrict__ k,
                                                             const float* __restrict__ lse, int B,
                                                             int S, int Hq, int Hkv, int max_rows,
                                                             float scale,
                                                             float* __restrict__ partial) {
  constexpr int QTL = 32, PITCH = HD + 8, NS = HD / 16, CPR = HD / 8;
  __shared__ __attribute__((aligned(16))) u16 sQ[QTL * PITCH];
  __shared__ float sL[QTL];
  const int nkb = (S + 127) / 128;
  const int g = blockIdx.x % Hkv;
  const int kb = (blockIdx.x / Hkv) % nkb;
  const int b = blockIdx.x / (Hkv * nkb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const int G = Hq / Hkv;
  const int key_a = min(kb * 128 + wave * 32 + lr, S - 1);  // A-operand row (clamped for loads)
  const float c = scale * kLog2e;

  bf16x8 kf[NS];
  {
    const u16* kp = k + (((size_t)b * S + key_a) * Hkv + g) * HD + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + 16 * s));
  }
  const int row0 = min(offsets[b], max_rows);
  const int nvec = (min(offsets[b + 1], max_rows) - row0) * G;
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int v0 = 0; v0 < nvec; v0 += QTL) {
    // stage 32 query vectors (2 x 16-byte chunks per thread for HD = 128)
    u32x4 st[QTL * CPR / 256 > 0 ? QTL * CPR / 256 : 1];
#pragma unroll
    for (int j = 0; j < QTL * CPR / 256; ++j) {
      const int cidx = tid + 256 * j, r = cidx / CPR, ch = cidx % CPR;
      const int v = min(v0 + r, nvec - 1);
      const int row = row0 + v / G, h = g * G + v % G;
      st[j] = *reinterpret_cast<const u32x4*>(q + ((size_t)row * Hq + h) * HD + ch * 8);
    }
    float lv = 0.f;
    if (tid < QTL) {
      const int v = v0 + tid;
      if (v < nvec) {
        const int row = row0 + v / G, h = g * G + v % G;
        lv = lse[(size_t)row * Hq + h] * kLog2e;
      } else {
        lv = INFINITY;  // padding query: contributes exp2(-inf) = 0
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < QTL * CPR / 256; ++j) {
      const int cidx = tid + 256 * j, r = cidx / CPR, ch = cidx % CPR;
      *reinterpret_cast<u32x4*>(sQ + r * PITCH + ch * 8) = st[j];
    }
    if (tid < QTL) sL[tid] = lv;
    __syncthreads();
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 qf = as_bf16x8(*reinterpret_cast<const u32x4*>(sQ + lr * PITCH + 16 * s + 8 * lg));
      sacc = mfma32x32x16(kf[s], qf, sacc);
    }
    const float l2 = sL[lr];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -l2));
  }
  // reduce each key's sum over the 32 query columns of its lane half
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) acc[i] += __shfl_xor(acc[i], o, 64);
  }
  if (lr == 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * 128 + wave * 32 + 8 * (i >> 2) + 4 * lg + (i & 3);
      if (key < S) partial[((size_t)g * B + b) * S + key] = acc[i];
    }
  }
}

__global__ __launch_bounds__(1024) void colsum_reduce_topk_kernel(const float* __restrict__ partial,
                                                                  int Hkv, int B, int S,
                                                                  float* __restrict__ colsum,
                                                                  int key_lo, int key_hi, int kk,
                                                                  int p2, int32_t* topk_idx,
                                                                  float* topk_val) {
  extern __shared__ unsigned long long skeys[];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int j = tid; j < S; j += 1024) {
    float cs = 0.f;
    for (int g = 0; g < Hkv; ++g) cs += partial[((size_t)g * B + b) * S + j];
    colsum[(size_t)b * S + j] = cs;
    if (kk > 0 && j >= key_lo && j < key_hi)
      skeys[j - key_lo] = ((unsigned long long)__float_as_uint(cs) << 32) | (0xFFFFFFFFu - (unsigned)j);
  }
  if (kk <= 0) return;
  for (int j = (key_hi - key_lo) + tid; j < p2; j += 1024) skeys[j] = 0ull;
  __syncthreads();
  for (int size = 2; size <= p2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (p2 >> 1); t += 1024) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const unsigned long long x = skeys[i], y = skeys[j];
        if ((x < y) == desc) {
          skeys[i] = y;
          skeys[j] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int t = tid; t < kk; t += 1024) {
    const unsigned long long u = skeys[t];
    if (topk_idx) topk_idx[(size_t)b * kk + t] = (int32_t)(0xFFFFFFFFu - (unsigned)(u & 0xFFFFFFFFull));
    if (topk_val) topk_val[(size_t)b * kk + t] = __uint_as_float((unsigned)(u >> 32));
  }
}

hipError_t launch_colsum(const void* q, const int32_t* offsets, int max_rows, const void* k,
                         const float* lse, int B, int S, int Hq, int Hkv, int hd, float scale,
                         float* partial, float* colsum, int key_lo, int key_hi, int kk,
                         int32_t* topk_idx, float* topk_val, hipStream_t st) {
  const int nkb = (S + 127) / 128;
  const int grid = B * nkb * Hkv;
  if (hd == 64)
    hipLaunchKernelGGL(colsum_bf16_kernel<64>, dim3(grid), dim3(256), 0, st,
                       static_cast<const u16*>(q), offsets, static_cast<const u16*>(k), lse, B, S,
                       Hq, Hkv, max_rows, scale, partial);
  else
    hipLaunchKernelGGL(colsum_bf16_kernel<128>, dim3(grid), dim3(256), 0, st,
                       static_cast<const u16*>(q), offsets, static_cast<const u16*>(k), lse, B, S,
                       Hq, Hkv, max_rows, scale, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int p2 = 1;
  while (p2 < key_hi - key_lo) p2 <<= 1;
  if (p2 < 2) p2 = 2;
  const size_t shmem = kk > 0 ? (size_t)p2 * sizeof(unsigned long long) : 0;
  hipLaunchKernelGGL(colsum_reduce_topk_kernel, dim3(B), dim3(1024), shmem, st, partial, Hkv, B, S,
                     colsum, key_lo, key_hi, kk, p2, topk_idx, topk_val);
  return hipGetLastError();
}

}  // namespace dlm
