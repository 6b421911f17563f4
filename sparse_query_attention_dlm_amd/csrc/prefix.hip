// Longest-stable-prefix commit.
//
// Beyond Scattered Acceptance (Longest Stable Prefixes), Methodologie: the
// scheduler commits, in one step, the longest contiguous run of stable
// positions at the start of the remaining active region, and commits at
// least one position when none is stable.  Stability here: the per-step
// argmax stayed the same over the last W steps (SlowFast Sampling,
// Metodologia, convergence principle) and the max probability is at least
// the confidence threshold.
//
// One workgroup per sequence: every thread pushes the latest argmax of its
// positions into the W-deep ring, tests stability against the ring's older
// entries, and the first unstable position at or after the frontier is found
// with an LDS atomicMin.  Integer work only; the one float comparison uses the
// float32 max-prob given.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

// WT > 0: the ring depth W == WT, known at compile time, so each thread's
// loads (argmax, max-prob and the W - 1 older ring entries of up to PP
// positions) all issue before any of them is used: one memory round trip per
// PP * 256 positions instead of several per position.  WT = 0: any W.
template <int WT>
__global__ __launch_bounds__(256) void stable_prefix_kernel(const int32_t* __restrict__ argmax,
                                                            const float* __restrict__ maxprob,
                                                            int S, int gen_lo, int gen_hi,
                                                            int32_t* __restrict__ ring, int W,
                                                            int step, float thr, int min_commit,
                                                            int32_t* __restrict__ committed) {
  constexpr int PP = 4;  // positions per thread per batch of loads
  __shared__ int s_first;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int S_gen = gen_hi - gen_lo;
  const int L = committed[b];
  if (tid == 0) s_first = S_gen;
  __syncthreads();
  const int slot = step % W;
  if constexpr (WT > 0) {
    for (int i0 = tid; i0 < S_gen; i0 += PP * 256) {
      int a[PP], old[PP][WT];
      float mp[PP];
#pragma unroll
      for (int k = 0; k < PP; ++k) {
        const int i = i0 + k * 256;
        const bool in = i < S_gen;
        const size_t pos = (size_t)b * S + gen_lo + (in ? i : 0);
        a[k] = in ? argmax[pos] : -1;
        mp[k] = in ? maxprob[pos] : 0.f;
        const int32_t* rr = ring + ((size_t)b * S_gen + (in ? i : 0)) * WT;
#pragma unroll
        for (int w = 0; w < WT; ++w) old[k][w] = in && w != slot ? rr[w] : 0;
      }
#pragma unroll
      for (int k = 0; k < PP; ++k) {
        const int i = i0 + k * 256;
        if (i >= S_gen) break;
        ring[((size_t)b * S_gen + i) * WT + slot] = a[k];
        bool stable = (a[k] != -1) && (mp[k] >= thr);
#pragma unroll
        for (int w = 0; w < WT; ++w) stable = stable && (w == slot || old[k][w] == a[k]);
        if (i >= L && !stable) atomicMin(&s_first, i);
      }
    }
  } else {
    for (int i = tid; i < S_gen; i += 256) {
      const size_t pos = (size_t)b * S + gen_lo + i;
      const int a = argmax[pos];
      int32_t* rr = ring + ((size_t)b * S_gen + i) * W;
      rr[slot] = a;
      bool stable = (a != -1) && (maxprob[pos] >= thr);
      for (int w = 0; w < W; ++w) stable = stable && (rr[w] == a);
      if (i >= L && !stable) atomicMin(&s_first, i);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int e = s_first;
    if (min_commit && e == L && L < S_gen) e = L + 1;
    committed[b] = e;
  }
}

// Adaptive-threshold commit (Longest Stable Prefixes, Methodologie: stability
// by the logit margin; the threshold is searched so that the stable block
// covers a fraction range of the active length; at least one token).  With A
// active positions, lo = max(1, ceil(frac_lo A)) and hi = max(lo, floor(frac_hi
// A)): tau is the largest threshold under which the first lo active positions
// are stable (their minimum margin), and the block is the run of leading
// positions with margin >= tau, cut at hi.  An optional absolute floor (the
// fallback's "stable enough"): the threshold used is max(tau, floor), and when
// the first active margin is already below it one position is committed.  One
// workgroup per sequence: a block min for tau, then an LDS atomicMin for the
// first position below the threshold.
__global__ __launch_bounds__(256) void lsp_adaptive_kernel(const float* __restrict__ margin, int S,
                                                           int gen_lo, int gen_hi, float frac_lo,
                                                           float frac_hi, float floor_m,
                                                           int32_t* __restrict__ committed,
                                                           float* __restrict__ tau) {
  __shared__ float s_min[4];
  __shared__ int s_first;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = committed[b];
  const int A = (gen_hi - gen_lo) - c;
  if (A <= 0) {
    if (tid == 0 && tau) tau[b] = __builtin_nanf("");
    return;
  }
  // integer bounds in double, from the float32 fractions given
  const int lo = max(1, (int)ceil((double)frac_lo * A));
  const int hi = max(lo, (int)floor((double)frac_hi * A));
  const float* act = margin + (size_t)b * S + gen_lo + c;
  float m = INFINITY;
  for (int i = tid; i < lo; i += 256) m = fminf(m, act[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fminf(m, __shfl_xor(m, o, 64));
  if (lane == 0) s_min[wave] = m;
  if (tid == 0) s_first = A;
  __syncthreads();
  const float t = fmaxf(fminf(fminf(s_min[0], s_min[1]), fminf(s_min[2], s_min[3])), floor_m);
  for (int i = tid; i < A; i += 256)
    if (act[i] < t) atomicMin(&s_first, i);
  __syncthreads();
  if (tid == 0) {
    committed[b] = c + max(1, min(s_first, hi));
    if (tau) tau[b] = t;
  }
}

hipError_t launch_lsp_adaptive(const float* margin, int B, int S, int gen_lo, int gen_hi,
                               float frac_lo, float frac_hi, float margin_floor, int32_t* committed,
                               float* tau, hipStream_t st) {
  hipLaunchKernelGGL(lsp_adaptive_kernel, dim3(B), dim3(256), 0, st, margin, S, gen_lo, gen_hi,
                     frac_lo, frac_hi, margin_floor, committed, tau);
  return hipGetLastError();
}

hipError_t launch_stable_prefix(const int32_t* argmax, const float* maxprob, int B, int S,
                                int gen_lo, int gen_hi, int32_t* ring, int W, int step, float thr,
                                int min_commit, int32_t* committed, hipStream_t st) {
  switch (W) {
    case 1:
      hipLaunchKernelGGL(stable_prefix_kernel<1>, dim3(B), dim3(256), 0, st, argmax, maxprob, S, gen_lo,
                         gen_hi, ring, W, step, thr, min_commit, committed);
      break;
    case 2:
      hipLaunchKernelGGL(stable_prefix_kernel<2>, dim3(B), dim3(256), 0, st, argmax, maxprob, S, gen_lo,
                         gen_hi, ring, W, step, thr, min_commit, committed);
      break;
    case 3:
      hipLaunchKernelGGL(stable_prefix_kernel<3>, dim3(B), dim3(256), 0, st, argmax, maxprob, S, gen_lo,
                         gen_hi, ring, W, step, thr, min_commit, committed);
      break;
    case 4:
      hipLaunchKernelGGL(stable_prefix_kernel<4>, dim3(B), dim3(256), 0, st, argmax, maxprob, S, gen_lo,
                         gen_hi, ring, W, step, thr, min_commit, committed);
      break;
    default:
      hipLaunchKernelGGL(stable_prefix_kernel<0>, dim3(B), dim3(256), 0, st, argmax, maxprob, S, gen_lo,
                         gen_hi, ring, W, step, thr, min_commit, committed);
  }
  return hipGetLastError();
}

}  // namespace dlm
