// Stability scoring and compaction of the positions to recompute.
//
// DyLLM (saliency-based token selection), Methodologie 1: a token's temporal
// cosine similarity against the previous step decides whether it is salient;
// SlowFast Sampling, Metodologia (certainty principle): the model's max
// softmax probability is the confidence signal; SureLock, Methodik: unlocked
// positions are the ones recomputed.  Selected iff score < threshold.
//
// Layout: one wave64 per scored row, 16-byte vector loads (a lane's whole
// batch of loads is issued before any arithmetic), float32 accumulation, wave
// reductions.  The compaction (flag -> prefix sum -> ascending index list,
// counts, offsets) is a second launch after the scores, one workgroup per
// batch row.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

constexpr int kCompactNT = 256;

// Block-wide sum of one int per thread (256 threads).
__device__ __forceinline__ int block_sum(int v, int* s_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if (lane == 0) s_wave[wave] = v;
  __syncthreads();
  return s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
}

// One chunk of NT*E consecutive positions [c0, c0 + NT*E) of a row's window:
// thread t holds positions c0 + E*t .. +E-1 in `v` (thr past the window), and
// writes its selected positions in ascending order after the block-wide
// exclusive count, from out0 = the chunk's first output slot.  Returns the
// chunk's selected count.
template <int E>
__device__ __forceinline__ int compact_chunk(const float (&v)[E], float thr, int lo, int c0, int out0,
                                             int32_t* idx, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned mask = 0;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool f = v[e] < thr;
    mask |= unsigned(f) << e;
    cnt += f;
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int wpre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int x = s_wave[w];
    wpre += (w < wave) ? x : 0;
    tot += x;
  }
  int out = out0 + wpre + incl - cnt;
  const int p0 = c0 + tid * E;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((mask >> e) & 1u) idx[out++] = lo + p0 + e;
  __syncthreads();  // s_wave is rewritten by the next chunk
  return tot;
}

// Loads one chunk of a row's window for compact_chunk (thr past the window).
template <int E>
__device__ __forceinline__ void load_chunk(const float* row, int W, float thr, int c0, float (&v)[E]) {
  const int p0 = c0 + (int)threadIdx.x * E;
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = p0 + e < W ? row[p0 + e] : thr;
}

// Block-wide (256 threads) compaction of [lo,hi) of batch rows [b0, b1),
// whose first index goes to idx[base].
__device__ void compact_rows(const float* scores, int B, int S, int lo, int hi, float thr, int b0,
                             int b1, int base, int32_t* idx, int32_t* counts, int32_t* offsets) {
  constexpr int NT = kCompactNT, E = 8;
  __shared__ int s_wave[4];
  const int tid = threadIdx.x;
  const int W = hi - lo;
  for (int b = b0; b < b1; ++b) {
    const float* row = scores + (size_t)b * S + lo;
    int rowcount = 0;
    for (int c0 = 0; c0 < W; c0 += NT * E) {
      float v[E];
      load_chunk<E>(row, W, thr, c0, v);
      rowcount += compact_chunk<E>(v, thr, lo, c0, base + rowcount, idx, s_wave);
    }
    if (tid == 0) {
      counts[b] = rowcount;
      offsets[b] = base;
    }
    base += rowcount;
  }
  if (tid == 0 && b1 == B) offsets[B] = base;
}

template <int DT>
__global__ __launch_bounds__(256) void cosine_select_kernel(const void* __restrict__ cur,
                                                            const void* __restrict__ prev, int B,
                                                            int S, int D, int lo, int hi, float thr,
                                                            float* scores) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int W = hi - lo;
  const int r = blockIdx.x * 4 + wave;
  if (r < B * W) {
    const int b = r / W, i = lo + r % W;
    const size_t off = ((size_t)b * S + i) * D;
    float dot = 0.f, nc = 0.f, np = 0.f;
    // 16-byte chunks: 8 bf16 or 4 f32.  Each lane issues a batch of 8 chunk
    // loads from each tensor before touching any of them, so a wave keeps
    // 16 KB in flight (one whole 4096-wide bf16 row pair).
    constexpr int EPC = DT == 1 ? 8 : 4;
    constexpr int BATCH = 8;
    const u32x4* pc = reinterpret_cast<const u32x4*>(static_cast<const char*>(cur) + off * (DT == 1 ? 2 : 4));
    const u32x4* pp = reinterpret_cast<const u32x4*>(static_cast<const char*>(prev) + off * (DT == 1 ? 2 : 4));
    const int nch = D / EPC;
    for (int c0 = 0; c0 < nch; c0 += 64 * BATCH) {
      u32x4 va[BATCH], vb[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int c = c0 + u * 64 + lane;
        if (c < nch) {
          va[u] = __builtin_nontemporal_load(pc + c);
          vb[u] = __builtin_nontemporal_load(pp + c);
        } else {
          va[u] = u32x4{0, 0, 0, 0};
          vb[u] = u32x4{0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        float fa[EPC], fb[EPC];
        if (DT == 1) {
          unpack8(va[u], fa);
          unpack8(vb[u], fb);
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            fa[e] = __uint_as_float(va[u][e]);
            fb[e] = __uint_as_float(vb[u][e]);
          }
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          dot = fmaf(fa[e], fb[e], dot);
          nc = fmaf(fa[e], fa[e], nc);
          np = fmaf(fb[e], fb[e], np);
        }
      }
    }
    dot = wave_sum(dot);
    nc = wave_sum(nc);
    np = wave_sum(np);
    if (lane == 0) {
      const float den = sqrtf(nc) * sqrtf(np);
      scores[(size_t)b * S + i] = den > 0.f ? dot / den : 0.f;
    }
  }
}

__global__ __launch_bounds__(256) void given_select_kernel(const float* __restrict__ scores, int B,
                                                           int S, int lo, int hi, float thr,
                                                           int32_t* idx, int32_t* counts,
                                                           int32_t* offsets) {
  if (gridDim.x == 1) {
    compact_rows(scores, B, S, lo, hi, thr, 0, B, 0, idx, counts, offsets);
    return;
  }
  // One workgroup per batch row: the rows before it are counted again here
  // (a few KB of scores each), which gives this row's first output slot
  // without any ordering between workgroups.  The row's own first chunk and
  // eight earlier rows at a time are loaded before anything is counted, so a
  // workgroup waits out one or two memory round trips, not one per row.
  constexpr int NT = kCompactNT, E = 8, RB = 8;
  __shared__ int s_sum[4], s_cw[4];  // block_sum's and the chunks' (no reuse between them)
  const int b = blockIdx.x, W = hi - lo, tid = threadIdx.x;
  const float* own = scores + (size_t)b * S + lo;
  float v0[E];
  load_chunk<E>(own, W, thr, 0, v0);
  int before = 0;
  for (int p0 = tid; p0 < W; p0 += E * NT) {
    for (int bb0 = 0; bb0 < b; bb0 += RB) {
      float v[RB][E];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int u = 0; u < E; ++u) {
          const int p = p0 + u * NT;
          v[r][u] = (bb0 + r < b && p < W) ? scores[(size_t)(bb0 + r) * S + lo + p] : thr;
        }
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int u = 0; u < E; ++u) before += v[r][u] < thr;
    }
  }
  const int base = block_sum(before, s_sum);
  int rowcount = compact_chunk<E>(v0, thr, lo, 0, base, idx, s_cw);
  for (int c0 = NT * E; c0 < W; c0 += NT * E) {
    float v[E];
    load_chunk<E>(own, W, thr, c0, v);
    rowcount += compact_chunk<E>(v, thr, lo, c0, base + rowcount, idx, s_cw);
  }
  if (tid == 0) {
    counts[b] = rowcount;
    offsets[b] = base;
    if (b == B - 1) offsets[B] = base + rowcount;
  }
}

// Merge of per-vocabulary-tile partials (max logit, sum exp(z - max), argmax,
// second-largest logit) into the score and argmax per evaluated row, then the
// compaction.  The score is the max-prob (SlowFast, Metodologia, certainty
// principle) or the logit margin, top-1 minus top-2 (LSP, Methodologie,
// stability diagnosis).
__global__ __launch_bounds__(256) void lmhead_combine_kernel(
    const float4* __restrict__ part, int ntile, const int32_t* __restrict__ eval_idx,
    const int32_t* __restrict__ eval_offsets, int max_eval, int B, int S, int margin, float* scores,
    int32_t* argmax) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  const int n_eval = min(eval_offsets[B], max_eval);
  if (r < n_eval) {
    float m = -INFINITY, s = 0.f, t2 = -INFINITY;
    int a = 0x7fffffff;
    for (int t = lane; t < ntile; t += 64) {
      const float4 p = part[(size_t)r * ntile + t];
      t2 = merge_second(m, t2, p.x, p.w);
      merge_part(m, s, a, p.x, p.y, __float_as_int(p.z));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64), q2 = __shfl_xor(t2, o, 64);
      const int a2 = __shfl_xor(a, o, 64);
      t2 = merge_second(m, t2, m2, q2);
      merge_part(m, s, a, m2, s2, a2);
    }
    if (lane == 0) {
      const int b = batch_of(eval_offsets, B, r);
      const size_t pos = (size_t)b * S + eval_idx[r];
      scores[pos] = margin ? m - t2 : 1.0f / s;
      argmax[pos] = a;
    }
  }
}

// SureLock (Stopping Computation for Converged Tokens), Methodik, Kriterium
// zum Sperren: the local KL divergence KL(p_t || p_{t-1}) of each evaluated
// position, from the LM head's per-tile partials of both steps (never the
// logits): with lse = m + log s per step and w / s = sum_v p_t(v) (z_t(v) -
// z_{t-1}(v)), KL = w / s_t - lse_t + lse_{t-1}.  Also the max probability
// 1 / s_t and the argmax of this step.  One wave per evaluated position.
__global__ __launch_bounds__(256) void kl_combine_kernel(
    const float4* __restrict__ part, int ntile, const int32_t* __restrict__ eval_idx,
    const int32_t* __restrict__ eval_offsets, int max_eval, int B, int S, float* kl, float* maxprob,
    int32_t* argmax) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  const int n_eval = min(eval_offsets[B], max_eval);
  if (r >= n_eval) return;
  float m = -INFINITY, s = 0.f, w = 0.f, mq = -INFINITY, sq = 0.f, wq = 0.f;
  int a = 0x7fffffff, aq = 0;
  for (int t = lane; t < ntile; t += 64) {
    const float4 p = part[2 * ((size_t)r * ntile + t)], q = part[2 * ((size_t)r * ntile + t) + 1];
    merge_part_w(m, s, w, a, p.x, p.y, p.w, __float_as_int(p.z));
    merge_part_w(mq, sq, wq, aq, q.x, q.y, 0.f, 0);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    merge_part_w(m, s, w, a, __shfl_xor(m, o, 64), __shfl_xor(s, o, 64), __shfl_xor(w, o, 64),
                 __shfl_xor(a, o, 64));
    merge_part_w(mq, sq, wq, aq, __shfl_xor(mq, o, 64), __shfl_xor(sq, o, 64), 0.f, 0);
  }
  if (lane == 0) {
    const int b = batch_of(eval_offsets, B, r);
    const size_t pos = (size_t)b * S + eval_idx[r];
    kl[pos] = w / s - (m + __logf(s)) + (mq + __logf(sq));
    maxprob[pos] = 1.0f / s;
    argmax[pos] = a;
  }
}

// The lock decision per sequence (one workgroup of 1024 threads): an
// evaluated position locks when KL < eps and, with the confidence gate on,
// its max probability is at least the k-th largest of its sequence's
// evaluated positions, k = max(1, ceil(gate_q * n)) (the nearest-rank
// percentile of the uncertainty 1 - max p, compared on max p itself).  The
// k-th largest is found by a radix select over the float bits (positive
// floats order as unsigned integers), 8 bits at a time from the top.
// Locked entries are set to 1; nothing else is written.
__global__ __launch_bounds__(1024) void kl_lock_kernel(const float* __restrict__ kl,
                                                       const float* __restrict__ maxprob,
                                                       const int32_t* __restrict__ eval_idx,
                                                       const int32_t* __restrict__ eval_offsets,
                                                       int max_eval, int S, float eps, float gate_q,
                                                       float* locked) {
  __shared__ unsigned hist[256];
  __shared__ unsigned s_bin, s_above;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = min(eval_offsets[b], max_eval), r1 = min(eval_offsets[b + 1], max_eval);
  const int n = r1 - r0;
  if (n <= 0) return;
  const float* klb = kl + (size_t)b * S;
  const float* mpb = maxprob + (size_t)b * S;
  unsigned thr = 0u;  // bits of the gate's max-prob threshold (0: no gate)
  if (gate_q > 0.f) {
    int k = (int)ceil((double)gate_q * (double)n);
    k = max(1, min(k, n));
    unsigned prefix = 0u, mask = 0u;
    unsigned rem = (unsigned)k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int r = r0 + tid; r < r1; r += 1024) {
        const unsigned u = __float_as_uint(mpb[eval_idx[r]]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 255-4l .. 252-4l, highest first
        unsigned c[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c[q] = hist[255 - 4 * lane - q];
          tot += c[q];
        }
        unsigned incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const unsigned t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        unsigned cum = incl - tot;  // candidates in the bins above this lane's
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum < rem && rem <= cum + c[q]) {
            s_bin = 255u - 4u * lane - q;
            s_above = cum;
          }
          cum += c[q];
        }
      }
      __syncthreads();
      prefix |= s_bin << shift;
      mask |= 0xFFu << shift;
      rem -= s_above;
      __syncthreads();  // s_bin / s_above are rewritten by the next digit
    }
    thr = prefix;  // the exact bits of the k-th largest max-prob
  }
  for (int r = r0 + tid; r < r1; r += 1024) {
    const int i = eval_idx[r];
    if (klb[i] < eps && __float_as_uint(mpb[i]) >= thr) locked[(size_t)b * S + i] = 1.0f;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_given_select(const float* scores, int B, int S, int lo, int hi, float thr,
                               int32_t* idx, int32_t* counts, int32_t* offsets, hipStream_t st) {
  // one workgroup per batch row while the repeated counting of the earlier
  // rows stays small (B*B*(hi-lo)/2 scores), else one workgroup for all rows
  const bool wide = B > 1 && (long long)B * B * (hi - lo) <= (32LL << 20);
  hipLaunchKernelGGL(given_select_kernel, dim3(wide ? B : 1), dim3(kCompactNT), 0, st, scores, B, S,
                     lo, hi, thr, idx, counts, offsets);
  return hipGetLastError();
}

// Scoring runs over many workgroups; the compaction is a second, single-
// workgroup launch.  (Ordering the two inside one kernel would need agent-scope
// fences, which on this multi-XCD part write back and invalidate whole L2s.)
hipError_t launch_cosine_select(int dtype, const void* cur, const void* prev, int B, int S, int D,
                                int lo, int hi, float thr, float* scores, int32_t* idx,
                                int32_t* counts, int32_t* offsets, hipStream_t st) {
  const int rows = B * (hi - lo);
  if (rows > 0) {
    const int grid = (rows + 3) / 4;
    if (dtype == 1)
      hipLaunchKernelGGL(cosine_select_kernel<1>, dim3(grid), dim3(256), 0, st, cur, prev, B, S, D,
                         lo, hi, thr, scores);
    else
      hipLaunchKernelGGL(cosine_select_kernel<0>, dim3(grid), dim3(256), 0, st, cur, prev, B, S, D,
                         lo, hi, thr, scores);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_given_select(scores, B, S, lo, hi, thr, idx, counts, offsets, st);
}

hipError_t launch_lmhead_combine(const float4* part, int ntile, const int32_t* eval_idx,
                                 const int32_t* eval_offsets, int max_eval, int B, int S, int lo,
                                 int hi, float thr, int margin, float* scores, int32_t* argmax,
                                 int32_t* idx, int32_t* counts, int32_t* offsets, hipStream_t st) {
  if (max_eval > 0) {
    const int grid = (max_eval + 3) / 4;
    hipLaunchKernelGGL(lmhead_combine_kernel, dim3(grid), dim3(256), 0, st, part, ntile, eval_idx,
                       eval_offsets, max_eval, B, S, margin, scores, argmax);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_given_select(scores, B, S, lo, hi, thr, idx, counts, offsets, st);
}

}  // namespace dlm

namespace dlm {

hipError_t launch_kl_lock(const float4* part, int ntile, const int32_t* eval_idx,
                          const int32_t* eval_offsets, int max_eval, int B, int S, float eps,
                          float gate_q, float* kl, float* maxprob, int32_t* argmax, float* locked,
                          hipStream_t st) {
  if (max_eval <= 0) return hipSuccess;
  hipLaunchKernelGGL(kl_combine_kernel, dim3((max_eval + 3) / 4), dim3(256), 0, st, part, ntile, eval_idx,
                     eval_offsets, max_eval, B, S, kl, maxprob, argmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kl_lock_kernel, dim3(B), dim3(1024), 0, st, kl, maxprob, eval_idx, eval_offsets,
                     max_eval, S, eps, gate_q, locked);
  return hipGetLastError();
}

}  // namespace dlm
