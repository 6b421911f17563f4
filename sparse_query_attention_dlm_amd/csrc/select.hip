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

// Block-wide (256 threads) compaction of [lo,hi) of batch rows [b0, b1),
// whose first index goes to idx[base].
__device__ void compact_rows(const float* scores, int B, int S, int lo, int hi, float thr, int b0,
                             int b1, int base, int32_t* idx, int32_t* counts, int32_t* offsets) {
  constexpr int NT = kCompactNT, E = 8;
  __shared__ int s_wave[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = hi - lo;
  for (int b = b0; b < b1; ++b) {
    const float* row = scores + (size_t)b * S + lo;
    int rowcount = 0;
    for (int c0 = 0; c0 < W; c0 += NT * E) {
      const int p0 = c0 + tid * E;
      unsigned mask = 0;
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int p = p0 + e;
        const bool f = (p < W) && (row[p] < thr);
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
        const int v = s_wave[w];
        wpre += (w < wave) ? v : 0;
        tot += v;
      }
      int out = base + rowcount + wpre + incl - cnt;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((mask >> e) & 1u) idx[out++] = lo + p0 + e;
      rowcount += tot;
      __syncthreads();
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
  // one workgroup per batch row: the rows before it are counted again here
  // (a few KB of scores each), which gives this row's first output slot
  // without any ordering between workgroups
  __shared__ int s_sum[4];
  const int b = blockIdx.x, W = hi - lo;
  int before = 0;
  for (int bb = 0; bb < b; ++bb) {
    const float* row = scores + (size_t)bb * S + lo;
    for (int p0 = threadIdx.x; p0 < W; p0 += 8 * kCompactNT) {
      float v[8];  // eight loads in flight before any compare
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int p = p0 + u * kCompactNT;
        v[u] = p < W ? row[p] : thr;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) before += v[u] < thr;
    }
  }
  const int base = block_sum(before, s_sum);
  compact_rows(scores, B, S, lo, hi, thr, b, b + 1, base, idx, counts, offsets);
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
