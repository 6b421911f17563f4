// Attention column sums and top-k decode order.
//
// Attention-Based Sampler for Diffusion Language Models, Methodologie 1-2:
// tokens are decoded in descending order of the column sums of the attention
// matrix (total attention a key receives), aggregated over all heads.
//
// Pass 1 (matrix cores): a workgroup owns 256 keys of one KV head of one
// sequence, 64 per wave, held in registers as two 32-row MFMA A-operands for
// the whole pass, and streams the selected query vectors of that KV head
// through a double-buffered LDS tile of 32 vectors (one barrier per tile).
// S^T = K . Q^T puts one query per lane column, so each fragment read from
// LDS feeds two MFMAs and p = exp2(s*scale*log2e - lse*log2e) is accumulated
// into the lane's own 32 key sums with no cross-lane traffic inside the
// loop; one 32-lane reduction at the end.  When there are too few such
// workgroups to fill the chip, the query vectors are split into up to 4
// ranges, one workgroup each.
// Results go to a [split][Hkv][B][S] partial array.
// Pass 2: sums the partials of every key in a fixed order, four threads per
// key (no float atomics: reruns are bit-identical).
// Pass 3 (k > 0): per sequence, the top-k keys of [key_lo,key_hi) ordered by
// (colsum bits, ~key) 64-bit keys: descending sums, equal sums ordered by the
// lower position.  k <= 64 over a window of 1024+ keys: radix select of the
// k-th key, then a sort of the k winners; otherwise a bitonic sort of the
// whole window in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

constexpr int kColsumMaxSplit = 4;

template <int HD, int WAVES, bool FAST>
__global__ __launch_bounds__(64 * WAVES, HD == 128 || FAST ? 3 : 4) void colsum_bf16_kernel(const u16* __restrict__ q,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const u16* __restrict__ k,
                                                                 const float* __restrict__ lse,
                                                                 int B, int S, int Hq, int Hkv,
                                                                 int gsh, int max_rows, int nsq,
                                                                 int kb0, int nkb, float scale,
                                                                 float* __restrict__ partial) {
  constexpr int NT = 64 * WAVES, KEYS = 64 * WAVES;
  constexpr int QTL = 32, PITCH = HD + 8, NS = HD / 16, CPR = HD / 8;
  constexpr int CH = QTL * CPR, CPT = (CH + NT - 1) / NT;
  __shared__ __attribute__((aligned(16))) u16 sQ[2][QTL * PITCH];
  __shared__ float sL[2][QTL];
  // key blocks kb0 .. kb0 + nkb - 1 of KEYS keys (all of them, or the
  // blocks that cover a key window)
  // workgroups of one KV head are Hkv apart, so with Hkv a multiple of 8 they
  // share an XCD (and its L2) and read each query tile from there
  const int g = blockIdx.x % Hkv;
  const int sp = (blockIdx.x / Hkv) % nsq;
  const int kb = (blockIdx.x / (Hkv * nsq)) % nkb;
  const int b = blockIdx.x / (Hkv * nsq * nkb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const int G = Hq / Hkv;
  const int key0 = (kb0 + kb) * KEYS + wave * 64;
  const float c = scale * kLog2e;

  // the wave's 64 keys as two 32-row MFMA A-operands, held for the whole pass
  bf16x8 kf[2][NS];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int key_a = min(key0 + 32 * kk + lr, S - 1);
    const u16* kp = k + (((size_t)b * S + key_a) * Hkv + g) * HD + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[kk][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(kp + 16 * s));
  }
  const int row0 = min(offsets[b], max_rows);
  const int nvec = (min(offsets[b + 1], max_rows) - row0) * G;
  // this workgroup's query tiles: [v_lo, v_hi) in vectors
  const int tchunk = ((nvec + QTL - 1) / QTL + nsq - 1) / nsq;
  const int v_lo = min(nvec, sp * tchunk * QTL), v_hi = min(nvec, (sp + 1) * tchunk * QTL);
  const u16* qb = q + ((size_t)row0 * Hq + g * G) * HD;
  const float* lb = lse + (size_t)row0 * Hq + g * G;

  // Tile of 32 query vectors starting at v0 into registers, and the LSE of
  // the lane's query column (every half-wave holds the same 32 values and
  // writes them, so the store needs no branch).  Rows past the end repeat the
  // last vector; their LSE is +inf so they add exp2(-inf) = 0.  Tiles are
  // loaded in order, v_lo first.
  //
  // FAST (G a power of two dividing 32, element offsets below 2^31): vector
  // v sits (v >> gsh) * Hq + (v & (G-1)) vectors after the base, which grows
  // with v and moves by a fixed step per tile, so each thread keeps its
  // chunk's offset and clamps it to the last vector's; otherwise the row and
  // head come from a division.
  u32x4 st[CPT];
  float lraw;
  bool lvalid;
  uint32_t qo[CPT], qlim = 0, lo = 0, llim = 0;  // NT is a multiple of CPR: one column per thread
  const uint32_t dq = (uint32_t)(QTL >> gsh) * Hq * HD, dl = (uint32_t)(QTL >> gsh) * Hq;
  auto vec_off = [&](int v) { return (uint32_t)(v >> gsh) * Hq + (uint32_t)(v & (G - 1)); };
  if constexpr (FAST) {
    if (v_lo < v_hi) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) qo[j] = vec_off(v_lo + (tid + NT * j) / CPR) * HD + (tid % CPR) * 8;
      qlim = vec_off(nvec - 1) * HD + (tid % CPR) * 8;
      lo = vec_off(v_lo + lr);
      llim = vec_off(nvec - 1);
    }
  }
  auto load_tile = [&](int v0) {
    if constexpr (FAST) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        if (CH % NT == 0 || tid + NT * j < CH) {
          st[j] = *reinterpret_cast<const u32x4*>(qb + min(qo[j], qlim));
          qo[j] += dq;
        }
      }
      lraw = lb[min(lo, llim)];
      lvalid = lo <= llim;  // the offset grows with the vector index
      lo += dl;
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int cidx = tid + NT * j;
        if (CH % NT == 0 || cidx < CH) {
          const int v = min(v0 + cidx / CPR, nvec - 1), r = v / G, h = v - r * G;
          st[j] = *reinterpret_cast<const u32x4*>(qb + ((size_t)r * Hq + h) * HD + (cidx % CPR) * 8);
        }
      }
      const int v = min(v0 + lr, nvec - 1), r = v / G, h = v - r * G;
      lraw = lb[(size_t)r * Hq + h];
      lvalid = v0 + lr < nvec;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = tid + NT * j;
      if (CH % NT == 0 || cidx < CH)
        *reinterpret_cast<u32x4*>(sQ[buf] + (cidx / CPR) * PITCH + (cidx % CPR) * 8) = st[j];
    }
    sL[buf][lr] = lvalid ? lraw * kLog2e : INFINITY;
  };

  float acc[2][16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[0][i] = acc[1][i] = 0.f;
  if (v_lo < v_hi) {
    load_tile(v_lo);
    store_tile(0);
  }
  // the K fragments are complete from here on; waiting once lets the
  // loop's waits count only the tile loads
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  // One barrier per tile: tile t is read from buffer t&1 while tile t+1 is
  // loaded into registers and then written to the other buffer.  The
  // scheduling fences keep the loads at the top of the iteration and the LDS
  // writes at its end, so the loads have the whole tile's work to land.
  for (int v0 = v_lo, t = 0; v0 < v_hi; v0 += QTL, ++t) {
    load_tile(v0 + QTL);
    __builtin_amdgcn_sched_barrier(0);
    const u16* sq = sQ[t & 1] + lr * PITCH + 8 * lg;
    const float l2 = sL[t & 1][lr];
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 qf = as_bf16x8(*reinterpret_cast<const u32x4*>(sq + 16 * s));
      s0 = mfma32x32x16(kf[0][s], qf, s0);
      s1 = mfma32x32x16(kf[1][s], qf, s1);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[0][i] += __builtin_amdgcn_exp2f(fmaf(s0[i], c, -l2));
      acc[1][i] += __builtin_amdgcn_exp2f(fmaf(s1[i], c, -l2));
    }
    __builtin_amdgcn_sched_barrier(0);
    store_tile((t + 1) & 1);
    __syncthreads();
  }
  // each key's sum over the 32 query columns of its lane half
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) acc[kk][i] += __shfl_xor(acc[kk][i], o, 64);
    }
  if (lr == 0) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 32 * kk + 8 * (i >> 2) + 4 * lg + (i & 3);
        if (key < S) partial[(((size_t)sp * Hkv + g) * B + b) * S + key] = acc[kk][i];
      }
  }
}

// colsum[b][j] = sum over splits and KV heads of the partials, in a fixed
// order: wave w of a workgroup adds parts [w*P/4, (w+1)*P/4) of 64
// consecutive keys (coalesced), wave 0 then adds the four sums in order.
// Keys w0 .. w0 + W - 1 of every sequence (all S keys: w0 = 0, W = S).
__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float* __restrict__ partial,
                                                            int parts, int B, int S, int w0, int W,
                                                            float* __restrict__ colsum) {
  __shared__ float s_part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p0 = parts * wave / 4, p1 = parts * (wave + 1) / 4;
  const size_t BS = (size_t)B * S;
  const int n = B * W;
  for (int j0 = blockIdx.x * 64; j0 < n; j0 += gridDim.x * 64) {
    const int j = j0 + lane;
    const size_t at = (size_t)(j / W) * S + w0 + j % W;
    float cs = 0.f;
    if (j < n)
      for (int p = p0; p < p1; ++p) cs += partial[(size_t)p * BS + at];
    s_part[wave][lane] = cs;
    __syncthreads();
    if (wave == 0 && j < n) colsum[at] = ((s_part[0][lane] + s_part[1][lane]) + s_part[2][lane]) + s_part[3][lane];
    __syncthreads();
  }
}

// Key of window position j: colsum bits (non-negative floats order as
// unsigned integers) above ~j, so that larger keys are larger sums and, for
// equal sums, lower positions; all keys of a window are distinct.
__device__ __forceinline__ unsigned long long topk_key(float cs, int j) {
  return ((unsigned long long)__float_as_uint(cs) << 32) | (0xFFFFFFFFu - (unsigned)j);
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const unsigned lo = __shfl_xor((unsigned)v, m, 64), hi = __shfl_xor((unsigned)(v >> 32), m, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Top-k of one sequence's key window [key_lo, key_hi) (one workgroup of 1024
// threads per sequence), written in descending key order.  FUSED: the kernel
// first sums the sequence's partials itself (few of them: the separate
// reduce launch would cost more than it saves).
//   SMALL (k <= 64, window of 1024+ keys): radix select.  Each thread keeps its (at most 8) keys in
//   registers; 8-bit digits from the top narrow the candidates to the k-th
//   largest key (a 256-bin LDS histogram per digit, scanned by one wave), and
//   stop as soon as the threshold bin holds exactly the keys still missing.
//   The k keys at or above the threshold are then sorted by one wave with a
//   bitonic network on shuffles.
//   Otherwise: bitonic sort of the whole window in LDS.
template <bool FUSED, bool SMALL>
__global__ __launch_bounds__(1024) void colsum_topk_kernel(const float* __restrict__ partial,
                                                           int parts, int B, int S,
                                                           float* __restrict__ colsum, int key_lo,
                                                           int key_hi, int kk, int p2, int w0, int W,
                                                           int32_t* topk_idx, float* topk_val) {
  extern __shared__ unsigned long long skeys[];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = key_hi - key_lo;
  float* crow = colsum + (size_t)b * S;
  if constexpr (FUSED) {
    // the sums of keys w0 .. w0 + W - 1 (all S keys, or the window's blocks)
    const size_t BS = (size_t)B * S;
    for (int j = w0 + tid; j < w0 + W; j += 1024) {
      float cs = 0.f;
      for (int p = 0; p < parts; ++p) cs += partial[p * BS + (size_t)b * S + j];
      crow[j] = cs;
    }
    if (kk <= 0) return;
    __syncthreads();  // the sums are re-read below by other threads of this workgroup
  }
  if constexpr (SMALL) {
    constexpr int KPT = 8;  // keys per thread (windows of at most 8192 keys)
    __shared__ unsigned hist[256];
    __shared__ int s_bin, s_above, s_cntb, s_pos;
    __shared__ unsigned long long s_out[64];
    unsigned long long key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int w = tid + 1024 * e;
      key[e] = w < n ? topk_key(crow[key_lo + w], key_lo + w) : 0ull;
    }
    unsigned long long prefix = 0, mask = 0;
    int rem = kk;
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < KPT; ++e)
        if (tid + 1024 * e < n && (key[e] & mask) == prefix)
          atomicAdd(&hist[(unsigned)(key[e] >> shift) & 255u], 1u);
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
          if (cum < (unsigned)rem && (unsigned)rem <= cum + c[q]) {
            s_bin = 255 - 4 * lane - q;
            s_above = (int)cum;
            s_cntb = (int)c[q];
          }
          cum += c[q];
        }
      }
      __syncthreads();
      prefix |= (unsigned long long)s_bin << shift;
      mask |= 0xFFull << shift;
      rem -= s_above;
      if (s_cntb == rem) break;  // the whole threshold bin is in the top k
    }
    // exactly k keys satisfy (key & mask) >= prefix
    if (tid == 0) s_pos = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < KPT; ++e)
      if (tid + 1024 * e < n && (key[e] & mask) >= prefix) {
        const int pos = atomicAdd(&s_pos, 1);
        if (pos < 64) s_out[pos] = key[e];
      }
    __syncthreads();
    if (wave != 0) return;
    unsigned long long v = lane < kk ? s_out[lane] : 0ull;
    for (int size = 2; size <= 64; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const unsigned long long o = shfl_xor_u64(v, stride);
        const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
        v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
      }
    }
    if (lane < kk) {
      if (topk_idx) topk_idx[(size_t)b * kk + lane] = (int32_t)(0xFFFFFFFFu - (unsigned)(v & 0xFFFFFFFFull));
      if (topk_val) topk_val[(size_t)b * kk + lane] = __uint_as_float((unsigned)(v >> 32));
    }
  } else {
    for (int w = tid; w < n; w += 1024) skeys[w] = topk_key(crow[key_lo + w], key_lo + w);
    for (int w = n + tid; w < p2; w += 1024) skeys[w] = 0ull;
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
}

// Query splits, only to fill the chip: with fewer (sequence, key block, KV
// head) units than resident workgroup slots, up to 4 workgroups share a
// unit's query vectors, each keeping at least 4 tiles of the average
// sequence.  (Splitting further to even out the last round of a full chip
// was measured slower: every extra workgroup reloads its 64 KB of keys.)
static int colsum_splits(int units, int occ, int max_rows, int B, int G) {
  const int slots = device_cus() * occ;
  const long long tiles = ((long long)max_rows * G / B + 31) / 32;
  int n = 1;
  while (n < kColsumMaxSplit && units * (long long)(n + 1) <= slots && tiles >= 4LL * (n + 1)) ++n;
  return n;
}

template <int HD, int WAVES>
static int launch_colsum_pass(const void* q, const int32_t* offsets, int max_rows, const void* k,
                              const float* lse, int B, int S, int Hq, int Hkv, float scale,
                              int kb0, int nkb, float* partial, hipStream_t st) {
  const int G = Hq / Hkv;
  int gsh = 0;
  while ((1 << gsh) < G) ++gsh;
  const bool fast = (1 << gsh) == G && G <= 32 && (long long)max_rows * Hq * HD < (1LL << 31);
  const int units = B * nkb * Hkv;
  // resident workgroups per CU: one wave per SIMD each, at most 168
  // registers per lane (128 for the generic d = 64 body)
  const int nsq = colsum_splits(units, HD == 128 || fast ? 3 : 4, max_rows, B, G);
  auto kern = fast ? colsum_bf16_kernel<HD, WAVES, true> : colsum_bf16_kernel<HD, WAVES, false>;
  hipLaunchKernelGGL(kern, dim3(units * nsq), dim3(64 * WAVES), 0, st, static_cast<const u16*>(q),
                     offsets, static_cast<const u16*>(k), lse, B, S, Hq, Hkv, gsh, max_rows, nsq,
                     kb0, nkb, scale, partial);
  return nsq;
}

size_t colsum_workspace_bytes(int B, int S, int Hkv) {
  return (size_t)kColsumMaxSplit * Hkv * B * S * sizeof(float);
}

hipError_t launch_colsum(const void* q, const int32_t* offsets, int max_rows, const void* k,
                         const float* lse, int B, int S, int Hq, int Hkv, int hd, float scale,
                         float* partial, float* colsum, int key_lo, int key_hi, int kk,
                         int32_t* topk_idx, float* topk_val, int window, hipStream_t st) {
  // all key blocks, or (window) only the 256-key blocks that cover [key_lo, key_hi)
  constexpr int KEYS = 256;
  if (window && key_hi <= key_lo) return hipSuccess;  // an empty window: nothing to compute
  const int kb0 = window ? key_lo / KEYS : 0;
  const int kb1 = window ? (key_hi + KEYS - 1) / KEYS : (S + KEYS - 1) / KEYS;
  if (kb1 <= kb0) return hipSuccess;  // empty window
  const int w0 = kb0 * KEYS, W = min(S, kb1 * KEYS) - w0;
  const int nsq = hd == 64 ? launch_colsum_pass<64, 4>(q, offsets, max_rows, k, lse, B, S, Hq, Hkv,
                                                        scale, kb0, kb1 - kb0, partial, st)
                           : launch_colsum_pass<128, 4>(q, offsets, max_rows, k, lse, B, S, Hq,
                                                         Hkv, scale, kb0, kb1 - kb0, partial, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // when a sequence has few partials over the keys summed (all S, or the
  // window's covering blocks), one kernel sums them and picks its top-k: at
  // most 16 partial loads per thread of its 1024, where a separate reduce
  // launch would cost more than it saves
  const int parts = nsq * Hkv;
  const bool fused = kk > 0 && (long long)parts * W <= 16384;
  if (!fused) {
    const int n = B * W;
    hipLaunchKernelGGL(colsum_reduce_kernel, dim3(min((n + 63) / 64, 2048)), dim3(256), 0, st,
                       partial, parts, B, S, w0, W, colsum);
    if (kk <= 0) return hipGetLastError();
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int p2 = 1;
  while (p2 < key_hi - key_lo) p2 <<= 1;
  if (p2 < 2) p2 = 2;
  // radix select for k <= 64 over windows of 1024+ keys (a short window
  // sorts faster than the select's histogram passes)
  const bool small = kk <= 64 && key_hi - key_lo >= 1024;
  auto topk = small ? (fused ? colsum_topk_kernel<true, true> : colsum_topk_kernel<false, true>)
                    : (fused ? colsum_topk_kernel<true, false> : colsum_topk_kernel<false, false>);
  hipLaunchKernelGGL(topk, dim3(B), dim3(1024), small ? 0 : (size_t)p2 * sizeof(unsigned long long), st,
                     partial, parts, B, S, colsum, key_lo, key_hi, kk, p2, w0, W, topk_idx, topk_val);
  return hipGetLastError();
}

}  // namespace dlm
