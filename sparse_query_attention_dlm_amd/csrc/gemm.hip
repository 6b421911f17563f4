// Gathered-row GEMM on the gfx950 matrix cores, with fused epilogues.
//
// SureLock (Stopping Computation for Converged Tokens), Methodik,
// Kernprinzipien: only the active positions compute Q/K/V, locked positions
// keep their cached K/V.  DyLLM, Methodologie 1: recomputed tokens overwrite
// their cached activations.  SlowFast Sampling, Metodologia (certainty
// principle): the max softmax probability of the LM head is the confidence.
//
// Computes D^T[n][m] = sum_k W[n][k] * A[row(m)][k] with W output-major, so
// both MFMA operands are K-contiguous and come straight from LDS rows:
//   A-operand = a 32-row block of W (output features), B-operand = 32 gathered
//   token rows.  The gather happens on load (row offsets resolved once per
//   tile from idx/offsets), so no compacted copy of the hidden states is made.
// Epilogues:
//   EPI_QKV    - Q rows written compact, K/V rows scattered into the caches
//                (8-byte bf16x4 stores of 4 consecutive features)
//   EPI_ROWS   - rows scattered into an output cache (W_o projection)
//   EPI_LMHEAD - per (token, 256-column vocabulary tile): max logit, sum of
//                exp(z - max) and the lowest argmax; logits never stored.
//   EPI_LMMARGIN - the same plus the second-largest logit (the logit margin)
// Tiles: TP (features) x TT (tokens) x 64 (k), 4 waves, 32x32x16 bf16 MFMA,
// double-buffered LDS with 16-byte row padding, a branch-free register ring
// of PF k-steps, operands fetched with buffer loads (one VGPR offset per
// chunk; padding token rows point past the end of the buffer and read zeros
// without touching memory).  The large tilings run on a resident grid (one
// workgroup per slot that fits on the GPU at once) that loops over the output
// tiles, so the tiles in flight on an XCD advance together and share their
// weight and row slices in its L2.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

// Store four consecutive features n..n+3 of token m (cache row drow) as bf16.
template <int EPI>
__device__ __forceinline__ void epi_store4(const GemmArgs& g, int m, int drow, int n, float v0, float v1,
                                           float v2, float v3) {
  if constexpr (EPI == EPI_SWIGLU) {
    // n..n+3 = (gate, up) of features n/2 and n/2 + 1 (n is a multiple of 4):
    // h = silu(gate) * up, silu(z) = z / (1 + e^-z), two bf16 to the compact row
    const float h0 = v0 / (1.f + __expf(-v0)) * v1;
    const float h1 = v2 / (1.f + __expf(-v2)) * v3;
    *reinterpret_cast<uint32_t*>(static_cast<u16*>(g.out) + (size_t)m * g.ld_out + (n >> 1)) = pack_bf16x2(h0, h1);
    return;
  }
  u32x2 pk;
  pk[0] = pack_bf16x2(v0, v1);
  pk[1] = pack_bf16x2(v2, v3);
  u16* dst;
  if constexpr (EPI == EPI_QKV) {
    if (n < g.nq)
      dst = static_cast<u16*>(g.q_out) + (size_t)m * g.nq + n;
    else if (n < g.nq + g.nk)
      dst = static_cast<u16*>(g.k_cache) + (size_t)drow * g.nk + (n - g.nq);
    else
      dst = static_cast<u16*>(g.v_cache) + (size_t)drow * g.nk + (n - g.nq - g.nk);
  } else {
    dst = static_cast<u16*>(g.out) + (size_t)drow * g.ld_out + n;
  }
  *reinterpret_cast<u32x2*>(dst) = pk;
}

// One MFMA block's 16 accumulators, read into VGPRs where the LM-head
// epilogues use them.  Left to itself the compiler copies all 256 accumulator
// registers of the 256 x 256 tile out of the AGPRs together when the k-loop
// ends, which pushes the loop's other live values to scratch (200-400 bytes
// per lane).  The compiler does not count MFMA hazards for inline asm, so the
// reads start with the 12 wait states it inserts itself between a 32x32x16
// MFMA and a VALU read of its result; the AGPR inputs keep the producing
// MFMA ahead of them.
__device__ __forceinline__ void read_acc(const f32x16& c, float (&v)[16]) {
  __asm__ volatile(
      "s_nop 11\n\t"
      "v_accvgpr_read_b32 %0, %8\n\tv_accvgpr_read_b32 %1, %9\n\t"
      "v_accvgpr_read_b32 %2, %10\n\tv_accvgpr_read_b32 %3, %11\n\t"
      "v_accvgpr_read_b32 %4, %12\n\tv_accvgpr_read_b32 %5, %13\n\t"
      "v_accvgpr_read_b32 %6, %14\n\tv_accvgpr_read_b32 %7, %15"
      : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5]), "=v"(v[6]), "=v"(v[7])
      : "a"(c[0]), "a"(c[1]), "a"(c[2]), "a"(c[3]), "a"(c[4]), "a"(c[5]), "a"(c[6]), "a"(c[7]));
  __asm__ volatile(
      "s_nop 11\n\t"
      "v_accvgpr_read_b32 %0, %8\n\tv_accvgpr_read_b32 %1, %9\n\t"
      "v_accvgpr_read_b32 %2, %10\n\tv_accvgpr_read_b32 %3, %11\n\t"
      "v_accvgpr_read_b32 %4, %12\n\tv_accvgpr_read_b32 %5, %13\n\t"
      "v_accvgpr_read_b32 %6, %14\n\tv_accvgpr_read_b32 %7, %15"
      : "=v"(v[8]), "=v"(v[9]), "=v"(v[10]), "=v"(v[11]), "=v"(v[12]), "=v"(v[13]), "=v"(v[14]), "=v"(v[15])
      : "a"(c[8]), "a"(c[9]), "a"(c[10]), "a"(c[11]), "a"(c[12]), "a"(c[13]), "a"(c[14]), "a"(c[15]));
}

// Epilogues on the accumulated tile.  Register i of acc[a][b] in lane l holds
// feature n0 + wp*WTP + 32a + 8(i/4) + 4(l/32) + i%4 of token m0 + wt*WTT + 32b + l%32.
template <int TP, int TT, int WP, int WT, int EPI, int TPV = TP>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g,
                                              f32x16 (&acc)[TP / WP / 32][TT / WT / 32], int m0,
                                              int n0, int nt, const int* s_drow) {
  constexpr int WTP = TP / WP, WTT = TT / WT, FP = WTP / 32, FT = WTT / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / WT, wt = wave % WT;
  const int lr = lane & 31, lg = lane >> 5;
  if constexpr (EPI == EPI_QKV || EPI == EPI_ROWS || EPI == EPI_SWIGLU) {
#pragma unroll
    for (int b = 0; b < FT; ++b) {
      const int ml = wt * WTT + b * 32 + lr;
      const int drow = s_drow[ml];
      if (drow < 0) continue;
#pragma unroll
      for (int a = 0; a < FP; ++a) {
        // the SwiGLU epilogue's exponentials and divisions spill the 256 x 256
        // tile's live values when the accumulators are all copied out at once
        float av[16];
        if constexpr (EPI == EPI_SWIGLU && FP * FT == 16) {
          read_acc(acc[a][b], av);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) av[i] = acc[a][b][i];
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int nl = wp * WTP + a * 32 + 8 * q4 + 4 * lg;  // feature within the tile
          if (TPV < TP && nl >= TPV) continue;                 // zero-filled padding rows
          epi_store4<EPI>(g, m0 + ml, drow, n0 + nl, av[4 * q4], av[4 * q4 + 1], av[4 * q4 + 2],
                          av[4 * q4 + 3]);
        }
      }
    }
  } else if constexpr (EPI == EPI_LMKL) {
    // Token columns c and c + 16 of a 32-column block hold one position's
    // logits at this step and at the previous step (same features, same
    // registers), so a lane reads its partner's 16 logits with one swizzle.
    // Per lane: this step's (max, sum e, sum e (z - z_prev), argmax) or the
    // previous step's (max, sum e) over its features (the lanes of the
    // previous step compute the cross sum too; it is not used).
    __shared__ float s_km[WP][TT], s_ks[WP][TT], s_kw[WP][TT];
    __shared__ int s_ka[WP][TT];
#pragma unroll
    for (int b = 0; b < FT; ++b) {
      const int ml = wt * WTT + b * 32 + lr;
      float m = -INFINITY, s = 0.f, w = 0.f;
      int am = 0x7fffffff;
#pragma unroll
      for (int a = 0; a < FP; ++a) {
        float av[16];
        read_acc(acc[a][b], av);
        float cm = av[0];
        int ca = n0 + wp * WTP + a * 32 + 4 * lg;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          const int n = n0 + wp * WTP + a * 32 + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (av[i] > cm) {  // rows grow with i, so ties keep the lower index
            cm = av[i];
            ca = n;
          }
        }
        const float cm2 = cm * kLog2e;
        float cs = 0.f, cw = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = av[i];
          const float e = __builtin_amdgcn_exp2f(fmaf(v, kLog2e, -cm2));
          cs += e;
          cw = fmaf(e, v - __shfl_xor(v, 16, 64), cw);
        }
        merge_part_w(m, s, w, am, cm, cs, cw, ca);
      }
      merge_part_w(m, s, w, am, __shfl_xor(m, 32, 64), __shfl_xor(s, 32, 64), __shfl_xor(w, 32, 64),
                   __shfl_xor(am, 32, 64));
      if (lg == 0) {
        s_km[wp][ml] = m;
        s_ks[wp][ml] = s;
        s_kw[wp][ml] = w;
        s_ka[wp][ml] = am;
      }
    }
    __syncthreads();
    for (int pp = tid; pp < TT / 2; pp += 256) {
      const int cc = (pp >> 4) * 32 + (pp & 15);  // the position's column at this step; cc + 16 the previous
      if (s_drow[cc] < 0) continue;
      float m = s_km[0][cc], s = s_ks[0][cc], w = s_kw[0][cc];
      int am = s_ka[0][cc];
      float mq = s_km[0][cc + 16], sq = s_ks[0][cc + 16], wq = 0.f;
      int aq = 0;
#pragma unroll
      for (int v = 1; v < WP; ++v) {
        merge_part_w(m, s, w, am, s_km[v][cc], s_ks[v][cc], s_kw[v][cc], s_ka[v][cc]);
        merge_part_w(mq, sq, wq, aq, s_km[v][cc + 16], s_ks[v][cc + 16], 0.f, 0);
      }
      float4* dst = g.lm_part + 2 * ((size_t)(m0 / 2 + pp) * g.ntile + nt);
      dst[0] = make_float4(m, s, __int_as_float(am), w);
      dst[1] = make_float4(mq, sq, 0.f, 0.f);
    }
  } else {
    __shared__ float s_pm[WP][TT], s_ps[WP][TT], s_p2[EPI == EPI_LMMARGIN ? WP : 1][TT];
    __shared__ int s_pa[WP][TT];
#pragma unroll
    for (int b = 0; b < FT; ++b) {
      const int ml = wt * WTT + b * 32 + lr;
      // running (max, sum exp(z - max), argmax) merged 16 logits at a time,
      // and for the margin the second-largest logit (the max itself when
      // attained twice); the confidence epilogue leaves it out
      constexpr bool TOP2 = EPI == EPI_LMMARGIN;
      float m = -INFINITY, s = 0.f, t2 = -INFINITY;
      int am = 0x7fffffff;
#pragma unroll
      for (int a = 0; a < FP; ++a) {
        float av[16];
        read_acc(acc[a][b], av);
        float cm = av[0], c2 = -INFINITY;
        int ca = n0 + wp * WTP + a * 32 + 4 * lg;
#pragma unroll
        for (int i = 1; i < 16; ++i) {
          const int n = n0 + wp * WTP + a * 32 + 8 * (i >> 2) + 4 * lg + (i & 3);
          const float v = av[i];
          if (v > cm) {  // rows grow with i, so ties keep the lower index
            if constexpr (TOP2) c2 = cm;
            cm = v;
            ca = n;
          } else if constexpr (TOP2) {
            c2 = fmaxf(c2, v);
          }
        }
        const float cm2 = cm * kLog2e;
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) cs += __builtin_amdgcn_exp2f(fmaf(av[i], kLog2e, -cm2));
        if constexpr (TOP2) t2 = merge_second(m, t2, cm, c2);
        merge_part(m, s, am, cm, cs, ca);
      }
      const float m2 = __shfl_xor(m, 32, 64), s2 = __shfl_xor(s, 32, 64);
      const int a2 = __shfl_xor(am, 32, 64);
      if constexpr (TOP2) t2 = merge_second(m, t2, m2, __shfl_xor(t2, 32, 64));
      merge_part(m, s, am, m2, s2, a2);
      if (lg == 0) {
        s_pm[wp][ml] = m;
        s_ps[wp][ml] = s;
        s_pa[wp][ml] = am;
        if constexpr (TOP2) s_p2[wp][ml] = t2;
      }
    }
    __syncthreads();
    for (int t = tid; t < TT; t += 256) {
      if (s_drow[t] < 0) continue;
      constexpr bool TOP2 = EPI == EPI_LMMARGIN;
      float m = s_pm[0][t], s = s_ps[0][t], t2 = TOP2 ? s_p2[0][t] : 0.f;
      int am = s_pa[0][t];
#pragma unroll
      for (int w = 1; w < WP; ++w) {
        if constexpr (TOP2) t2 = merge_second(m, t2, s_pm[w][t], s_p2[w][t]);
        merge_part(m, s, am, s_pm[w][t], s_ps[w][t], s_pa[w][t]);
      }
      g.lm_part[(size_t)(m0 + t) * g.ntile + nt] = make_float4(m, s, __int_as_float(am), t2);
    }
  }
}

// Split-K plan, computed on the device from the real row count (and, for
// the reduce pass, recomputed from the same inputs).
//   Fewer than SB output tiles: K is split over spare workgroups of the grid:
//     ks is a power of two (<= 8) that divides the k-steps into whole
//     prefetch rings (at least two rings per split), doubled while all
//     units * ks items still fit in one round of the G-workgroup grid (in
//     ST items when the grid is not known yet) and within kSplitCap (the
//     workspace).  A split that needs more rounds does the same number of
//     item-rounds of work and adds the partials' round trip: measured on
//     the lock loop's Q/K/V GEMM with 240 tiles of 256 x 256 on 256
//     workgroups, 4 splits (960 items) took 227 us.
//   SB tiles or more: whole rounds of the G-workgroup resident grid run
//     unsplit; only the rem = units % G tiles of the last, partial round are
//     split, ks >= 4 ways with rem * ks <= G, so that the last round nearly
//     fills the grid instead of leaving G - rem workgroups idle for a whole
//     tile.
// Tiles [0, whole) run unsplit, tiles [whole, units) are split ks ways.
constexpr int kSplitCap = 1024;

// The weight-streaming case (<= kSkinnyRows rows): 64-feature tiles, no
// split-K.  Measured on this GPU (n = 102, N = 12288, K = 4096): splitting K
// over 192-feature tiles (one workgroup per CU, 1/4 of the rows each) ran the
// product in 31.8 us against 35 us, but its partial tiles cost a 9.8 us
// reduction pass; with all CUs streaming from HBM each gets only ~20 GB/s, so
// the partials cost about what the saved row reads gain.
constexpr int kSkinnyRows = 128;
// Reduction pass: workgroups per split tile are chosen so that about
// kReduceTarget of them share the partials.
constexpr int kReduceTarget = 256;

struct GemmSplit {
  int units;  // output tiles
  int ks;     // K splits of each split tile
  int whole;  // tiles [0, whole) unsplit
  __host__ __device__ int items() const { return whole + (units - whole) * ks; }
  __host__ __device__ int splits_of(int unit) const { return unit >= whole ? ks : 1; }
};
__host__ __device__ inline GemmSplit gemm_split(int units, int nk, int pf, int SB, int ST, int G) {
  GemmSplit s{units, 1, units};
  if (units <= 0 || SB <= 0) return s;
  auto can_split = [&](int k2) { return k2 <= 8 && nk % k2 == 0 && (nk / k2) % pf == 0 && nk / k2 >= 2 * pf; };
  if (units < SB) {
    s.whole = 0;
    const int fit = G > 0 ? G : ST;
    while (true) {
      const int k2 = s.ks * 2;
      if (units * k2 > fit || units * k2 > kSplitCap || !can_split(k2)) break;
      s.ks = k2;
    }
    return s;
  }
  const int rem = G > 0 ? units % G : 0;
  if (rem == 0) return s;
  int ks = 1;
  while (rem * ks * 2 <= G && can_split(ks * 2)) ks *= 2;
  // the reduce pass over the split tiles' partials costs about what a 2-way
  // split saves (measured: the LM head with 128 of 1920 tiles left over ran
  // 1.04 ms either way), so only splits of 4 or more are taken
  if (ks >= 4) {
    s.ks = ks;
    s.whole = units - rem;
  }
  return s;
}

// Order of the output tiles: groups of kGroupM row tiles, walked feature tile
// by feature tile within a group (consecutive positions share a feature
// tile's weights, and every kGroupM of them one set of token rows).  A
// bijection of [0, m_tiles * n_tiles).  Measured on the lock loop's Q/K/V
// GEMM: groups of 4 ran ~1 % faster than groups of 8, groups of 16 ~2 %
// slower.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_of(int q, int m_tiles, int n_tiles, int& mt, int& nt) {
  const int grp = q / (kGroupM * n_tiles);
  const int first = grp * kGroupM;
  const int gsize = min(kGroupM, m_tiles - first);
  const int r = q - grp * kGroupM * n_tiles;
  mt = first + r % gsize;
  nt = r / gsize;
}

// The hardware deals the workgroups of a launch round-robin to the 8 XCDs
// (workgroup b on XCD b % 8), each with its own L2.  Items of a loop handled
// round-robin by G workgroups (item w on workgroup w % G) are renumbered so
// that the workgroups of one XCD take consecutive positions of each round:
// with the grouped tile order, an XCD's tiles then form a compact block of
// feature and row tiles whose slices its L2 fetches once, instead of every
// weight slice being fetched by up to 8 L2s.  A bijection of [0, n).
__device__ __forceinline__ int xcd_local(int w, int n, int G) {
  const int r0 = w - w % G, b = w - r0;
  const int L = min(G, n - r0);  // items of this round
  const int x = b & 7, a = L >> 3, c = L & 7;
  return r0 + x * a + min(x, c) + (b >> 3);
}

// u16 elements of the double-buffered LDS tile (rows padded by 8 elements)
constexpr int gemm_lds_u16(int TP, int TT, int BK) { return 2 * (TP + TT) * (BK + 8); }

// Resolve the tile's token rows: cache row (b*S + idx[m], -1 for padding) and
// the byte offset of the operand row (past the end of the buffer for padding,
// so that its loads return zeros).
// PAIRS (EPI_LMKL): token row m is position (m/32)*16 + m%16, loaded from x
// (m%32 < 16) or x2; n_rows counts positions.
template <int TT, int AMODE, bool PAIRS = false>
__device__ __forceinline__ void gemm_rows(const GemmArgs& g, int n_rows, int m0, uint32_t* s_xoff,
                                          int* s_drow) {
  for (int t = threadIdx.x; t < TT; t += 256) {
    const int m = m0 + t;
    const int p = PAIRS ? (m >> 5) * 16 + (m & 15) : m;
    uint32_t xo = 0x80000000u;
    int drow = -1;
    if (p < n_rows) {
      const int b = batch_of(g.offsets, g.B, p);
      drow = b * g.S + g.idx[p];
      xo = (uint32_t)((AMODE == A_GATHER ? (size_t)drow : (size_t)p) * g.K * 2);
    }
    s_xoff[t] = xo;
    s_drow[t] = drow;
  }
}

// One output tile (or one K-split of it) of the gathered GEMM; the caller
// provides the LDS buffers so that several tilings can share one allocation.
// WK = 2: eight waves; waves 4..7 repeat the layout of waves 0..3 on the
// other half of every k-step's 16-wide sub-steps, two waves per SIMD hide each
// other's LDS and barrier latency, and the halves are added through LDS.
template <int TP, int TT, int WP, int WT, int BK, int PF, int EPI, int AMODE, int SB, int ST, int WK,
          int TPV>
__device__ __forceinline__ void gemm_tile_work(const GemmArgs& g, int n_rows, u16* lds, uint32_t* s_xoff,
                                               int* s_drow, const GemmSplit sp, int unit, int ksi,
                                               int n_tiles);

// TPV (<= TP): weight rows a tile really owns.  A tile of TP MFMA rows with
// TPV = 48 < TP = 64 lets the 12288-feature Q/K/V projection spread over 256
// tiles (one per CU) instead of 192: the other rows load zeros without memory
// traffic and the epilogue skips them (the weight-streaming body is bound by
// the bytes each CU reads, not by its MFMAs).
template <int TP, int TT, int WP, int WT, int BK, int PF, int EPI, int AMODE, int SB, int ST, int WK = 1,
          int TPV = TP>
__device__ __forceinline__ void gemm_tile_body(const GemmArgs& g, int n_rows, u16* lds,
                                               uint32_t* s_xoff, int* s_drow) {
  constexpr int NT = 256 * WK;   // threads
  constexpr int PITCH = BK + 8;  // u16 elements per LDS row (16 bytes of padding)
  constexpr int ROWS = TP + TT;
  constexpr int CPR = BK / 8;    // 16-byte chunks per row and k-step
  constexpr int RPJ = NT / CPR;  // rows covered by one chunk index of the workgroup
  constexpr int CHUNKS = ROWS * CPR;
  static_assert(CHUNKS % NT == 0 && TP % RPJ == 0, "tile rows must fill the workgroup");
  constexpr int CPT = CHUNKS / NT;
  constexpr int WTP = TP / WP, WTT = TT / WT, FP = WTP / 32, FT = WTT / 32;
  static_assert(WP * WT == 4 && FP >= 1 && FT >= 1, "wave layout");
  static_assert(PF >= 1, "prefetch depth");
  static_assert(2 * ROWS * PITCH == gemm_lds_u16(TP, TT, BK), "LDS size");
  static_assert(WK == 1 || (WK == 2 && !epi_lm(EPI) && (BK / 16) % 2 == 0 &&
                            FP * FT * 16 * 256 * 4 <= 2 * ROWS * PITCH * 2),
                "two k-halves: row epilogues only, partial sums fit the tile's LDS");

  const int m_tiles = (gemm_token_rows(EPI, n_rows) + TT - 1) / TT;
  const int n_tiles = g.N / TPV;
  const int nk_all = g.K / BK;
  const GemmSplit sp = gemm_split(m_tiles * n_tiles, nk_all, PF, SB, ST, g.tile_grid);
  const int total = sp.items();
  const int G = (int)gridDim.x;
  // Work items (tile position, k-split) go to workgroups round-robin: item w
  // runs on workgroup w % G, so a grid of one workgroup per CU keeps every
  // workgroup on the same k-step of its current tile.  Within each round the
  // items are renumbered XCD by XCD (xcd_local) and the positions walk the
  // grouped tile order (tile_of), so that the tiles running together on an
  // XCD share their weight and row slices in its L2.  The split tiles'
  // items come last (the last round; the renumbering needs the split
  // region to start a round, which it does unless the grid runs one item
  // per workgroup with unsplit tiles before it).
  for (int work = (int)blockIdx.x; work < total; work += (WK == 1 ? G : total)) {
    int unit, ksi = 0;
    if (work < sp.whole) {
      unit = xcd_local(work, sp.whole, G);
    } else {
      int j = work - sp.whole;
      const int ns = sp.units - sp.whole;
      if (sp.whole % G == 0) j = xcd_local(j, total - sp.whole, G);
      unit = sp.whole + j % ns;
      ksi = j / ns;
    }
    gemm_tile_work<TP, TT, WP, WT, BK, PF, EPI, AMODE, SB, ST, WK, TPV>(g, n_rows, lds, s_xoff, s_drow,
                                                                        sp, unit, ksi, n_tiles);
    if constexpr (WK == 1) __syncthreads();  // the next item rewrites the row table and tiles
  }
}

template <int TP, int TT, int WP, int WT, int BK, int PF, int EPI, int AMODE, int SB, int ST, int WK,
          int TPV>
__device__ __forceinline__ void gemm_tile_work(const GemmArgs& g, int n_rows, u16* lds, uint32_t* s_xoff,
                                               int* s_drow, const GemmSplit sp, int unit, int ksi,
                                               int n_tiles) {
  constexpr int NT = 256 * WK;   // threads
  constexpr int PITCH = BK + 8;  // u16 elements per LDS row (16 bytes of padding)
  constexpr int ROWS = TP + TT;
  constexpr int CPR = BK / 8;    // 16-byte chunks per row and k-step
  constexpr int RPJ = NT / CPR;  // rows covered by one chunk index of the workgroup
  constexpr int CHUNKS = ROWS * CPR;
  constexpr int CPT = CHUNKS / NT;
  constexpr int WTP = TP / WP, WTT = TT / WT, FP = WTP / 32, FT = WTT / 32;
  const int m_tiles = (gemm_token_rows(EPI, n_rows) + TT - 1) / TT;
  const int nk_all = g.K / BK;
  int mt, nt;  // unit: the tile's position in the grouped order
  tile_of(unit, m_tiles, n_tiles, mt, nt);
  const int m0 = mt * TT, n0 = nt * TPV;
  const int tid = threadIdx.x, lane = tid & 63, wave = (tid >> 6) & 3, wk = tid >> 8;
  const int ks = sp.splits_of(unit);
  const int nk = nk_all / ks;           // k-steps of this split
  const int kbase = ksi * nk;           // first k-step of this split

  gemm_rows<TT, AMODE, EPI == EPI_LMKL>(g, n_rows, m0, s_xoff, s_drow);
  __syncthreads();

  // Chunk j of this thread covers LDS row (tid/CPR + RPJ j), 16-byte column
  // tid%CPR.  Rows [0,TP) are weight rows (VGPR offset of row tid/CPR, the
  // rest of the offset uniform); rows [TP, TP+TT) are gathered token rows.
  constexpr int CW = TP / RPJ;  // chunks of weight rows per thread
  constexpr int CX = CPT - CW;  // chunks of token rows per thread
  const int r0 = tid / CPR, kc = tid % CPR;
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.w, (uint32_t)((size_t)g.N * g.K * 2));
  const void* xsrc = g.x;
  if constexpr (EPI == EPI_LMKL) {
    // a thread's token rows are all (tid/CPR) % 32 within their 32-row
    // groups: waves 0-1 load this step's rows (x), waves 2-3 the previous
    // step's (x2); the choice is uniform per wave, so the resource stays scalar
    static_assert(NT == 256 && RPJ == 32 && TP % 32 == 0, "paired token rows need 32 rows per chunk index");
    if (__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 7)) xsrc = g.x2;
  }
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(xsrc, g.x_bytes);
  const uint32_t woff = (uint32_t)(((size_t)(n0 + r0) * g.K + kc * 8) * 2);
  const uint32_t wstride = (uint32_t)(RPJ * g.K * 2);
  uint32_t xoff[CX];
#pragma unroll
  for (int j = 0; j < CX; ++j) {
    const uint32_t o = s_xoff[r0 + RPJ * j];
    xoff[j] = o + (o & 0x80000000u ? 0u : (uint32_t)(kc * 16));
  }
  u16* const ldsw = lds + r0 * PITCH + kc * 8;
  // The 64-feature weight-streaming tiling (short selections) walks each
  // workgroup's k-steps from its own starting point (wrapping around):
  // workgroups are dealt round-robin to the 8 XCDs, so the workgroups sharing
  // an XCD's L2 read different k-slices of the gathered rows (which all of
  // them re-read, and which fit in L2) instead of all hitting the same lines.
  // The larger tilings keep one order, so that tiles running together share
  // each weight and row slice while it is in L2.
  const int krot = TP == 64 ? ((int)blockIdx.x >> 3) % nk : 0;
  // weight rows past TPV: an offset past the resource's end reads zeros
  uint32_t wvoff[CW];
#pragma unroll
  for (int j = 0; j < CW; ++j) wvoff[j] = (TPV == TP || r0 + RPJ * j < TPV) ? woff : 0x80000000u;
  auto gload = [&](int j, int kstep) -> u32x4 {
    int kp = kstep + krot;
    kp -= kp >= nk ? nk : 0;
    const uint32_t ko = (uint32_t)(kbase + kp) * (BK * 2);
    if (j < CW) return buffer_load16(rW, wvoff[j], ko + (uint32_t)j * wstride);
    return buffer_load16(rX, xoff[j - CW], ko);
  };

  f32x16 acc[FP][FT];
#pragma unroll
  for (int a = 0; a < FP; ++a)
#pragma unroll
    for (int b = 0; b < FT; ++b) acc[a][b] = f32x16{};

  // Register ring of PF k-steps in flight; slot s holds k-step j with j % PF == s.
  // The steady-state loop is branch-free (loads past the end re-read the last
  // k-step, stores past the end go to the idle LDS buffer) and nk % PF == 0,
  // so the compiler can count outstanding loads exactly and waits only for
  // the oldest slot instead of draining the queue every k-step.
  u32x4 stg[PF][CPT];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) stg[p][j] = gload(j, min(p, nk - 1));
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) *reinterpret_cast<u32x4*>(ldsw + RPJ * j * PITCH) = stg[0][j];
#pragma unroll
  for (int j = 0; j < CPT; ++j) stg[0][j] = gload(j, min(PF, nk - 1));
  __syncthreads();

  const int wp = wave / WT, wt = wave % WT;
  const int lr = lane & 31, lg = lane >> 5;
  constexpr bool kBig = TP == 256 && TT == 256 && PF == 1 && WK == 1 && BK == 64;
  if constexpr (kBig) {
    // 256 x 256 tiles run one wave per SIMD, each wave a 128 x 128 block (16
    // accumulators), so the matrix pipe idles whenever an MFMA has to wait for
    // its fragments.  The fragment registers are double-buffered across the
    // k-step's four 16-wide substeps: the 16 MFMAs of substep kh issue
    // one-for-one with the 8 LDS reads of substep kh + 1; half of the last
    // substep's MFMAs carry the staging writes of the next k-step (into the
    // other LDS buffer, free since the last barrier) and the global loads of
    // the one after; its other half issues after the barrier, alongside the
    // reads of the next k-step's first fragments.
    static_assert(FP == 4 && FT == 4 && CPT == 16 && BK / 16 == 4, "the 256 x 256 schedule");
    bf16x8 fa[2][FP], fb[2][FT];
    auto rd = [&](int buf, int kk, int set) {
      const u16* sW = lds + buf * ROWS * PITCH;
      const u16* sX = sW + TP * PITCH;
#pragma unroll
      for (int a = 0; a < FP; ++a)
        fa[set][a] = as_bf16x8(*reinterpret_cast<const u32x4*>(sW + (wp * WTP + a * 32 + lr) * PITCH +
                                                                kk * 16 + lg * 8));
#pragma unroll
      for (int b = 0; b < FT; ++b)
        fb[set][b] = as_bf16x8(*reinterpret_cast<const u32x4*>(sX + (wt * WTT + b * 32 + lr) * PITCH +
                                                                kk * 16 + lg * 8));
    };
    auto mma = [&](int set, int a0, int a1) {
#pragma unroll
      for (int a = a0; a < a1; ++a)
#pragma unroll
        for (int b = 0; b < FT; ++b) acc[a][b] = mfma32x32x16(fa[set][a], fb[set][b], acc[a][b]);
    };
    // staging of chunks [j0, j1) of the next k-step: write them into the other
    // LDS buffer (free since the last barrier), then reuse their registers for
    // the loads of the k-step after it
    auto stage = [&](int buf, int kt, int j0, int j1) {
      u16* dst = ldsw + (buf ^ 1) * ROWS * PITCH;
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        *reinterpret_cast<u32x4*>(dst + RPJ * j * PITCH) = stg[0][j];
        stg[0][j] = gload(j, min(kt + 2, nk - 1));
      }
    };
    constexpr int CQ = CPT / 4;  // chunks staged per substep
    rd(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
#pragma unroll
      for (int kh = 0; kh < 3; ++kh) {
        rd(buf, kh + 1, (kh + 1) & 1);
        stage(buf, kt, kh * CQ, (kh + 1) * CQ);
        mma(kh & 1, 0, FP);
      }
      stage(buf, kt, 3 * CQ, CPT);
      mma(1, 0, FP / 2);
      // The 64 KB of staging loads per k-step pass the CU's vector memory
      // pipeline at 64 bytes a clock (1,024 cycles), so they are spread over
      // the four substeps, a quarter beside each one's MFMAs, instead of
      // being issued together in the last one.
#pragma unroll
      for (int kh = 0; kh < 3; ++kh) {
#pragma unroll
        for (int i = 0; i < FP + FT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
#pragma unroll
        for (int i = 0; i < CQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, FP * FT - (FP + FT) - CQ, 0);
      }
#pragma unroll
      for (int i = 0; i < CQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FP * FT / 2 - CQ, 0);
      __syncthreads();
      rd(buf ^ 1, 0, 0);
      mma(1, FP / 2, FP);
#pragma unroll
      for (int i = 0; i < FP + FT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      }
    }
  } else
  for (int kt0 = 0; kt0 < nk; kt0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int kt = kt0 + u;
      const int buf = (PF % 2 == 0) ? (u & 1) : (kt & 1);
      const u16* sW = lds + buf * ROWS * PITCH;
      const u16* sX = sW + TP * PITCH;
      if constexpr (TP == 64) {
        // Weight-streaming tiles do only 2-8 MFMAs per wave and k-step, too few
        // to cover an LDS round trip per 16-wide substep: all of the k-step's
        // fragments are read first, then the staging writes and loads issue
        // beside the MFMAs.
        constexpr int KH = BK / 16 / WK;
        bf16x8 af[KH][FP], bfr[KH][FT];
#pragma unroll
        for (int kh = 0; kh < KH; ++kh) {
          const int kk = wk * KH + kh;
#pragma unroll
          for (int a = 0; a < FP; ++a)
            af[kh][a] = as_bf16x8(*reinterpret_cast<const u32x4*>(sW + (wp * WTP + a * 32 + lr) * PITCH +
                                                                  kk * 16 + lg * 8));
#pragma unroll
          for (int b = 0; b < FT; ++b)
            bfr[kh][b] = as_bf16x8(*reinterpret_cast<const u32x4*>(sX + (wt * WTT + b * 32 + lr) * PITCH +
                                                                   kk * 16 + lg * 8));
        }
        const int slot = (u + 1) % PF;  // compile-time after unrolling
        u16* dst = ldsw + (buf ^ 1) * ROWS * PITCH;
#pragma unroll
        for (int j = 0; j < CPT; ++j) *reinterpret_cast<u32x4*>(dst + RPJ * j * PITCH) = stg[slot][j];
#pragma unroll
        for (int j = 0; j < CPT; ++j) stg[slot][j] = gload(j, min(kt + 1 + PF, nk - 1));
#pragma unroll
        for (int kh = 0; kh < KH; ++kh)
#pragma unroll
          for (int a = 0; a < FP; ++a)
#pragma unroll
            for (int b = 0; b < FT; ++b) acc[a][b] = mfma32x32x16(af[kh][a], bfr[kh][b], acc[a][b]);
        constexpr int NMF = KH * FP * FT;
        __builtin_amdgcn_sched_group_barrier(0x100, KH * (FP + FT), 0);  // DS read
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
          if (i < NMF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        }
        if (NMF > CPT) __builtin_amdgcn_sched_group_barrier(0x008, NMF - CPT, 0);
        __syncthreads();
        continue;
      }
#pragma unroll
      for (int kh = 0; kh < BK / 16 / WK; ++kh) {
        const int kk = wk * (BK / 16 / WK) + kh;
        bf16x8 af[FP], bfr[FT];
#pragma unroll
        for (int a = 0; a < FP; ++a)
          af[a] = as_bf16x8(*reinterpret_cast<const u32x4*>(sW + (wp * WTP + a * 32 + lr) * PITCH +
                                                            kk * 16 + lg * 8));
#pragma unroll
        for (int b = 0; b < FT; ++b)
          bfr[b] = as_bf16x8(*reinterpret_cast<const u32x4*>(sX + (wt * WTT + b * 32 + lr) * PITCH +
                                                             kk * 16 + lg * 8));
#pragma unroll
        for (int a = 0; a < FP; ++a)
#pragma unroll
          for (int b = 0; b < FT; ++b) acc[a][b] = mfma32x32x16(af[a], bfr[b], acc[a][b]);
      }
      const int slot = (u + 1) % PF;  // compile-time after unrolling
      u16* dst = ldsw + (buf ^ 1) * ROWS * PITCH;
#pragma unroll
      for (int j = 0; j < CPT; ++j) *reinterpret_cast<u32x4*>(dst + RPJ * j * PITCH) = stg[slot][j];
#pragma unroll
      for (int j = 0; j < CPT; ++j) stg[slot][j] = gload(j, min(kt + 1 + PF, nk - 1));
      __syncthreads();
    }
  }

  if constexpr (WK == 2) {
    // add the second k-half into the first: waves 4..7 park their sums in the
    // (now idle) tile LDS in register order, waves 0..3 add them
    float* red = reinterpret_cast<float*>(lds);
    if (wk == 1) {
#pragma unroll
      for (int a = 0; a < FP; ++a)
#pragma unroll
        for (int b = 0; b < FT; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) red[(((a * FT + b) * 16 + i) * 4 + wave) * 64 + lane] = acc[a][b][i];
    }
    __syncthreads();
    if (wk == 1) return;
#pragma unroll
    for (int a = 0; a < FP; ++a)
#pragma unroll
      for (int b = 0; b < FT; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] += red[(((a * FT + b) * 16 + i) * 4 + wave) * 64 + lane];
  }

  if (ks > 1) {
    // split-K: store the partial tile in register order (16-byte vectors,
    // consecutive threads adjacent; padding tokens are skipped, the reduction
    // skips them too); gemm_splitk_reduce_kernel sums the splits in a fixed
    // order after this kernel has finished
    constexpr int NQ = FP * FT * 4;
    float4* mine = reinterpret_cast<float4*>(g.part) + ((size_t)(unit - sp.whole) * ks + ksi) * (NQ * 256);
#pragma unroll
    for (int b = 0; b < FT; ++b) {
      if (s_drow[wt * WTT + b * 32 + lr] < 0) continue;
#pragma unroll
      for (int a = 0; a < FP; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          mine[((a * FT + b) * 4 + q) * 256 + tid] = make_float4(
              acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
    }
    return;
  }
  gemm_epilogue<TP, TT, WP, WT, EPI, TPV>(g, acc, m0, n0, nt, s_drow);
}

// GATE: 0 = always run; 1 = run only when the device row count is <= kSkinnyRows;
// 2 = run only when it is larger.
template <int TP, int TT, int WP, int WT, int BK, int PF, int EPI, int AMODE, int GATE, int SB, int ST,
          int WK = 1, int TPV = TP>
__global__ __launch_bounds__(256 * WK) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) u16 lds[gemm_lds_u16(TP, TT, BK)];
  __shared__ uint32_t s_xoff[TT];
  __shared__ int s_drow[TT];
  const int n_rows = min(g.offsets[g.B], g.max_rows);
  if ((GATE == 1 && n_rows > kSkinnyRows) || (GATE == 2 && n_rows <= kSkinnyRows)) return;
  gemm_tile_body<TP, TT, WP, WT, BK, PF, EPI, AMODE, SB, ST, WK, TPV>(g, n_rows, lds, s_xoff, s_drow);
}

// One launch for a host that only knows a loose row bound: the device row
// count picks the weight-streaming tiling (<= kSkinnyRows rows) or the large
// tiling, so no second launch has to start just to exit.  Both bodies share
// one LDS allocation sized for the larger of the two.
template <int TP, int TT, int BK, int PF, int SB, int ST, int TP2, int TT2, int BK2, int PF2, int SB2,
          int ST2, int EPI, int AMODE, int TPV1>
__global__ __launch_bounds__(256) void gemm_dual_kernel(GemmArgs g) {
  // TPV1: weight rows per tile of the weight-streaming body (see gemm_tile_body)
  constexpr int L1 = gemm_lds_u16(TP, TT, BK), L2 = gemm_lds_u16(TP2, TT2, BK2);
  constexpr int TTM = TT > TT2 ? TT : TT2;
  __shared__ __attribute__((aligned(16))) u16 lds[L1 > L2 ? L1 : L2];
  __shared__ uint32_t s_xoff[TTM];
  __shared__ int s_drow[TTM];
  const int n_rows = min(g.offsets[g.B], g.max_rows);
  if (n_rows <= kSkinnyRows)
    gemm_tile_body<TP, TT, 2, 2, BK, PF, EPI, AMODE, SB, ST, 1, TPV1>(g, n_rows, lds, s_xoff, s_drow);
  else
    gemm_tile_body<TP2, TT2, 2, 2, BK2, PF2, EPI, AMODE, SB2, ST2>(g, n_rows, lds, s_xoff, s_drow);
}

// Second pass of split-K.  The plan is recomputed from the same inputs (the
// pass exits at once when the device did not split).  For the row epilogues a
// tile's 16-byte register groups are shared out over several workgroups
// (about kReduceTarget in all), each summing its groups over the splits in
// split order and storing them; the LM-head epilogue needs whole rows, so one
// workgroup reduces one tile.
template <int TP, int TT, int WP, int WT, int BK, int PF, int EPI, int AMODE, int GATE, int SB, int ST>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(GemmArgs g) {
  constexpr int WTP = TP / WP, WTT = TT / WT, FP = WTP / 32, FT = WTT / 32;
  constexpr int NQ = FP * FT * 4;
  __shared__ int s_drow[TT];
  __shared__ uint32_t s_xoff[TT];
  const int n_rows = min(g.offsets[g.B], g.max_rows);
  if ((GATE == 1 && n_rows > kSkinnyRows) || (GATE == 2 && n_rows <= kSkinnyRows)) return;
  const int m_tiles = (gemm_token_rows(EPI, n_rows) + TT - 1) / TT;
  const int n_tiles = g.N / TP;
  const GemmSplit sp = gemm_split(m_tiles * n_tiles, g.K / BK, PF, SB, ST, g.tile_grid);
  const int n_split = sp.units - sp.whole;  // tiles whose K was split
  if (sp.ks <= 1 || n_split <= 0) return;
  const int RS = epi_lm(EPI) ? 1 : min(NQ, (kReduceTarget + n_split - 1) / n_split);
  if ((int)blockIdx.x >= n_split * RS) return;
  const int unit = sp.whole + (int)blockIdx.x / RS, slice = (int)blockIdx.x % RS;
  int mt, nt;
  tile_of(unit, m_tiles, n_tiles, mt, nt);
  const int m0 = mt * TT, n0 = nt * TP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const int wp = wave / WT, wt = wave % WT;
  gemm_rows<TT, AMODE, EPI == EPI_LMKL>(g, n_rows, m0, s_xoff, s_drow);
  __syncthreads();
  const float4* all = reinterpret_cast<const float4*>(g.part) + (size_t)(unit - sp.whole) * sp.ks * (NQ * 256);
  auto sum_splits = [&](int gi) {
    const int o = gi * 256 + tid;
    float4 v[8];
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2)  // splits past ks re-read split 0 (not added below)
      v[k2] = all[(size_t)(k2 < sp.ks ? k2 : 0) * (NQ * 256) + o];
    float4 sum = v[0];
#pragma unroll
    for (int k2 = 1; k2 < 8; ++k2)
      if (k2 < sp.ks) {
        sum.x += v[k2].x;
        sum.y += v[k2].y;
        sum.z += v[k2].z;
        sum.w += v[k2].w;
      }
    return sum;
  };
  if constexpr (epi_lm(EPI)) {
    f32x16 acc[FP][FT];
#pragma unroll
    for (int a = 0; a < FP; ++a)
#pragma unroll
      for (int b = 0; b < FT; ++b)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // padding tokens hold no partials: their sums are never used
          const float4 s = s_drow[wt * WTT + b * 32 + lr] >= 0 ? sum_splits((a * FT + b) * 4 + q)
                                                             : make_float4(0.f, 0.f, 0.f, 0.f);
          acc[a][b][4 * q] = s.x;
          acc[a][b][4 * q + 1] = s.y;
          acc[a][b][4 * q + 2] = s.z;
          acc[a][b][4 * q + 3] = s.w;
        }
    gemm_epilogue<TP, TT, WP, WT, EPI>(g, acc, m0, n0, nt, s_drow);
  } else {
    const int per = (NQ + RS - 1) / RS;
    const int g_end = min(NQ, (slice + 1) * per);
    // four groups at a time, so that their partial loads are in flight together
    for (int g0 = slice * per; g0 < g_end; g0 += 4) {
      float4 sv[4];
      int drow[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int gi = min(g0 + u, g_end - 1);
        drow[u] = g0 + u < g_end ? s_drow[wt * WTT + ((gi / 4) % FT) * 32 + lr] : -1;
        sv[u] = sum_splits(gi);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (drow[u] < 0) continue;  // padding token or past the slice
        const int gi = g0 + u;
        const int a = gi / (FT * 4), b = (gi / 4) % FT, q = gi % 4;
        epi_store4<EPI>(g, m0 + wt * WTT + b * 32 + lr, drow[u], n0 + wp * WTP + a * 32 + 8 * q + 4 * lg,
                        sv[u].x, sv[u].y, sv[u].z, sv[u].w);
      }
    }
  }
}

// fp32 path (small fp32 layers): one thread per output element, float4 loads
// issued eight at a time before they are used (the layer is latency-bound),
// float32 accumulation over k in four partial sums.
template <int EPI, int AMODE>
__global__ __launch_bounds__(64) void gemm_f32_kernel(GemmArgs g) {
  const int m = blockIdx.y, n = blockIdx.x * 64 + threadIdx.x;
  const int n_rows = min(g.offsets[g.B], g.max_rows);
  if (m >= n_rows || n >= g.N) return;
  const int b = batch_of(g.offsets, g.B, m);
  const int drow = b * g.S + g.idx[m];
  const float4* xr = reinterpret_cast<const float4*>(static_cast<const float*>(g.x) +
                     (AMODE == A_GATHER ? (size_t)drow * g.K : (size_t)m * g.K));
  const float4* wr = reinterpret_cast<const float4*>(static_cast<const float*>(g.w) + (size_t)n * g.K);
  float part[4] = {0.f, 0.f, 0.f, 0.f};
  const int k4 = g.K / 4;
  int c = 0;
  for (; c + 8 <= k4; c += 8) {
    float4 xv[8], wv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      xv[u] = xr[c + u];
      wv[u] = wr[c + u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float& acc = part[u & 3];
      acc = fmaf(xv[u].x, wv[u].x, acc);
      acc = fmaf(xv[u].y, wv[u].y, acc);
      acc = fmaf(xv[u].z, wv[u].z, acc);
      acc = fmaf(xv[u].w, wv[u].w, acc);
    }
  }
  for (; c < k4; ++c) {
    const float4 xv = xr[c], wv = wr[c];
    part[0] = fmaf(xv.x, wv.x, part[0]);
    part[1] = fmaf(xv.y, wv.y, part[1]);
    part[2] = fmaf(xv.z, wv.z, part[2]);
    part[3] = fmaf(xv.w, wv.w, part[3]);
  }
  const float acc = (part[0] + part[1]) + (part[2] + part[3]);
  float* dst;
  if constexpr (EPI == EPI_QKV) {
    if (n < g.nq)
      dst = static_cast<float*>(g.q_out) + (size_t)m * g.nq + n;
    else if (n < g.nq + g.nk)
      dst = static_cast<float*>(g.k_cache) + (size_t)drow * g.nk + (n - g.nq);
    else
      dst = static_cast<float*>(g.v_cache) + (size_t)drow * g.nk + (n - g.nq - g.nk);
  } else {
    dst = static_cast<float*>(g.out) + (size_t)drow * g.ld_out + n;
  }
  *dst = acc;
}

// ---------------------------------------------------------------------------
// Host dispatch.  Tile shapes (features x tokens, prefetch depth):
//   <= kSkinnyRows rows: 64 x 128, 4-deep ring, one workgroup per CU.
//   loose bounds up to 1024 rows: 128 x 128 for the large case, 4-deep ring.
//   LM head and looser bounds: 256 x 256, each wave a 128 x 128 block, so
//     every LDS fragment feeds four MFMAs; 1-deep ring; K split when the
//     device finds fewer than 256 output tiles.
constexpr int kLmTP = 256;
int gemm_lmhead_ntile(int V) { return V / kLmTP; }

static int pf_for(int nk, int pfmax) {
  for (int pf = pfmax; pf > 1; pf /= 2)
    if (nk % pf == 0) return pf;
  return 1;
}

// Split-K partial tiles (fp32) of the tilings that may split.  The device
// plans the split from the real row count, which may be anything up to the
// bound, so the workspace holds the most partial tiles any count <= the bound
// can take: ks <= 8 splits of at most every output tile of the bound, and
// never more than kSplitCap (a split of every tile stays below it; a split
// last round holds fewer tiles than the resident grid).
size_t gemm_workspace_bytes(int epi, int max_rows, int N, int K) {
  if (max_rows <= 0) return 0;
  const int rows = gemm_token_rows(epi, max_rows);
  int TP;
  if (epi_lm(epi))
    TP = kLmTP;
  else if (rows > 1024 && N % 256 == 0 && (K / 64) % 4 == 0)
    TP = 256;  // the 256 x 256 tiling (other shapes never split)
  else
    return 0;
  const long long units = (long long)(N / TP) * ((rows + 255) / 256);
  const long long tiles = units * 8 < kSplitCap ? units * 8 : kSplitCap;
  return (size_t)tiles * TP * 256 * sizeof(float);
}

// The weight-streaming tiling of a narrow output: N = 4096 features (the
// FFN's down projection) make 64 tiles, so 64 CUs stream the weights while
// the rest idle.  A caller that passes the partial tiles' memory
// (GemmArgs::skinny_split) has K split while the work items stay within
// kSkinnySplitItems (one per CU), each streaming a K-slice; the reduce pass
// then adds the fp32 partials in split order.
constexpr int kSkinnySplitUnits = 128;  // split only outputs of fewer tiles
constexpr int kSkinnySplitItems = 256;  // at most this many items (tiles x splits)
size_t gemm_skinny_split_bytes(int max_rows, int N, int K) {
  if (max_rows <= 0 || max_rows > kSkinnyRows || N % 64 != 0 || K % 64 != 0 || (K / 64) % 4 != 0)
    return 0;
  const int units = N / 64;  // one row tile (at most 128 rows)
  if (units >= kSkinnySplitUnits) return 0;
  const GemmSplit s = gemm_split(units, K / 64, 4, kSkinnySplitUnits, kSkinnySplitItems, 0);
  if (s.ks <= 1) return 0;
  return (size_t)s.items() * 64 * 128 * sizeof(float);
}

template <int TP, int TT, int WP, int WT, int BK, int PF, int EPI, int AMODE, int GATE, int SB, int ST>
static void launch_reduce(const GemmArgs& g, hipStream_t st) {
  hipLaunchKernelGGL((gemm_splitk_reduce_kernel<TP, TT, WP, WT, BK, PF, EPI, AMODE, GATE, SB, ST>),
                     dim3(SB + kReduceTarget), dim3(256), 0, st, g);
}

// Grid of a tiling whose work items loop over workgroups: as many workgroups
// as are resident at once (one per CU for the 256-wide tiles, two otherwise),
// never more than there are items.
static int persistent_grid(int items, int TP, int TT) {
  const int resident = device_cus() * (TP * TT >= 256 * 256 ? 1 : 2);
  return items < resident ? items : resident;
}

template <int TP, int TT, int BK, int PF, int EPI, int AMODE, int GATE, int SB, int ST, int WK = 1,
          int TPV = TP>
static void launch_bf16(const GemmArgs& g, hipStream_t st) {
  static_assert(SB == 0 || TPV == TP, "split tiles own all their weight rows");
  // every output tile (and every split the device may choose when the real
  // selection turns out short) is a work item; the two-k-half tiling runs one
  // item per workgroup, the others loop over a resident grid
  const int m_tiles_max = (gemm_token_rows(EPI, g.max_rows) + TT - 1) / TT;
  int items = (g.N / TPV) * m_tiles_max;
  if (SB > 0) {
    const int cap = ST < kSplitCap ? 2 * ST : kSplitCap;
    if (WK == 2 && m_tiles_max <= 1)
      items = gemm_split(items, g.K / BK, PF, SB, ST, 0).items();  // the device plans these tiles or none
    else if (items < cap)
      items = cap;
  }
  const int grid = WK == 1 ? persistent_grid(items, TP, TT) : items;
  GemmArgs ga = g;
  ga.tile_grid = grid;  // the split plan fills the last round of this grid
  hipLaunchKernelGGL((gemm_bf16_kernel<TP, TT, 2, 2, BK, PF, EPI, AMODE, GATE, SB, ST, WK, TPV>),
                     dim3(grid), dim3(256 * WK), 0, st, ga);
  if (SB > 0) launch_reduce<TP, TT, 2, 2, BK, PF, EPI, AMODE, GATE, SB, ST>(ga, st);
}

// the weight-streaming tiling alone (GATE 0 or 1).  Measured at n = 102:
// 128-wide k-steps with a 2-deep ring (half the barriers, same bytes in
// flight) ran 36.7 us against 34.7 us for 64-wide steps with a 4-deep ring.
template <int EPI, int AMODE, int GATE>
static void launch_skinny(const GemmArgs& g, hipStream_t st) {
  if constexpr (EPI == EPI_ROWS) {
    if (g.skinny_split && gemm_skinny_split_bytes(g.max_rows, g.N, g.K) > 0) {
      launch_bf16<64, 128, 64, 4, EPI, AMODE, GATE, kSkinnySplitUnits, kSkinnySplitItems, 2>(g, st);
      return;
    }
  }
  // 48 weight rows per tile when they divide N, as in the dual launch: the
  // 24576 gate/up features of the salient FFN make 512 tiles, two per CU,
  // instead of 384 tiles that leave half the CUs with one
  if (pf_for(g.K / 64, 4) == 4 && g.N % 48 == 0)
    launch_bf16<64, 128, 64, 4, EPI, AMODE, GATE, 0, 0, 2, 48>(g, st);
  else if (pf_for(g.K / 64, 4) == 4)
    launch_bf16<64, 128, 64, 4, EPI, AMODE, GATE, 0, 0, 2>(g, st);
  else if (pf_for(g.K / 64, 4) == 2)
    launch_bf16<64, 128, 64, 2, EPI, AMODE, GATE, 0, 0>(g, st);
  else
    launch_bf16<64, 128, 64, 1, EPI, AMODE, GATE, 0, 0>(g, st);
}

// loose bound: one launch whose device row count picks the body, then the
// split-K pass of the large body when it may split
template <int BK1, int PF1, int TP2, int TT2, int PF2, int SB2, int ST2, int EPI, int AMODE>
static void launch_dual(const GemmArgs& g, hipStream_t st) {
  int items2 = (g.N / TP2) * ((g.max_rows + TT2 - 1) / TT2);
  if (SB2 > 0 && items2 < kSplitCap) items2 = kSplitCap;
  // 48 weight rows per weight-streaming tile when they divide N (every CU gets a tile)
  const bool t48 = g.N % 48 == 0;
  const int grid1 = persistent_grid(g.N / (t48 ? 48 : 64), 64, 128), grid2 = persistent_grid(items2, TP2, TT2);
  const int grid = grid1 > grid2 ? grid1 : grid2;
  GemmArgs ga = g;
  ga.tile_grid = grid;  // the split plan fills the last round of this grid
  if (t48)
    hipLaunchKernelGGL((gemm_dual_kernel<64, 128, BK1, PF1, 0, 0, TP2, TT2, 64, PF2, SB2, ST2, EPI, AMODE, 48>),
                       dim3(grid), dim3(256), 0, st, ga);
  else
    hipLaunchKernelGGL((gemm_dual_kernel<64, 128, BK1, PF1, 0, 0, TP2, TT2, 64, PF2, SB2, ST2, EPI, AMODE, 64>),
                       dim3(grid), dim3(256), 0, st, ga);
  if (SB2 > 0) launch_reduce<TP2, TT2, 2, 2, 64, PF2, EPI, AMODE, 2, SB2, ST2>(ga, st);
}

template <int EPI, int AMODE>
static void launch_by_rows(const GemmArgs& g, hipStream_t st) {
  if (g.max_rows <= kSkinnyRows || g.N % 128 != 0) {
    launch_skinny<EPI, AMODE, 0>(g, st);
    return;
  }
  // loose bound (K / 64 is a multiple of 4 here)
  if (g.max_rows <= 1024 || g.N % 256 != 0)
    launch_dual<64, 4, 128, 128, 4, 0, 0, EPI, AMODE>(g, st);
  else
    launch_dual<64, 4, 256, 256, 1, 256, 768, EPI, AMODE>(g, st);
}

hipError_t launch_gemm(int dtype, int epi, int amode, const GemmArgs& g, hipStream_t st) {
  if (g.max_rows <= 0) return hipSuccess;
  if (dtype == 0) {
    const dim3 grid((g.N + 63) / 64, g.max_rows);
    if (epi == EPI_QKV)
      hipLaunchKernelGGL((gemm_f32_kernel<EPI_QKV, A_GATHER>), grid, dim3(64), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_f32_kernel<EPI_ROWS, A_COMPACT>), grid, dim3(64), 0, st, g);
    return hipGetLastError();
  }
  if (epi == EPI_LMHEAD) {
    launch_bf16<kLmTP, 256, 64, 1, EPI_LMHEAD, A_GATHER, 0, 256, 768>(g, st);
  } else if (epi == EPI_LMMARGIN) {
    launch_bf16<kLmTP, 256, 64, 1, EPI_LMMARGIN, A_GATHER, 0, 256, 768>(g, st);
  } else if (epi == EPI_LMKL) {
    launch_bf16<kLmTP, 256, 64, 1, EPI_LMKL, A_GATHER, 0, 256, 768>(g, st);
  } else if ((g.K / 64) % 4 != 0 && g.max_rows > kSkinnyRows && g.N % 128 == 0) {
    // short K: the 4-deep skinny ring does not divide it; one large tiling
    // (its 128-feature tiles must divide N; otherwise the 64-feature tiling
    // below, whose ring depth divides any K)
    if (epi == EPI_QKV)
      launch_bf16<128, 128, 64, 1, EPI_QKV, A_GATHER, 0, 0, 0>(g, st);
    else if (epi == EPI_SWIGLU)
      launch_bf16<128, 128, 64, 1, EPI_SWIGLU, A_GATHER, 0, 0, 0>(g, st);
    else
      launch_bf16<128, 128, 64, 1, EPI_ROWS, A_COMPACT, 0, 0, 0>(g, st);
  } else if (epi == EPI_QKV) {
    launch_by_rows<EPI_QKV, A_GATHER>(g, st);
  } else if (epi == EPI_SWIGLU) {
    launch_by_rows<EPI_SWIGLU, A_GATHER>(g, st);
  } else {
    launch_by_rows<EPI_ROWS, A_COMPACT>(g, st);
  }
  return hipGetLastError();
}

}  // namespace dlm
