// Bidirectional partial attention of the selected queries over all keys.
//
// DyLLM, Methodologie 2 (salient path): attention rows of the selected tokens
// are recomputed in full against every key; SureLock, Methodik,
// Kernprinzipien: active tokens attend to the cached K/V of locked tokens, so
// the cost is O(M N d) for M active rows.  No mask: the model is bidirectional.
//
// bf16 kernel (gfx950 matrix cores), flash-style online softmax:
//   * A workgroup owns 128 or 256 query vectors (row, head) that share one KV
//     head of one sequence (GQA packs the G query heads of a KV head
//     together); each wave owns 32 of them.  256-vector workgroups (eight
//     waves) serve MHA-like selections (fewer than 4 query heads per KV head)
//     with many query tiles: every K/V tile is read from L2 once per 256
//     vectors instead of once per 128.
//   * Per 64-key tile (32-key tiles for long GQA selections at head dim 128,
//     which then run three workgroups per CU), K and V come in through buffer
//     loads (one tile ahead, in registers) and are staged in LDS; every wave
//     computes the transposed score tiles S^T = K . Q^T (32 keys x 32 queries
//     each) with 32x32x16 MFMAs; Q^T stays in registers for the whole key
//     loop.  The key mask is compiled only into the copy of the tile math that
//     runs the split's partial last tile.
//   * In that layout a lane holds 16 keys of one query, so the running max and
//     sum are in-lane reductions plus one v_permlane32_swap with the lane that
//     holds the other 16 keys of the same query.
//   * P^T (bf16) is already in the B-operand layout of O^T = V^T . P^T; the
//     V^T operand is read with ds_read_b64_tr_b16, which transposes 4x16
//     blocks of V on the way out of LDS.
//   * Few queries (short selections): the key range is split over workgroups
//     and a merge pass combines the partial outputs by their LSE.
// fp32 kernel (small fp32 layers): one wave per (row, head), float32 FMA,
// loads issued in batches ahead of use (the layer is latency-bound).
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace dlm {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 lds_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Work plan shared by the attention and merge kernels, computed on the device
// from the selection counts (the host only knows an upper bound):
//   units  = sum_b ceil(n_b * G / QT) query tiles of QT vectors, times Hkv
//   nsplit = CUs / units (rounded down) when at least two splits fit one
//            workgroup per CU, else 1; capped at 16 and at S/256.  So short
//            selections still spread their K/V reads over the whole GPU (one
//            CU streams only a few tens of GB/s, so a few workgroups cannot
//            read a long cache fast); the merge pass combines the split
//            partials by their LSE.  Splitting further, to two workgroups per
//            CU, gains nothing in these short launches (a CU's second
//            workgroup adds no throughput here) and costs partial outputs,
//            written and merged: measured at B = 8, S = 2048, 32/8 heads,
//            256 units took 51.7 us unsplit and 62.3 us in two splits, 192
//            units 49.9 against 62.2 us in three.  Each split keeps at least
//            256 keys: shorter ones cost more in partials than they gain.
// A last cap keeps nsplit * n_rows * Hq <= kPartRows, the bound the
// workspace is sized for.
constexpr int kShortUnits = 512;  // a row bound of fewer 128-vector tiles: a short selection
constexpr int kPartRows = 2 * kShortUnits * 128;
constexpr int kAttnKT = 64;      // keys per K/V tile (and the split granule)
constexpr int kMinSplitKeys = 256;  // keys per split at least
constexpr float kLaneSumCap = 0x1p64f;  // a lane's tile sum above this: rescale
constexpr int kMergeGrid = 1024; // workgroups of the merge pass (grid-stride)

struct AttnPlan {
  int units;
  int nsplit;
  int kps;     // keys per split (a multiple of kAttnKT)
  int n_rows;
};

__device__ __forceinline__ AttnPlan attn_plan(const AttnArgs& a, int QT) {
  const int G = a.Hq / a.Hkv;
  int tiles = 0;
  for (int bb = 0; bb < a.B; ++bb) {
    const int n_b = min(a.offsets[bb + 1], a.max_rows) - min(a.offsets[bb], a.max_rows);
    tiles += (n_b * G + QT - 1) / QT;
  }
  AttnPlan p;
  p.units = tiles * a.Hkv;
  p.n_rows = min(a.offsets[a.B], a.max_rows);
  int ns = 1;
  if (p.units > 0 && 2 * p.units <= a.split_fill) {
    ns = a.split_fill / p.units;
    ns = min(ns, 16);
    ns = min(ns, max(1, a.S / kMinSplitKeys));
    if (p.n_rows > 0) ns = min(ns, max(1, kPartRows / (p.n_rows * a.Hq)));
  }
  // keys per split are rounded up to whole tiles; recount the splits from that
  // size so that none of them is empty
  p.kps = ((a.S + ns - 1) / ns + kAttnKT - 1) / kAttnKT * kAttnKT;
  p.nsplit = (a.S + p.kps - 1) / p.kps;
  return p;
}

// LDS of the attention kernel (u16 elements)
template <int HD, int KT = kAttnKT>
// Row pitches (u16) chosen for conflict-free LDS access:
//   K rows are read as 16-byte A-fragments by 16 lanes on 16 consecutive rows:
//     a pitch of HD + 8 moves each row by 4 banks (HD = 128) or 36 banks (64).
//   V rows are read transposed (ds_read_b64_tr_b16): 32 lanes touch 4
//     consecutive rows x 32 elements (16 banks each), so consecutive rows must
//     sit 16 banks apart: a pitch of HD + 32 (320 or 192 bytes).
struct AttnLds {
  static constexpr int KPITCH = HD + 8;
  static constexpr int VPITCH = HD + 32;
  static constexpr int WIDE = KT * (KPITCH + VPITCH);
};

// Locate the (batch row, kv head, query tile) of a unit: tiles of QT query
// vectors are counted per batch row, Hkv units per tile.
struct AttnUnit {
  int b, nb, row_base, g, t, split;
};
__device__ __forceinline__ AttnUnit attn_unit(const AttnArgs& a, const AttnPlan& plan, int QT) {
  AttnUnit u;
  u.split = blockIdx.x % plan.nsplit;
  const int rest = blockIdx.x / plan.nsplit;
  u.g = rest % a.Hkv;
  int t = rest / a.Hkv;
  const int G = a.Hq / a.Hkv;
  u.b = -1;
  u.nb = 0;
  u.row_base = 0;
  for (int bb = 0; bb < a.B; ++bb) {
    const int lo_b = min(a.offsets[bb], a.max_rows), hi_b = min(a.offsets[bb + 1], a.max_rows);
    const int n_b = hi_b - lo_b;
    const int tb = (n_b * G + QT - 1) / QT;
    if (t < tb) {
      u.b = bb;
      u.nb = n_b;
      u.row_base = lo_b;
      break;
    }
    t -= tb;
  }
  u.t = t;
  return u;
}

// Store 32 rows d0..d0+31 (one O^T block) of a query vector, already divided
// by the softmax sum: bf16 to o (and the context row of the output cache), or
// fp32 to the split partials.  Register i of the block holds d = 8(i/4) +
// 4*lg + i%4 of the query in column lr.
template <int HD>
__device__ __forceinline__ void attn_store_block(const AttnArgs& a, const AttnPlan& plan, int split,
                                                 int b, int row, int h, int dblk, const f32x16& o,
                                                 float inv, int lg) {
  if (plan.nsplit == 1) {
    u16* op = static_cast<u16*>(a.o) + ((size_t)row * a.Hq + h) * HD;
    u16* cp = a.ctx_out ? static_cast<u16*>(a.ctx_out) + ((size_t)(b * a.S + a.idx[row]) * a.Hq + h) * HD
                        : nullptr;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dblk + 8 * q4 + 4 * lg;
      u32x2 pk;
      pk[0] = pack_bf16x2(o[4 * q4] * inv, o[4 * q4 + 1] * inv);
      pk[1] = pack_bf16x2(o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + d0) = pk;
      if (cp) *reinterpret_cast<u32x2*>(cp + d0) = pk;
    }
  } else {
    float* po = a.part_o + (((size_t)split * plan.n_rows + row) * a.Hq + h) * HD;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * dblk + 8 * q4 + 4 * lg;
      *reinterpret_cast<float4*>(po + d0) =
          make_float4(o[4 * q4] * inv, o[4 * q4 + 1] * inv, o[4 * q4 + 2] * inv, o[4 * q4 + 3] * inv);
    }
  }
}

template <int HD>
__device__ __forceinline__ void attn_store_lse(const AttnArgs& a, const AttnPlan& plan, int split,
                                               int row, int h, float lse_nat) {
  if (plan.nsplit == 1) {
    if (a.lse) a.lse[(size_t)row * a.Hq + h] = lse_nat;
  } else {
    a.part_lse[((size_t)split * plan.n_rows + row) * a.Hq + h] = lse_nat;
  }
}

// Multiply P^T into O^T for one 32-key block whose first LDS row is kb0:
// O^T[d] += V^T(32 d x 16 keys) . P^T(16 keys x 32 queries), two 16-key chunks.
// pw[cc] holds the block's probabilities as bf16 pairs, word j of chunk cc =
// registers 8cc + 2j and 8cc + 2j + 1; register i of the block is key
// 8(i/4) + 4*lg + i%4.  The V^T operand is read with ds_read_b64_tr_b16 in the
// matching key-slot order: k-slots 8*ga+0..3 <-> keys 16cc+4ga+0..3, slots
// 8*ga+4..7 <-> keys 16cc+8+4ga+0..3.
template <int HD>
__device__ __forceinline__ void attn_pv_block(const u16* sV, int kb0, const u32x4 (&pw)[2],
                                              f32x16 (&acc)[HD / 32], int lane) {
  constexpr int PITCH = AttnLds<HD>::VPITCH, NDB = HD / 32;
  const int g16 = lane >> 4, j16 = lane & 15, ga = g16 >> 1;
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    const int m0 = 32 * d + 16 * (g16 & 1);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u16* pa = sV + (kb0 + 16 * cc + 4 * ga + (j16 >> 2)) * PITCH + m0 + 4 * (j16 & 3);
      const i16x4 va = lds_read_tr16(pa);
      const i16x4 vb = lds_read_tr16(pa + 8 * PITCH);
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[d] = mfma32x32x16(av, as_bf16x8(pw[cc]), acc[d]);
    }
  }
}

// QT = 128*WQ query vectors per workgroup of 4*WQ waves (wave w owns vectors
// 32w..32w+31) share every KT-key tile of the split: each tile is read from
// L2 once per QT vectors, so WQ = 2 halves the K/V bytes a CU pulls per flop.
template <int HD, int WQ, int KT>
__device__ __forceinline__ void attn_body(const AttnArgs& a, const AttnPlan& plan, u16* smem) {
  constexpr int QT = 128 * WQ;   // query vectors per workgroup
  constexpr int NT = 256 * WQ;   // threads per workgroup
  constexpr int NKB = KT / 32;   // 32-key MFMA blocks per tile (1 or 2)
  static_assert(KT == 32 || KT == 64, "tiles of one or two 32-key blocks");
  constexpr int PITCH = AttnLds<HD>::KPITCH, VPITCH = AttnLds<HD>::VPITCH;  // u16 per LDS row
  constexpr int NS = HD / 16;    // k-chunks of Q.K^T
  constexpr int NDB = HD / 32;   // 32-row blocks of O^T
  constexpr int CPR = HD / 8;    // 16-byte chunks per K/V row
  constexpr int CPT = 2 * KT * CPR / NT;
  u16* sK = smem;
  u16* sV = smem + KT * PITCH;  // V rows at VPITCH

  if ((int)blockIdx.x >= plan.units * plan.nsplit) return;
  const AttnUnit u = attn_unit(a, plan, QT);
  if (u.b < 0) return;
  const int G = a.Hq / a.Hkv;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const int nvec = u.nb * G;
  const int vq = u.t * QT + wave * 32 + lr;
  const bool qvalid = vq < nvec;
  const int vqc = qvalid ? vq : (nvec - 1);
  const int row = u.row_base + vqc / G;
  const int h = u.g * G + vqc % G;

  bf16x8 qf[NS];
  {
    const u16* qp = static_cast<const u16*>(a.q) + ((size_t)row * a.Hq + h) * HD + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
  }

  const int kbeg = u.split * plan.kps, kend = min(a.S, kbeg + plan.kps);
  // K/V of this (sequence, kv head) through buffer loads: key j at j*rowbytes
  // from the base; the resource ends after key S-1, so rows past the end of
  // the sequence read zeros (the whole offset sits in the VGPR)
  const uint32_t rowbytes = (uint32_t)a.Hkv * HD * 2;
  const size_t base_el = ((size_t)u.b * a.S * a.Hkv + u.g) * HD;
  const uint32_t nbytes = (uint32_t)(a.S - 1) * rowbytes + HD * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const u16*>(a.k) + base_el, nbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const u16*>(a.v) + base_el, nbytes);
  constexpr int RPJ = NT / CPR;        // key rows between a thread's chunks
  constexpr int JT = KT * CPR / NT;    // chunks per tensor per thread
  static_assert(2 * JT == CPT, "K and V chunks");
  const uint32_t voff = (uint32_t)(tid / CPR) * rowbytes + (tid % CPR) * 16;
  const float c = a.scale * kLog2e;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};

  // K/V tile loads: chunk j < JT of this thread is K row (tid/CPR + RPJ j),
  // 16-byte column tid%CPR; chunk JT + j the same V row.  Keys of the tile
  // past the split's end (but inside the sequence) are loaded and masked.
  u32x4 st[CPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const uint32_t o = voff + (uint32_t)(k0 + RPJ * j) * rowbytes;
      st[j] = buffer_load16(rk, o);
      st[JT + j] = buffer_load16(rv, o);
    }
  };
  // One K/V tile's scores, online softmax and P.V.  `masked` (a
  // std::integral_constant) compiles the key mask in for the last, partial tile.
  auto tile_math = [&](int nvalid, auto masked) {
    // with two 32-key blocks their MFMA chains alternate, so each MFMA issues
    // two slots after the one it depends on (a lone chain waits out its
    // latency; with one block per tile the third wave of the SIMD covers it)
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kf = as_bf16x8(
            *reinterpret_cast<const u32x4*>(sK + (32 * kb + lr) * PITCH + 16 * s + 8 * lg));
        sacc[kb] = mfma32x32x16(kf, qf[s], sacc[kb]);
      }
    }
    // keep four K-fragment reads in flight: 4 reads, then (MFMA, read)
    // pairs, then the last 4 MFMAs (left alone the scheduler issues each read
    // right before its MFMA and waits out the whole LDS latency 16 times)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NKB * NS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kb + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (key >= nvalid) sacc[kb][i] = -INFINITY;
        }
    }
    // Exponentials against the running reference m_run (log2 units), checked
    // afterwards.  fp32 sums and bf16 P keep the same relative precision at
    // any magnitude, so the reference only has to keep the numbers finite:
    // while a lane's tile sum stays <= kLaneSumCap every probability of the
    // tile is <= 2^64, and O and l stay far from the fp32 range even summed
    // over the whole sequence.  Otherwise (every split's first tile, where
    // m_run = -inf and the sums are inf or NaN, or a score far above the
    // reference) the wave takes the exact tile max, rescales O and l and redoes
    // the exponentials.  No max is computed on the common path.
    // The probabilities are rounded to bf16 pairs as they are produced (the
    // P.V operand), and the lane sum adds those pairs with v_dot2_f32_bf16
    // against (1, 1): 16 instructions for 32 values instead of 32 adds, and
    // the sum holds exactly the weights that P.V applies.
    u32x4 pw[NKB][2];
    auto tile_exp = [&]() {
      const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
      float lq[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums (short dependency chains)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][2 * j], c, -m_run));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][2 * j + 1], c, -m_run));
          const uint32_t w = pack_bf16x2(e0, e1);
          pw[kb][j >> 2][j & 3] = w;
          lq[j & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, lq[j & 3], false);
        }
      return (lq[0] + lq[1]) + (lq[2] + lq[3]);
    };
    float lt = tile_exp();
    if (__any(!(lt <= kLaneSumCap))) {
      // tile max: four independent partial maxima (short dependency chains),
      // then the lane pair that holds the other half of the query's keys
      float mq[4];
      constexpr int PER = 8 * NKB / 2;  // registers per partial maximum
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& sa = sacc[(j * PER) / 16];
        const int i0 = (j * PER) % 16;
        mq[j] = fmaxf(sa[i0], sa[i0 + 1]);
#pragma unroll
        for (int i = 2; i < PER; ++i) mq[j] = fmaxf(mq[j], sa[i0 + i]);
      }
      const float mt = pair_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
      // the first tile of a split always holds a valid key, so m_run leaves
      // -inf there (alpha = 0 on the empty sums)
      const float m_new = fmaxf(m_run, mt * c);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[d][i] *= alpha;
      m_run = m_new;
      lt = tile_exp();
    }
    l_run += lt;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) attn_pv_block<HD>(sV, 32 * kb, pw[kb], acc, lane);
  };

  if (kbeg < kend) load_tile(kbeg);

  // Stage tile k0 from registers into LDS and start loading the next one,
  // which streams in during this tile's math.
  auto stage = [&](int k0) {
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int r = tid / CPR + RPJ * j, ch = tid % CPR;
      *reinterpret_cast<u32x4*>(sK + r * PITCH + ch * 8) = st[j];
      *reinterpret_cast<u32x4*>(sV + r * VPITCH + ch * 8) = st[JT + j];
    }
    __syncthreads();
    if (k0 + KT < kend) load_tile(k0 + KT);
  };
  // Full tiles run a copy of the math without the key mask; the partial last
  // tile of the split (if any) runs the masked copy after the loop.
  int k0 = kbeg;
  for (; k0 + KT <= kend; k0 += KT) {
    stage(k0);
    tile_math(KT, std::false_type{});
  }
  if (k0 < kend) {
    stage(k0);
    tile_math(kend - k0, std::true_type{});
  }

  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  const float lse_nat = (m_run + __log2f(l_tot)) * kLn2;
  if (!qvalid) return;
#pragma unroll
  for (int d = 0; d < NDB; ++d) attn_store_block<HD>(a, plan, u.split, u.b, row, h, d, acc[d], inv, lg);
  if (lg == 0) attn_store_lse<HD>(a, plan, u.split, row, h, lse_nat);
}

// WQ = 1: 128 query vectors, two workgroups per CU (short selections, whose
// splits spread the K/V stream over the CUs, and GQA with 4 or more query
// heads per KV head); WQ = 2: 256 query vectors in eight waves, one workgroup
// per CU (MHA-like selections with many query tiles, where every tile of K/V
// is re-read by each query tile of its head from L2).  KT = 32: one 32-key
// block per tile, which needs 168 VGPRs instead of 221, so three workgroups
// share a CU (three waves per SIMD, from different workgroups); for the long
// GQA selections at head dim 128.
template <int HD, int WQ, int KT>
__global__ __launch_bounds__(256 * WQ, WQ == 2 ? 1 : (KT == 32 ? 3 : 2)) void attn_fwd_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) u16 smem[AttnLds<HD, KT>::WIDE];
  const AttnPlan plan = attn_plan(a, 128 * WQ);
  attn_body<HD, WQ, KT>(a, plan, smem);
}

// Combine split-KV partials: O = sum_s exp(lse_s - L) O_s with L = logsumexp_s lse_s.
// One wave per (row, head): lane s < nsplit reads split s's LSE, the weights are
// broadcast, and all splits' partial rows are loaded before any accumulation
// (NS2 = the split count rounded up to 2, 4, 8 or 16 slots, branch-free; unused
// slots re-read a valid split with weight 0).
// One (row, head) pair of the split-KV merge, in two phases so that a wave
// can issue the loads of several pairs before it waits for any of them.
template <int HD, int NS2>
struct MergeLoads {
  float ls;            // this lane's split LSE (lanes < nsplit)
  float v[NS2][HD / 64];  // this lane's output columns of every split slot
};

template <int HD, int NS2>
__device__ __forceinline__ void merge_load(const AttnArgs& a, const AttnPlan& plan, int pr, int lane,
                                           MergeLoads<HD, NS2>& m) {
  constexpr int E = HD / 64;
  const int nsplit = plan.nsplit;
  const size_t split_stride = (size_t)plan.n_rows * a.Hq;
  m.ls = lane < nsplit ? a.part_lse[lane * split_stride + pr] : -INFINITY;
#pragma unroll
  for (int s = 0; s < NS2; ++s) {
    const int sc = min(s, nsplit - 1);  // slots past nsplit get weight 0
    const float* po = a.part_o + (sc * split_stride + pr) * HD + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) m.v[s][e] = po[e];
  }
}

template <int HD, int NS2>
__device__ __forceinline__ void merge_finish(const AttnArgs& a, int pr, int lane,
                                             const MergeLoads<HD, NS2>& m, int nsplit) {
  constexpr int E = HD / 64;
  const float M = wave_max(m.ls);
  const float wl = lane < nsplit ? __expf(m.ls - M) : 0.f;
  const float tot = wave_sum(wl);
  const float L = M + __logf(tot);
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
#pragma unroll
  for (int s = 0; s < NS2; ++s) {
    const float w = __shfl(wl, s, 64) / tot;  // zero for slots past nsplit
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(w, m.v[s][e], o[e]);
  }
  const int row = pr / a.Hq, h = pr % a.Hq;
  u16* op = static_cast<u16*>(a.o) + (size_t)pr * HD + lane * E;
  u16* cp = nullptr;
  if (a.ctx_out) {
    const int b = batch_of(a.offsets, a.B, row);
    cp = static_cast<u16*>(a.ctx_out) + ((size_t)(b * a.S + a.idx[row]) * a.Hq + h) * HD + lane * E;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const u16 bv = f32_to_bf16(o[e]);
    op[e] = bv;
    if (cp) cp[e] = bv;
  }
  if (lane == 0 && a.lse) a.lse[pr] = L;
}

// A wave merges pairs pr and pr + stride together: both pairs' loads are in
// flight before either is combined.
template <int HD, int NS2>
__device__ __forceinline__ void merge_pairs(const AttnArgs& a, const AttnPlan& plan, int first,
                                            int stride, int pairs, int lane) {
  for (int pr = first; pr < pairs; pr += 2 * stride) {
    const int pr2 = pr + stride;
    MergeLoads<HD, NS2> m0, m1;
    merge_load<HD, NS2>(a, plan, pr, lane, m0);
    if (pr2 < pairs) merge_load<HD, NS2>(a, plan, pr2, lane, m1);
    merge_finish<HD, NS2>(a, pr, lane, m0, plan.nsplit);
    if (pr2 < pairs) merge_finish<HD, NS2>(a, pr2, lane, m1, plan.nsplit);
  }
}

template <int HD, int QT>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const AttnPlan plan = attn_plan(a, QT);
  if (plan.nsplit <= 1) return;  // the attention kernel already wrote the outputs
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pairs = plan.n_rows * a.Hq;
  const int first = blockIdx.x * 4 + wave, stride = gridDim.x * 4;
  // slices read per pair: the split count rounded up to a power of two
  if (plan.nsplit <= 2)
    merge_pairs<HD, 2>(a, plan, first, stride, pairs, lane);
  else if (plan.nsplit <= 4)
    merge_pairs<HD, 4>(a, plan, first, stride, pairs, lane);
  else if (plan.nsplit <= 8)
    merge_pairs<HD, 8>(a, plan, first, stride, pairs, lane);
  else
    merge_pairs<HD, 16>(a, plan, first, stride, pairs, lane);
}

template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(AttnArgs a) {
  __shared__ float sq[4][HD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pr = blockIdx.x * 4 + wave;
  const int n_rows = min(a.offsets[a.B], a.max_rows);
  const bool active = pr < n_rows * a.Hq;
  const int row = active ? pr / a.Hq : 0, h = active ? pr % a.Hq : 0;
  constexpr int E = HD / 64;
  if (active) {
    const float* q = static_cast<const float*>(a.q) + ((size_t)row * a.Hq + h) * HD;
#pragma unroll
    for (int e = 0; e < E; ++e) sq[wave][lane + 64 * e] = q[lane + 64 * e];
  }
  __syncthreads();
  if (!active) return;
  const int b = batch_of(a.offsets, a.B, row);
  const int g = h / (a.Hq / a.Hkv);
  const size_t kstride = (size_t)a.Hkv * HD;
  const float* kb = static_cast<const float*>(a.k) + ((size_t)b * a.S * a.Hkv + g) * HD;
  const float* vb = static_cast<const float*>(a.v) + ((size_t)b * a.S * a.Hkv + g) * HD;
  float m = -INFINITY, l = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int k0 = 0; k0 < a.S; k0 += 64) {
    const int key = k0 + lane;
    // HD = 64: this lane's V column over the whole tile is loaded together with
    // its K row, so the tile costs one memory round trip (rows past the
    // sequence re-read its last row, with p = 0)
    float vt[HD == 64 ? 64 : 1];
    if constexpr (HD == 64) {
#pragma unroll
      for (int j = 0; j < 64; ++j) vt[j] = vb[(size_t)min(k0 + j, a.S - 1) * kstride + lane];
    }
    float s = -INFINITY;
    if (key < a.S) {
      // the key row's float4 loads go out in groups of 8 before use; four
      // partial dot products
      const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)key * kstride);
      float dp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d0 = 0; d0 < HD / 4; d0 += 8) {
        float4 kv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) kv[u] = kr[d0 + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int d = d0 + u;
          float& dot = dp[u & 3];
          dot = fmaf(sq[wave][4 * d], kv[u].x, dot);
          dot = fmaf(sq[wave][4 * d + 1], kv[u].y, dot);
          dot = fmaf(sq[wave][4 * d + 2], kv[u].z, dot);
          dot = fmaf(sq[wave][4 * d + 3], kv[u].w, dot);
        }
      }
      s = ((dp[0] + dp[1]) + (dp[2] + dp[3])) * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = __expf(m - mn);
    const float p = key < a.S ? __expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
    // P.V over the tile's keys, 16 V rows loaded before they are used (rows
    // past the sequence re-read its last row, with p = 0)
    const int nk = min(64, a.S - k0);
    if constexpr (HD == 64) {
#pragma unroll
      for (int j = 0; j < 64; ++j) o[0] = fmaf(__shfl(p, j, 64), vt[j], o[0]);
    } else
    for (int j0 = 0; j0 < nk; j0 += 16) {
      float vv[16][E];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float* vr = vb + (size_t)min(k0 + j0 + u, a.S - 1) * kstride;
#pragma unroll
        for (int e = 0; e < E; ++e) vv[u][e] = vr[lane + 64 * e];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float pj = __shfl(p, j0 + u, 64);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = fmaf(pj, vv[u][e], o[e]);
      }
    }
    m = mn;
  }
  const float inv = 1.f / l;
  float* op = static_cast<float*>(a.o) + ((size_t)row * a.Hq + h) * HD;
  float* cp = a.ctx_out ? static_cast<float*>(a.ctx_out) +
                              ((size_t)(b * a.S + a.idx[row]) * a.Hq + h) * HD
                        : nullptr;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    op[lane + 64 * e] = o[e] * inv;
    if (cp) cp[lane + 64 * e] = o[e] * inv;
  }
  if (lane == 0 && a.lse) a.lse[(size_t)row * a.Hq + h] = m + __logf(l);
}

// ---------------------------------------------------------------------------
static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

size_t attn_workspace_bytes(int dtype, int max_rows, int B, int S, int Hq, int Hkv, int hd) {
  if (dtype != 1 || S < 2 * kMinSplitKeys) return 0;  // such sequences are never split
  return (size_t)kPartRows * (hd + 1) * sizeof(float);
}

// Split-KV partials of the allocation-free entry point: a file-scope device
// array of the largest workspace the attention ever asks for (head dim 128),
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in, not a device
// address); it looks up each device's address once with hipGetSymbolAddress
// and passes that.  The partials need no clearing: the merge pass reads only
// slots the attention kernel of the same call wrote.  Calls that overlap in
// time on one GPU share the array and race.
constexpr size_t kAttnScratchBytes = (size_t)kPartRows * (128 + 1) * sizeof(float);
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

size_t attn_scratch_bytes() { return kAttnScratchBytes; }

hipError_t attn_scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_attn(int dtype, const AttnArgs& a0, void* workspace, hipStream_t st) {
  if (a0.max_rows <= 0) return hipSuccess;
  AttnArgs a = a0;
  if (dtype == 0) {
    const int grid = (a.max_rows * a.Hq + 3) / 4;
    if (a.hd == 64)
      hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const int G = a.Hq / a.Hkv;
  const bool may_split = a.S >= 2 * kMinSplitKeys;
  a.part_o = may_split ? static_cast<float*>(workspace) : nullptr;
  a.part_lse = may_split ? a.part_o + (size_t)kPartRows * a.hd : nullptr;
  // A bound of fewer than kShortUnits 128-vector tiles (a short selection,
  // which the device may split along the keys): 128-vector workgroups.
  // Otherwise, with fewer than 4 query heads per KV head, 256-vector
  // workgroups, which halve the K/V re-reads.  With 4 or more the K/V bytes
  // per query are already a quarter of MHA's, and 128-vector workgroups (two
  // per CU, from different tiles, so the two waves of a SIMD are not held in
  // step by one workgroup's barriers; twice the tiles, so a step's last round
  // is less empty) run the GQA lock loop's steps as fast or faster (t = 32:
  // 338 -> 322 us, t = 56: 133 -> 112 us).
  auto max_units = [&](int QT) {
    return (ceil_div((long long)a.max_rows * G, QT) + a.B - 1) * (long long)a.Hkv;
  };
  const bool short_sel = may_split && max_units(128) < kShortUnits;
  const bool wide = G < 4 && !short_sel;
  const int QT = wide ? 256 : 128;
  // enough workgroups for every tile and for the split factor the device may
  // choose (split units fill at most one workgroup per CU)
  a.split_fill = device_cus();
  const int grid = (int)max_units(QT) + a.split_fill;
  const int threads = wide ? 512 : 256;
  // Long GQA selections at head dim 128 take 32-key tiles and three
  // workgroups per CU (same-process A/B on the lock loop, two rounds:
  // attention stage 20.58 / 20.72 -> 20.46 / 20.44 ms per loop); short
  // selections keep 64-key tiles (the lock loop's last step, 824 rows, took
  // 51 -> 57 us with 32-key tiles).
  if (a.hd == 64) {
    if (wide)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, 2, 64>), dim3(grid), dim3(threads), 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, 1, 64>), dim3(grid), dim3(threads), 0, st, a);
  } else {
    if (wide)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 2, 64>), dim3(grid), dim3(threads), 0, st, a);
    else if (short_sel)
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 1, 64>), dim3(grid), dim3(threads), 0, st, a);
    else
      hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, 1, 32>), dim3(grid), dim3(threads), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !may_split) return e;
  // the merge runs only when the device chose to split; otherwise it exits at once
  const long long quads = ((long long)a.max_rows * a.Hq + 3) / 4;
  const int mgrid = (int)(quads < kMergeGrid ? quads : kMergeGrid);
  if (a.hd == 64) {
    if (wide)
      hipLaunchKernelGGL((attn_merge_kernel<64, 256>), dim3(mgrid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_merge_kernel<64, 128>), dim3(mgrid), dim3(256), 0, st, a);
  } else {
    if (wide)
      hipLaunchKernelGGL((attn_merge_kernel<128, 256>), dim3(mgrid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((attn_merge_kernel<128, 128>), dim3(mgrid), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dlm
