// Bidirectional partial attention of the selected queries over all keys.
//
// DyLLM, Methodologie 2 (salient path): attention rows of the selected tokens
// are recomputed in full against every key; SureLock, Methodik,
// Kernprinzipien: active tokens attend to the cached K/V of locked tokens, so
// the cost is O(M N d) for M active rows.  No mask: the model is bidirectional.
//
// bf16 kernel (gfx950 matrix cores), flash-style online softmax:
//   * A workgroup owns 128 query vectors (row, head) that share one KV head of
//     one sequence (GQA packs the G query heads of a KV head together); each
//     wave owns 32 of them.
//   * Per 32-key tile, K and V are staged in LDS and every wave computes the
//     transposed score tile S^T = K . Q^T (32 keys x 32 queries) with eight
//     32x32x16 MFMAs; Q^T stays in registers for the whole key loop.
//   * In that layout a lane holds 16 keys of one query, so the running max and
//     sum are in-lane reductions plus one v_permlane32_swap with the lane that
//     holds the other 16 keys of the same query.
//   * P^T (bf16) is already in the B-operand layout of O^T = V^T . P^T; the
//     V^T operand is read with ds_read_b64_tr_b16, which transposes 4x16
//     blocks of V on the way out of LDS.
//   * Few queries (short selections): the key range is split over workgroups
//     and a merge pass combines the partial outputs by their LSE.
// fp32 kernel (small fp32 layers): one wave per (row, head), float32 FMA.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ i16x4 lds_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Work plan shared by the attention and merge kernels, computed on the device
// from the selection counts (the host only knows an upper bound):
//   units  = sum_b ceil(n_b * G / 128) query tiles, times Hkv
//   nsplit = 1 when units >= kSplitTarget, else ceil(kSplitTarget / units)
//            capped at 16 and at S/128, so short selections still fill the chip.
// With nsplit > 1, units < kSplitTarget implies nsplit * n_rows * Hq <=
// 2 * kSplitTarget * 128 = kPartRows, the bound the workspace is sized for.
constexpr int kSplitTarget = 512;
constexpr int kPartRows = 2 * kSplitTarget * 128;

constexpr int kAttnKT = 64;  // keys per K/V tile of the bf16 kernel

struct AttnPlan {
  int units;
  int nsplit;
  int kps;     // keys per split (a multiple of kAttnKT)
  int n_rows;
};

__device__ __forceinline__ AttnPlan attn_plan(const AttnArgs& a) {
  const int G = a.Hq / a.Hkv;
  int tiles = 0;
  for (int bb = 0; bb < a.B; ++bb) {
    const int n_b = min(a.offsets[bb + 1], a.max_rows) - min(a.offsets[bb], a.max_rows);
    tiles += (n_b * G + 127) / 128;
  }
  AttnPlan p;
  p.units = tiles * a.Hkv;
  p.n_rows = min(a.offsets[a.B], a.max_rows);
  int ns = 1;
  if (p.units > 0 && p.units < kSplitTarget) {
    ns = (kSplitTarget + p.units - 1) / p.units;
    ns = min(ns, 16);
    ns = min(ns, max(1, a.S / 128));
    if (p.n_rows > 0) ns = min(ns, max(1, kPartRows / (p.n_rows * a.Hq)));
  }
  // keys per split are rounded up to whole 64-key tiles; recount the splits
  // from that size so that none of them is empty
  p.kps = ((a.S + ns - 1) / ns + kAttnKT - 1) / kAttnKT * kAttnKT;
  p.nsplit = (a.S + p.kps - 1) / p.kps;
  return p;
}

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int QT = 128;        // query vectors per workgroup
  constexpr int KT = kAttnKT;    // keys per tile (two 32-key MFMA blocks)
  constexpr int PITCH = HD + 8;  // u16 per LDS row
  constexpr int NS = HD / 16;    // k-chunks of Q.K^T
  constexpr int NDB = HD / 32;   // 32-row blocks of O^T
  constexpr int CPR = HD / 8;    // 16-byte chunks per K/V row
  constexpr int CPT = 2 * KT * CPR / 256;
  __shared__ __attribute__((aligned(16))) u16 sK[KT * PITCH];
  __shared__ __attribute__((aligned(16))) u16 sV[KT * PITCH];

  const AttnPlan plan = attn_plan(a);
  const int nsplit = plan.nsplit;
  if ((int)blockIdx.x >= plan.units * nsplit) return;
  const int split = blockIdx.x % nsplit;
  const int rest = blockIdx.x / nsplit;
  const int g = rest % a.Hkv;
  int t = rest / a.Hkv;
  const int G = a.Hq / a.Hkv;
  int b = -1, nb = 0, row_base = 0;
  for (int bb = 0; bb < a.B; ++bb) {
    const int lo_b = min(a.offsets[bb], a.max_rows), hi_b = min(a.offsets[bb + 1], a.max_rows);
    const int n_b = hi_b - lo_b;
    const int tb = (n_b * G + QT - 1) / QT;
    if (t < tb) {
      b = bb;
      nb = n_b;
      row_base = lo_b;
      break;
    }
    t -= tb;
  }
  if (b < 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const int nvec = nb * G;
  const int vq = t * QT + wave * 32 + lr;
  const bool qvalid = vq < nvec;
  const int vqc = qvalid ? vq : (nvec - 1);
  const int row = row_base + vqc / G;
  const int h = g * G + vqc % G;

  bf16x8 qf[NS];
  {
    const u16* qp = static_cast<const u16*>(a.q) + ((size_t)row * a.Hq + h) * HD + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
  }

  const int kbeg = split * plan.kps, kend = min(a.S, kbeg + plan.kps);
  const size_t kstride = (size_t)a.Hkv * HD;
  const u16* kbase = static_cast<const u16*>(a.k) + ((size_t)b * a.S * a.Hkv + g) * HD;
  const u16* vbase = static_cast<const u16*>(a.v) + ((size_t)b * a.S * a.Hkv + g) * HD;
  const float c = a.scale * kLog2e;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};

  const int g16 = lane >> 4, j16 = lane & 15, ga = g16 >> 1;

  // K/V tile loads: chunk j of this thread is (tensor, key row, 16-byte column)
  u32x4 st[CPT];
  auto load_tile = [&](int k0) {
    const int nvalid = min(KT, kend - k0);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = tid + 256 * j;
      const int tensor = cidx / (KT * CPR), rem = cidx % (KT * CPR);
      const int r = rem / CPR, ch = rem % CPR;
      if (r < nvalid)
        st[j] = *reinterpret_cast<const u32x4*>((tensor ? vbase : kbase) + (size_t)(k0 + r) * kstride + ch * 8);
      else
        st[j] = u32x4{0, 0, 0, 0};
    }
  };
  if (kbeg < kend) load_tile(kbeg);

  for (int k0 = kbeg; k0 < kend; k0 += KT) {
    const int nvalid = min(KT, kend - k0);
    __syncthreads();  // every wave is done reading the previous tile
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int cidx = tid + 256 * j;
      const int tensor = cidx / (KT * CPR), rem = cidx % (KT * CPR);
      const int r = rem / CPR, ch = rem % CPR;
      *reinterpret_cast<u32x4*>((tensor ? sV : sK) + r * PITCH + ch * 8) = st[j];
    }
    __syncthreads();
    if (k0 + KT < kend) load_tile(k0 + KT);  // next tile streams in during this tile's math

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 kf = as_bf16x8(
            *reinterpret_cast<const u32x4*>(sK + (32 * kb + lr) * PITCH + 16 * s + 8 * lg));
        sacc[kb] = mfma32x32x16(kf, qf[s], sacc[kb]);
      }
    }
    if (nvalid < KT) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kb + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (key >= nvalid) sacc[kb][i] = -INFINITY;
        }
    }
    float mt = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = pair_max(mt);
    const float m_new = fmaxf(m_run, mt * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[2][16];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, -m_new));
        ls += p[kb][i];
      }
    l_run = fmaf(l_run, alpha, ls);
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][i] *= alpha;
    m_run = m_new;

    // P^T in B-operand layout: register i of key block kb is key 32kb+8(i/4)+4*lg+(i%4)
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 w0, w1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0[j] = pack_bf16x2(p[kb][2 * j], p[kb][2 * j + 1]);
        w1[j] = pack_bf16x2(p[kb][8 + 2 * j], p[kb][8 + 2 * j + 1]);
      }
      pb[kb][0] = as_bf16x8(w0);
      pb[kb][1] = as_bf16x8(w1);
    }
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int m0 = 32 * d + 16 * (g16 & 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          // k-slots 8*ga+0..3 <-> keys 16cc+4ga+0..3, slots 8*ga+4..7 <-> keys 16cc+8+4ga+0..3
          const u16* pa = sV + (32 * kb + 16 * cc + 4 * ga + (j16 >> 2)) * PITCH + m0 + 4 * (j16 & 3);
          const i16x4 va = lds_read_tr16(pa);
          const i16x4 vb = lds_read_tr16(pa + 8 * PITCH);
          const bf16x8 av =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[d] = mfma32x32x16(av, pb[kb][cc], acc[d]);
        }
    }
  }

  const float l_tot = pair_sum(l_run);
  const float inv = 1.f / l_tot;
  const float lse_nat = (m_run + __log2f(l_tot)) * kLn2;
  if (!qvalid) return;
  if (nsplit == 1) {
    u16* op = static_cast<u16*>(a.o) + ((size_t)row * a.Hq + h) * HD;
    u16* cp = a.ctx_out ? static_cast<u16*>(a.ctx_out) +
                              ((size_t)(b * a.S + a.idx[row]) * a.Hq + h) * HD
                        : nullptr;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * d + 8 * q4 + 4 * lg;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[d][4 * q4] * inv, acc[d][4 * q4 + 1] * inv);
        pk[1] = pack_bf16x2(acc[d][4 * q4 + 2] * inv, acc[d][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = pk;
        if (cp) *reinterpret_cast<u32x2*>(cp + d0) = pk;
      }
    if (lg == 0 && a.lse) a.lse[(size_t)row * a.Hq + h] = lse_nat;
  } else {
    float* po = a.part_o + (((size_t)split * plan.n_rows + row) * a.Hq + h) * HD;
#pragma unroll
    for (int d = 0; d < NDB; ++d)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * d + 8 * q4 + 4 * lg;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(acc[d][4 * q4] * inv, acc[d][4 * q4 + 1] * inv, acc[d][4 * q4 + 2] * inv,
                        acc[d][4 * q4 + 3] * inv);
      }
    if (lg == 0) a.part_lse[((size_t)split * plan.n_rows + row) * a.Hq + h] = lse_nat;
  }
}

// Combine split-KV partials: O = sum_s exp(lse_s - L) O_s with L = logsumexp_s lse_s.
// One wave per (row, head): lane s < nsplit reads split s's LSE, the weights are
// broadcast, and all splits' partial rows are loaded before any accumulation
// (NS2 = 8 or 16 slots, branch-free; unused slots re-read a valid split with
// weight 0).
template <int HD, int NS2>
__device__ __forceinline__ void merge_row(const AttnArgs& a, const AttnPlan& plan, int pr, int lane) {
  constexpr int E = HD / 64;
  const int nsplit = plan.nsplit;
  const size_t split_stride = (size_t)plan.n_rows * a.Hq;
  const float ls = lane < nsplit ? a.part_lse[lane * split_stride + pr] : -INFINITY;
  const float M = wave_max(ls);
  const float wl = lane < nsplit ? __expf(ls - M) : 0.f;
  const float tot = wave_sum(wl);
  const float L = M + __logf(tot);
  float v[NS2][E];
#pragma unroll
  for (int s = 0; s < NS2; ++s) {
    const int sc = min(s, nsplit - 1);
    const float* po = a.part_o + (sc * split_stride + pr) * HD + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) v[s][e] = po[e];
  }
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
#pragma unroll
  for (int s = 0; s < NS2; ++s) {
    const float w = __shfl(wl, s, 64) / tot;  // zero for slots past nsplit
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(w, v[s][e], o[e]);
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

template <int HD>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const AttnPlan plan = attn_plan(a);
  if (plan.nsplit <= 1) return;  // the attention kernel already wrote the outputs
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pr = blockIdx.x * 4 + wave;
  if (pr >= plan.n_rows * a.Hq) return;
  if (plan.nsplit <= 8)
    merge_row<HD, 8>(a, plan, pr, lane);
  else
    merge_row<HD, 16>(a, plan, pr, lane);
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
    float s = -INFINITY;
    if (key < a.S) {
      const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)key * kstride);
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < HD / 4; ++d) {
        const float4 kv = kr[d];
        dot = fmaf(sq[wave][4 * d], kv.x, dot);
        dot = fmaf(sq[wave][4 * d + 1], kv.y, dot);
        dot = fmaf(sq[wave][4 * d + 2], kv.z, dot);
        dot = fmaf(sq[wave][4 * d + 3], kv.w, dot);
      }
      s = dot * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = __expf(m - mn);
    const float p = key < a.S ? __expf(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
    const int nk = min(64, a.S - k0);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j, 64);
      const float* vr = vb + (size_t)(k0 + j) * kstride;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pj, vr[lane + 64 * e], o[e]);
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
static int attn_tiles_max(int max_rows, int B, int G) { return (max_rows * G + 127) / 128 + B - 1; }

size_t attn_workspace_bytes(int dtype, int max_rows, int B, int S, int Hq, int Hkv, int hd) {
  if (dtype != 1) return 0;
  return (size_t)kPartRows * (hd + 1) * sizeof(float);
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
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)kPartRows * a.hd;
  // enough workgroups for every tile and for the split factor the device may choose
  const int grid = attn_tiles_max(a.max_rows, a.B, G) * a.Hkv + 2 * kSplitTarget;
  if (a.hd == 64)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, dim3(grid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, dim3(grid), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the merge runs only when the device chose to split; otherwise it exits at once
  const long long pairs = (long long)a.max_rows * a.Hq;
  const long long cap = (long long)kPartRows;
  const int mgrid = (int)(((pairs < cap ? pairs : cap) + 3) / 4);
  if (a.hd == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(mgrid), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(mgrid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dlm
