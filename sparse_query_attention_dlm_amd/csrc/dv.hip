// Non-salient rows: the value-change update of their cached attention outputs,
// and the row gather/scatter that keeps the caches it reads.
//
// DyLLM, Methodologie 2 (non-salient path): for a stable token the attention
// weights are taken as unchanged, and its output moves only by the salient
// tokens' value change times its existing weights, at cost O(N |A|):
//   o[b,i,h] += sum_{j in A_b} exp(scale q[b,i,h] . k_old[j,g] - lse[b,i,h])
//                              (v[b,idx[j],g] - v_old[j,g]),   g = h / (Hq/Hkv)
// for every position i not in A_b; salient rows are not touched (the salient
// path recomputes them).  The weights are token i's softmax weights of its last
// computation: its cached query and natural-log LSE and the salient rows' K
// from before this step's scatter.
//
// bf16 kernel (gfx950 matrix cores), a skinny attention without a running max
// (the cached LSE bounds every weight by about 1):
//   * A workgroup of four (eight) waves owns 128 (256) query vectors:
//     consecutive stable positions of one sequence (the salient ones are
//     skipped: the salient path recomputes them) times the G query heads of
//     one KV head (vector v = stable rank * G + head-in-group); each wave
//     owns 32 and finds its positions from the salient list itself.
//   * Per 64-row tile of the salient set, K_old rows and the value change
//     dV = v_new - v_old (rounded to bf16) are staged in LDS; S^T = K . Q^T and
//     dO^T = dV^T . P^T run on 32x32x16 MFMAs in the layouts of the attention
//     kernel (P^T is the B operand, dV^T comes from transposed LDS reads).
//   * The epilogue adds dO to the cached output of every vector's position.
// fp32 kernel (small fp32 layers): one wave per (position, head), float32 FMA.
#include "common.hpp"
#include "launch.hpp"

namespace dlm {

typedef __attribute__((address_space(3))) i16x4 dv_lds_i16x4;

__device__ __forceinline__ i16x4 dv_read_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((dv_lds_i16x4*)(p));
}

constexpr int kDvKT = 64;   // salient rows per tile

// Work units are (sequence, KV head, tile of stable vectors), tiles fastest;
// the units of one (sequence, KV head) all stream the same salient K_old,
// V_old and new V rows.  The hardware deals a launch's workgroups round-robin
// to the 8 XCDs, each with its own L2, so workgroup b takes unit
// dv_xcd_unit(b, n) instead of unit b: each XCD then runs a contiguous range of
// units and fetches a (sequence, KV head)'s rows into its L2 once.  A bijection
// of [0, n).  Measured at B = 8, S = 2048, 32 / 8 heads, 1024 salient rows:
// 478 -> 272 us (with the round-robin order the stable-only tiles spread every
// XCD's resident units over twice the row sets its L2 holds).
__device__ __forceinline__ int dv_xcd_unit(int b, int n) {
  const int x = b & 7, a = n >> 3, c = n & 7;
  return x * a + min(x, c) + (b >> 3);
}

// Row pitches (u16) for conflict-free LDS reads, as in the attention kernel:
// K rows are 16-byte A-fragments read by 16 lanes on 16 consecutive rows
// (pitch HD + 8); dV rows are read transposed by 32 lanes on 4 consecutive
// rows (pitch HD + 32 puts consecutive rows 16 banks apart).
template <int HD>
struct DvLds {
  static constexpr int KPITCH = HD + 8;
  static constexpr int VPITCH = HD + 32;
  static constexpr int WORDS = kDvKT * (KPITCH + VPITCH);
};

// WQ = 1: 128 query vectors in four waves, two workgroups per CU; WQ = 2: 256
// vectors in eight waves, one per CU, for selections with many position tiles
// (every salient tile is read from L2 once per 256 vectors instead of 128).
template <int HD, int WQ>
__global__ __launch_bounds__(256 * WQ, WQ == 1 ? 2 : 1) void dv_update_bf16_kernel(DvArgs a) {
  constexpr int QT = 128 * WQ, NT = 256 * WQ;
  constexpr int NS = HD / 16, NDB = HD / 32, CPR = HD / 8;
  constexpr int PITCH = DvLds<HD>::KPITCH, VPITCH = DvLds<HD>::VPITCH;
  constexpr int RPJ = NT / CPR;        // tile rows between a thread's chunks
  constexpr int JT = kDvKT * CPR / NT; // chunks per tensor per thread
  __shared__ __attribute__((aligned(16))) u16 smem[DvLds<HD>::WORDS];
  u16* sK = smem;
  u16* sV = smem + kDvKT * PITCH;

  const int G = a.Hq / a.Hkv;
  const int tiles = (a.S * G + QT - 1) / QT;
  const int unit = dv_xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int t = unit % tiles;
  const int g = (unit / tiles) % a.Hkv;
  const int b = unit / (tiles * a.Hkv);
  const int r0 = min(a.offsets[b], a.max_rows), r1 = min(a.offsets[b + 1], a.max_rows);
  const int nb = r1 - r0;
  if (nb <= 0) return;  // no salient rows: every output stays
  const int nstable = a.S - nb;  // positions outside the salient set
  if ((long long)t * QT >= (long long)nstable * G) return;  // this tile holds no stable position

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const u16* kold = static_cast<const u16*>(a.k_old);
  const u16* vold = static_cast<const u16*>(a.v_old);
  const u16* vcache = static_cast<const u16*>(a.v);
  const int ch = tid % CPR;
  // The first salient tiles' loads go out before the positions of this
  // workgroup's vectors are searched (they do not depend on them).
  // staging registers of one tile: chunk ch of tile rows tid / CPR + RPJ j
  // (rows past the salient set give zeros).  A row's new V
  // sits at its position idx[r]: the positions are loaded one tile ahead of
  // the rows, so no tile waits for two memory round trips in a row.
  u32x4 kr[JT], vn[JT], vo[JT];
  int pnext[JT];
  // branch-free: a row past the salient set reads the set's first row and is
  // then zeroed
  auto row_of = [&](int k0, int j) {
    const int rr = k0 + tid / CPR + RPJ * j;
    return r0 + (rr < nb ? rr : 0);
  };
  auto load_pos = [&](int k0, int (&ps)[JT]) {
#pragma unroll
    for (int j = 0; j < JT; ++j) ps[j] = a.idx[row_of(k0, j)];
  };
  auto load_tile = [&](int k0, const int (&ps)[JT]) {
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const bool ok = k0 + tid / CPR + RPJ * j < nb;
      const size_t r = (size_t)row_of(k0, j);
      const u32x4 k = *reinterpret_cast<const u32x4*>(kold + (r * a.Hkv + g) * HD + ch * 8);
      const u32x4 o = *reinterpret_cast<const u32x4*>(vold + (r * a.Hkv + g) * HD + ch * 8);
      const u32x4 n = *reinterpret_cast<const u32x4*>(vcache + (((size_t)b * a.S + ps[j]) * a.Hkv + g) * HD + ch * 8);
      const u32x4 z = u32x4{0, 0, 0, 0};
      kr[j] = ok ? k : z;
      vo[j] = ok ? o : z;
      vn[j] = ok ? n : z;
    }
  };
  {
    int p0[JT];
    load_pos(0, p0);
    load_tile(0, p0);
  }
  if (kDvKT < nb) load_pos(kDvKT, pnext);

  // Vector v is (stable rank v / G, head v % G of the group).  Stable rank r
  // sits at position r + J(r), J(r) = #{j : f(j) <= r} with f(j) = idx[j] - j,
  // the number of stable positions before salient row j (non-decreasing along
  // the ascending positions).  J <= nb and r < nstable keep every position
  // inside the sequence whatever the index list holds.
  const int vq = t * QT + wave * 32 + lr;
  const bool qvalid = vq < nstable * G;
  const int vqc = qvalid ? vq : nstable * G - 1;
  const int rank = vqc / G, h = g * G + vqc % G;
  const int rw0 = min(t * QT + wave * 32, nstable * G - 1) / G;       // the wave's ranks
  const int rw1 = min(t * QT + wave * 32 + 31, nstable * G - 1) / G;
  const int32_t* sidx = a.idx + r0;
  // Skip the salient rows before the wave's first rank by a 64-way search
  // (each lane probes one point of the interval, a ballot counts the probes
  // with f <= rw0: a prefix of the lanes) until one 64-entry window is left:
  // every row below lo then has f <= rw0.
  int lo = 0, hi = nb;
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) >> 6;
    const int j = lo + lane * step;
    const int cnt_le = __popcll(__ballot(j < hi && sidx[min(j, nb - 1)] - j <= rw0));
    if (cnt_le == 0) break;  // f(lo) > rw0 already
    hi = min(hi, lo + cnt_le * step);
    lo += (cnt_le - 1) * step + 1;
  }
  // J(rank) - lo for each lane's rank from 64-entry windows of the salient list
  // from lo on, one ballot per rank of the wave (at most 32 of them)
  int extra = 0;
  for (int base = lo; base < nb; base += 64) {
    const int k = base + lane;
    const int fk = k < nb ? sidx[k] - k : 0x7fffffff;
    bool full = false;
    for (int rr = rw0; rr <= rw1; ++rr) {
      const unsigned long long m = __ballot(fk <= rr);
      if (rank == rr) extra += __popcll(m);
      if (rr == rw1) full = m == ~0ull;
    }
    if (!full) break;  // the window reaches past the wave's last rank
  }
  const int pos = rank + lo + extra;

  const size_t qrow = ((size_t)b * a.S + pos) * a.Hq + h;
  bf16x8 qf[NS];
  {
    const u16* qp = static_cast<const u16*>(a.q) + qrow * HD + lg * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * s));
  }
  const float c = a.scale * kLog2e;
  const float l2 = a.lse[qrow] * kLog2e;

  f32x16 acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) acc[d] = f32x16{};

  // One tile of the salient set.  `masked` (a std::integral_constant)
  // compiles the zero weights of rows past the salient set in, for the
  // partial last tile only: full tiles skip the ~64 compares and selects.
  auto tile = [&](int k0, auto masked) {
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int rl = tid / CPR + RPJ * j;
      float fn[8], fo[8];
      unpack8(vn[j], fn);
      unpack8(vo[j], fo);
      u32x4 dv;
#pragma unroll
      for (int e = 0; e < 4; ++e) dv[e] = pack_bf16x2(fn[2 * e] - fo[2 * e], fn[2 * e + 1] - fo[2 * e + 1]);
      *reinterpret_cast<u32x4*>(sK + rl * PITCH + ch * 8) = kr[j];
      *reinterpret_cast<u32x4*>(sV + rl * VPITCH + ch * 8) = dv;
    }
    __syncthreads();
    // the next tile streams in during this tile's math, and the positions of
    // the one after it
    if (k0 + kDvKT < nb) load_tile(k0 + kDvKT, pnext);
    if (k0 + 2 * kDvKT < nb) load_pos(k0 + 2 * kDvKT, pnext);

    // S^T = K_old . Q^T for the tile's two 32-row blocks
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(sK + (32 * kb + lr) * PITCH + 16 * s + 8 * lg));
        sacc[kb] = mfma32x32x16(kf, qf[s], sacc[kb]);
      }
    // four K-fragment reads kept in flight: 4 reads, then (MFMA, read) pairs,
    // then the last 4 MFMAs (left alone, the scheduler issues each read right
    // before its MFMA and waits out the LDS latency every time)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * NS - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // weights against the cached LSE; register i of block kb is tile row
    // 32 kb + 8 (i / 4) + 4 lg + i % 4; rows past the salient set weigh 0
    const int nvalid = nb - k0;
    u32x4 pw[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * j + u;
          e[u] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, -l2));
          if constexpr (decltype(masked)::value) {
            const int key = 32 * kb + 8 * (i >> 2) + 4 * lg + (i & 3);
            if (key >= nvalid) e[u] = 0.f;
          }
        }
        pw[kb][j >> 2][j & 3] = pack_bf16x2(e[0], e[1]);
      }
    // dO^T += dV^T . P^T (the V^T operand read as in the attention kernel)
    const int g16 = lane >> 4, j16 = lane & 15, ga = g16 >> 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        const int m0 = 32 * d + 16 * (g16 & 1);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const u16* pa = sV + (32 * kb + 16 * cc + 4 * ga + (j16 >> 2)) * VPITCH + m0 + 4 * (j16 & 3);
          const i16x4 va = dv_read_tr16(pa);
          const i16x4 vb = dv_read_tr16(pa + 8 * VPITCH);
          const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[d] = mfma32x32x16(av, as_bf16x8(pw[kb][cc]), acc[d]);
        }
      }
  };
  int k0 = 0;
  for (; k0 + kDvKT <= nb; k0 += kDvKT) tile(k0, std::false_type{});
  if (k0 < nb) tile(k0, std::true_type{});
  if (!qvalid) return;
  // o += dO: register i of block d holds dimension 32 d + 8 (i / 4) + 4 lg + i % 4
  u16* op = static_cast<u16*>(a.o) + qrow * HD;
  u32x2 oin[NDB][4];  // all of the lane's cached output words in flight at once
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) oin[d][q4] = *reinterpret_cast<const u32x2*>(op + 32 * d + 8 * q4 + 4 * lg);
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * d + 8 * q4 + 4 * lg;
      u32x2 w = oin[d][q4];
      const float o0 = __uint_as_float(w[0] << 16) + acc[d][4 * q4];
      const float o1 = __uint_as_float(w[0] & 0xFFFF0000u) + acc[d][4 * q4 + 1];
      const float o2 = __uint_as_float(w[1] << 16) + acc[d][4 * q4 + 2];
      const float o3 = __uint_as_float(w[1] & 0xFFFF0000u) + acc[d][4 * q4 + 3];
      w[0] = pack_bf16x2(o0, o1);
      w[1] = pack_bf16x2(o2, o3);
      *reinterpret_cast<u32x2*>(op + d0) = w;
    }
}

// fp32: one wave per (position, head); lane e-slices of the head dimension.
template <int HD>
__global__ __launch_bounds__(256) void dv_update_f32_kernel(DvArgs a) {
  constexpr int E = HD / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long pr = (long long)blockIdx.x * 4 + wave;  // (b, pos, h) flattened
  if (pr >= (long long)a.B * a.S * a.Hq) return;
  const int h = (int)(pr % a.Hq);
  const int pos = (int)((pr / a.Hq) % a.S);
  const int b = (int)(pr / ((long long)a.Hq * a.S));
  const int r0 = min(a.offsets[b], a.max_rows), r1 = min(a.offsets[b + 1], a.max_rows);
  if (r1 <= r0) return;
  // salient positions are left alone (idx ascending per batch row)
  int lo = r0, hi = r1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a.idx[mid] < pos) lo = mid + 1; else hi = mid;
  }
  if (lo < r1 && a.idx[lo] == pos) return;
  const int g = h / (a.Hq / a.Hkv);
  const float* q = static_cast<const float*>(a.q) + (((size_t)b * a.S + pos) * a.Hq + h) * HD;
  float qv[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    qv[e] = q[lane + 64 * e];
    o[e] = 0.f;
  }
  const float lse = a.lse[((size_t)b * a.S + pos) * a.Hq + h];
  const float* ko = static_cast<const float*>(a.k_old);
  const float* vo = static_cast<const float*>(a.v_old);
  const float* vc = static_cast<const float*>(a.v);
  for (int r = r0; r < r1; ++r) {
    const float* kr = ko + ((size_t)r * a.Hkv + g) * HD;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(qv[e], kr[lane + 64 * e], s);
    const float p = __expf(wave_sum(s) * a.scale - lse);
    const float* vn = vc + (((size_t)b * a.S + a.idx[r]) * a.Hkv + g) * HD;
    const float* vr = vo + ((size_t)r * a.Hkv + g) * HD;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmaf(p, vn[lane + 64 * e] - vr[lane + 64 * e], o[e]);
  }
  float* op = static_cast<float*>(a.o) + (((size_t)b * a.S + pos) * a.Hq + h) * HD;
#pragma unroll
  for (int e = 0; e < E; ++e) op[lane + 64 * e] += o[e];
}

// Row gather (rows[r] = cache[b, idx[r]]) or scatter (cache[b, idx[r]] =
// rows[r]) of row_bytes per row, one workgroup per selected row (grid-stride
// past 16384 rows, so every row's position lookup starts at once); T is the
// copy unit (16 or 4 bytes).  Loads and stores are non-temporal: each byte is
// touched once, and the streamed rows do not evict what the next kernel reads
// from the caches.
template <typename T>
__global__ __launch_bounds__(256) void row_copy_kernel(const char* src, char* dst, const int32_t* idx,
                                                       const int32_t* offsets, int max_rows, int B,
                                                       int S, int row_bytes, int scatter) {
  const int n = min(offsets[B], max_rows);
  const int units = row_bytes / (int)sizeof(T);
  for (int r = blockIdx.x; r < n; r += gridDim.x) {
    const int b = batch_of(offsets, B, r);
    const size_t cache_row = (size_t)b * S + idx[r];
    const T* __restrict__ s = reinterpret_cast<const T*>(src + (scatter ? (size_t)r : cache_row) * row_bytes);
    T* __restrict__ d = reinterpret_cast<T*>(dst + (scatter ? cache_row : (size_t)r) * row_bytes);
    // up to four units per thread loaded before any is stored, so their
    // loads are in flight together
    for (int u0 = threadIdx.x; u0 < units; u0 += 4 * 256) {
      T v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (u0 + 256 * k < units) v[k] = __builtin_nontemporal_load(s + u0 + 256 * k);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (u0 + 256 * k < units) __builtin_nontemporal_store(v[k], d + u0 + 256 * k);
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_dv_update(int dtype, const DvArgs& a, hipStream_t st) {
  if (a.max_rows <= 0) return hipSuccess;
  if (dtype == 0) {
    const long long pairs = (long long)a.B * a.S * a.Hq;
    const int grid = (int)((pairs + 3) / 4);
    if (a.hd == 64)
      hipLaunchKernelGGL(dv_update_f32_kernel<64>, dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(dv_update_f32_kernel<128>, dim3(grid), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // 256-vector workgroups once they still give two workgroups per CU, unless
  // 4 or more query heads share a KV head: then the salient rows' bytes per
  // query are a quarter of MHA's and 128-vector workgroups (several per CU,
  // from different position tiles) run faster (B = 8, S = 2048, 32 / 8 heads,
  // 1024 salient rows per sequence: 252 -> 242 us, same-process A/B)
  const int G = a.Hq / a.Hkv;
  const long long wide_grid = ((long long)a.S * G + 255) / 256 * a.Hkv * a.B;
  const bool wide = wide_grid >= 2LL * device_cus() && G < 4;
  const int QT = wide ? 256 : 128;
  const int grid = (int)(((long long)a.S * G + QT - 1) / QT * a.Hkv * a.B);
  const dim3 block(wide ? 512 : 256);
  if (a.hd == 64) {
    if (wide)
      hipLaunchKernelGGL((dv_update_bf16_kernel<64, 2>), dim3(grid), block, 0, st, a);
    else
      hipLaunchKernelGGL((dv_update_bf16_kernel<64, 1>), dim3(grid), block, 0, st, a);
  } else {
    if (wide)
      hipLaunchKernelGGL((dv_update_bf16_kernel<128, 2>), dim3(grid), block, 0, st, a);
    else
      hipLaunchKernelGGL((dv_update_bf16_kernel<128, 1>), dim3(grid), block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_row_copy(const void* src, void* dst, const int32_t* idx, const int32_t* offsets,
                           int max_rows, int B, int S, int row_bytes, int scatter, hipStream_t st) {
  if (max_rows <= 0) return hipSuccess;
  const int grid = max_rows < 16384 ? max_rows : 16384;
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  if (row_bytes % 16 == 0)
    hipLaunchKernelGGL(row_copy_kernel<u32x4>, dim3(grid), dim3(256), 0, st, s, d, idx, offsets, max_rows,
                       B, S, row_bytes, scatter);
  else
    hipLaunchKernelGGL(row_copy_kernel<uint32_t>, dim3(grid), dim3(256), 0, st, s, d, idx, offsets,
                       max_rows, B, S, row_bytes, scatter);
  return hipGetLastError();
}

}  // namespace dlm
