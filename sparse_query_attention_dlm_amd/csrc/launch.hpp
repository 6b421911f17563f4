// Host-side launchers of the gfx950 kernels (internal to libdlm; the public
// surface is include/dlm.h).  Every launcher enqueues on `st`, performs no
// synchronisation and returns hipGetLastError() after its launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlm {

// CUs of the current device (queried once per device; 256 on MI355X)
inline int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// select.hip
hipError_t launch_cosine_select(int dtype, const void* cur, const void* prev, int B, int S, int D,
                                int lo, int hi, float thr, float* scores, int32_t* idx,
                                int32_t* counts, int32_t* offsets, hipStream_t st);
hipError_t launch_given_select(const float* scores, int B, int S, int lo, int hi, float thr,
                               int32_t* idx, int32_t* counts, int32_t* offsets, hipStream_t st);
hipError_t launch_lmhead_combine(const float4* part, int ntile, const int32_t* eval_idx,
                                 const int32_t* eval_offsets, int max_eval, int B, int S, int lo,
                                 int hi, float thr, int margin, float* scores, int32_t* argmax,
                                 int32_t* idx, int32_t* counts, int32_t* offsets, hipStream_t st);

// KL lock (select.hip): merge the EPI_LMKL tile partials into KL, max-prob and
// argmax of every evaluated position, then the per-sequence lock decision
hipError_t launch_kl_lock(const float4* part, int ntile, const int32_t* eval_idx,
                          const int32_t* eval_offsets, int max_eval, int B, int S, float eps,
                          float gate_q, float* kl, float* maxprob, int32_t* argmax, float* locked,
                          hipStream_t st);

// gemm.hip -- D^T[n][m] = sum_k W[n][k] * A[row(m)][k]; W output-major [N][K].
enum GemmEpilogue { EPI_QKV = 0, EPI_ROWS = 1, EPI_LMHEAD = 2, EPI_SWIGLU = 3, EPI_LMMARGIN = 4, EPI_LMKL = 5 };
// the LM-head epilogues (the margin one also keeps the second-largest logit;
// the KL one reduces the logits of two steps of each position, see below)
constexpr bool epi_lm(int epi) { return epi == EPI_LMHEAD || epi == EPI_LMMARGIN || epi == EPI_LMKL; }
// EPI_LMKL: every selected position contributes two token rows, its hidden
// state at this step (from x) and at the previous step (from x2), interleaved
// by 16: token row m is position (m/32)*16 + m%16, of this step when m%32 < 16.
// GEMM token rows for n selected positions:
constexpr int gemm_token_rows(int epi, int n) { return epi == EPI_LMKL ? ((n + 15) / 16) * 32 : n; }
enum GemmAMode { A_GATHER = 0, A_COMPACT = 1 };
struct GemmArgs {
  const void* w;            // [N][K]
  const void* x;            // A_GATHER: x[B][S][K], row (b, idx[m]); A_COMPACT: x[m][K]
  const void* x2;           // EPI_LMKL: the previous step's hidden states, laid out as x
  uint32_t x_bytes;         // size of x (and x2) (operand loads are range-checked against it)
  int K, N, B, S;
  const int32_t* idx;       // selected positions (packed)
  const int32_t* offsets;   // [B+1]
  int max_rows;
  // EPI_QKV: columns [0,nq) -> q_out[m][nq], [nq,nq+nk) -> k_cache row, then v_cache row
  void* q_out;
  void* k_cache;
  void* v_cache;
  int nq, nk;
  // EPI_ROWS: out[(b*S + idx[m])*ld_out + n]
  // EPI_SWIGLU: features (2f, 2f+1) = (gate, up) of f; out[m*ld_out + f] =
  //             silu(gate) * up
  void* out;
  int ld_out;
  // EPI_LMHEAD: lm_part[m*ntile + tile] = {max, sum exp(z-max), argmax bits, 0};
  // EPI_LMMARGIN: the same with the second-largest logit in the last slot;
  // EPI_LMKL: two per (position p, tile): lm_part[2(p*ntile + tile)] = {max,
  //   sum e, argmax bits, sum e * (z - z_prev)} of this step's logits z,
  //   lm_part[... + 1] = {max, sum exp(z_prev - max), 0, 0} of the previous step's
  float4* lm_part;
  int ntile;
  // split-K scratch (workspace): partial tiles
  float* part;
  // nonzero: the weight-streaming tiling (at most 128 rows) of a narrow
  // output (fewer than 128 tiles of 64 features) may split K over several
  // workgroups; part then holds gemm_skinny_split_bytes() of partial tiles
  int skinny_split;
  // set by the launcher: workgroups of the persistent grid (the split plan
  // fills its last round)
  int tile_grid;
};
size_t gemm_workspace_bytes(int epi, int max_rows, int N, int K);
size_t gemm_skinny_split_bytes(int max_rows, int N, int K);
hipError_t launch_gemm(int dtype, int epi, int amode, const GemmArgs& g, hipStream_t st);
int gemm_lmhead_ntile(int V);

// attn.hip
struct AttnArgs {
  const void* q;            // [max_rows][Hq][hd]
  const int32_t* idx;
  const int32_t* offsets;
  int max_rows;
  const void* k;            // [B][S][Hkv][hd]
  const void* v;
  int B, S, Hq, Hkv, hd;
  float scale;
  void* o;                  // [max_rows][Hq][hd]
  float* lse;               // [max_rows][Hq] or null
  void* ctx_out;            // out_cache [B][S][Hq*hd] or null (no W_o)
  float* part_o;            // split-KV partials (workspace)
  float* part_lse;
  int split_fill;           // set by the launcher: CUs of the device (the split plan fills them)
};
size_t attn_workspace_bytes(int dtype, int max_rows, int B, int S, int Hq, int Hkv, int hd);
hipError_t launch_attn(int dtype, const AttnArgs& a, void* workspace, hipStream_t st);
// the allocation-free variant's split-KV scratch: its size (every head dim)
// and this device's address of it (looked up once per device)
size_t attn_scratch_bytes();
hipError_t attn_scratch_ptr(void** out);
hipError_t launch_probe_mfma(int iters, int grid, float* sink, hipStream_t st);

// colsum.hip
size_t colsum_workspace_bytes(int B, int S, int Hkv);
hipError_t launch_colsum(const void* q, const int32_t* offsets, int max_rows, const void* k,
                         const float* lse, int B, int S, int Hq, int Hkv, int hd, float scale,
                         float* partial, float* colsum, int key_lo, int key_hi, int kk,
                         int32_t* topk_idx, float* topk_val, int window, hipStream_t st);

// dv.hip
struct DvArgs {
  const void* q;            // [B][S][Hq][hd] cached queries
  const float* lse;         // [B][S][Hq] cached natural-log LSE
  const int32_t* idx;       // salient positions
  const int32_t* offsets;
  int max_rows;
  const void* k_old;        // [n][Hkv][hd] salient K rows before the scatter
  const void* v_old;        // [n][Hkv][hd]
  const void* v;            // [B][S][Hkv][hd] V cache after the scatter
  int B, S, Hq, Hkv, hd;
  float scale;
  void* o;                  // [B][S][Hq][hd] context cache, updated in place
};
hipError_t launch_dv_update(int dtype, const DvArgs& a, hipStream_t st);
hipError_t launch_row_copy(const void* src, void* dst, const int32_t* idx, const int32_t* offsets,
                           int max_rows, int B, int S, int row_bytes, int scatter, hipStream_t st);

// validate.hip: the opt-in check of a selection's index arrays.  Runs one
// check kernel on `st`, waits for it and returns its verdict (0 = valid, else
// a mask of the flags below).
enum ValidateFlags {
  kBadFirstOffset = 1,    // offsets[0] != 0
  kOffsetsDecrease = 2,   // offsets[b+1] < offsets[b]
  kOffsetsPastBound = 4,  // offsets[B] > max_rows
  kIndexOutside = 8,      // a position outside [0, S)
  kIndexOrder = 16,       // positions of a batch row not strictly increasing
};
hipError_t validate_rows(const int32_t* idx, const int32_t* offsets, int B, int S, int max_rows,
                         int check_idx, hipStream_t st, int* verdict);

// prefix.hip
hipError_t launch_lsp_adaptive(const float* margin, int B, int S, int gen_lo, int gen_hi,
                               float frac_lo, float frac_hi, float margin_floor, int32_t* committed,
                               float* tau, hipStream_t st);
hipError_t launch_stable_prefix(const int32_t* argmax, const float* maxprob, int B, int S,
                                int gen_lo, int gen_hi, int32_t* ring, int W, int step, float thr,
                                int min_commit, int32_t* committed, hipStream_t st);

}  // namespace dlm
