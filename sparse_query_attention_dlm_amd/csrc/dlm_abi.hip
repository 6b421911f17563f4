// C ABI of libdlm (declared in include/dlm.h): host-side argument validation
// and dispatch to the gfx950 kernels.  Validation runs before any HIP call, so
// a rejected request enqueues nothing and works without a GPU present.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "../../include/dlm.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DLM_OK;
  return fail(DLM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
size_t elt(int dtype) { return dtype == DLM_BF16 ? 2 : 4; }

#define REQUIRE(cond, ...)                                  \
  do {                                                      \
    if (!(cond)) return fail(DLM_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)
#define REQUIRE_PTR(p) REQUIRE((p) != nullptr, "%s must not be NULL", #p)
#define REQUIRE_ALIGNED(p) REQUIRE(aligned16(p), "%s must be 16-byte aligned", #p)

constexpr size_t kSelectTicketBytes = 256;

// DLM_VALIDATE=1 in the environment (read at every call): the calls that take
// a selection check its index arrays on the device before any other launch
// (and wait for the verdict).  Off by default: the arrays are trusted.
bool validate_on() {
  const char* v = std::getenv("DLM_VALIDATE");
  return v != nullptr && v[0] == '1' && v[1] == '\0';
}

int check_rows(const int32_t* idx, const int32_t* offsets, int B, int S, int max_rows, bool check_idx,
               void* stream, const char* what) {
  if (max_rows <= 0 || !validate_on()) return DLM_OK;
  int verdict = 0;
  if (hipError_t e = dlm::validate_rows(idx, offsets, B, S, max_rows, check_idx ? 1 : 0,
                                        static_cast<hipStream_t>(stream), &verdict);
      e != hipSuccess)
    return fail(DLM_ERR_HIP, "%s: selection check: %s", what, hipGetErrorString(e));
  if (verdict == 0) return DLM_OK;
  std::string why;
  if (verdict & dlm::kBadFirstOffset) why += " offsets[0] != 0;";
  if (verdict & dlm::kOffsetsDecrease) why += " offsets decrease;";
  if (verdict & dlm::kOffsetsPastBound) why += " offsets[B] exceeds max_rows;";
  if (verdict & dlm::kIndexOutside) why += " a position outside [0, S);";
  if (verdict & dlm::kIndexOrder) why += " positions of a batch row not strictly increasing;";
  return fail(DLM_ERR_INVALID_ARG, "%s: invalid selection (DLM_VALIDATE):%s", what, why.c_str());
}

#define CHECK_ROWS(idx, offsets, B, S, max_rows, check_idx, stream, what)                    \
  do {                                                                                     \
    if (int rc_ = check_rows(idx, offsets, B, S, max_rows, check_idx, stream, what); rc_) \
      return rc_;                                                                          \
  } while (0)

}  // namespace

extern "C" {

const char* dlm_status_string(int status) {
  switch (status) {
    case DLM_OK: return "DLM_OK";
    case DLM_ERR_INVALID_ARG: return "DLM_ERR_INVALID_ARG";
    case DLM_ERR_UNSUPPORTED: return "DLM_ERR_UNSUPPORTED";
    case DLM_ERR_WORKSPACE: return "DLM_ERR_WORKSPACE";
    case DLM_ERR_HIP: return "DLM_ERR_HIP";
    default: return "DLM_ERR_UNKNOWN";
  }
}

const char* dlm_last_error(void) { return g_last_error.c_str(); }
const char* dlm_version(void) { return "libdlm 0.1 (gfx950)"; }

// ---------------------------------------------------------------------------
size_t dlm_select_workspace_size(int mode, int B, int S, int V, int max_eval) {
  size_t n = kSelectTicketBytes;
  if (B > 0 && S > 0) n += round_up((size_t)B * S * sizeof(float), 256);
  if ((mode == DLM_SCORE_CONFIDENCE || mode == DLM_SCORE_MARGIN) && V > 0 && max_eval > 0) {
    n += round_up((size_t)max_eval * dlm::gemm_lmhead_ntile(V) * sizeof(float4), 256);
    n += dlm::gemm_workspace_bytes(dlm::EPI_LMHEAD, max_eval, V, 0);
  }
  return n;
}

int dlm_saliency_select(int mode, int dtype, const void* a, const void* b, int B, int S, int D,
                        int V, const int32_t* eval_idx, const int32_t* eval_offsets, int max_eval,
                        int lo, int hi, float threshold, float* scores, int32_t* argmax,
                        int32_t* idx, int32_t* counts, int32_t* offsets, void* workspace,
                        size_t workspace_bytes, void* stream) {
  REQUIRE(mode == DLM_SCORE_COSINE || mode == DLM_SCORE_CONFIDENCE || mode == DLM_SCORE_GIVEN ||
              mode == DLM_SCORE_MARGIN,
          "unknown scoring mode %d", mode);
  REQUIRE(dtype == DLM_F32 || dtype == DLM_BF16, "unknown dtype %d", dtype);
  REQUIRE(B > 0 && S > 0, "B and S must be positive (B=%d S=%d)", B, S);
  REQUIRE(0 <= lo && lo <= hi && hi <= S, "window [lo,hi) = [%d,%d) outside [0,%d]", lo, hi, S);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(counts);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(a);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == DLM_SCORE_GIVEN) {
    REQUIRE_ALIGNED(a);
    return hip_status(dlm::launch_given_select(static_cast<const float*>(a), B, S, lo, hi,
                                               threshold, idx, counts, offsets, st),
                      "given-score select");
  }
  REQUIRE_PTR(b);
  REQUIRE(D > 0, "D must be positive");
  REQUIRE_ALIGNED(a);
  REQUIRE_ALIGNED(b);
  if (mode == DLM_SCORE_COSINE) {
    REQUIRE(D % (dtype == DLM_BF16 ? 8 : 4) == 0, "D=%d must be a multiple of %d", D,
            dtype == DLM_BF16 ? 8 : 4);
  } else {
    REQUIRE(dtype == DLM_BF16, "confidence scoring needs bf16 hidden states and W_lm");
    REQUIRE_PTR(eval_idx);
    REQUIRE_PTR(eval_offsets);
    REQUIRE_PTR(scores);
    REQUIRE_PTR(argmax);
    REQUIRE(D % 64 == 0, "D=%d must be a multiple of 64", D);
    REQUIRE(V > 0 && V % 256 == 0, "V=%d must be a positive multiple of 256", V);
    REQUIRE(max_eval >= 0 && (long long)max_eval <= (long long)B * S, "max_eval=%d out of range",
            max_eval);
    REQUIRE((long long)B * S * D * 2 < (1ll << 31), "hidden states of 2 GiB or more");
    REQUIRE((long long)V * D * 2 < (1ll << 32), "W_lm of 4 GiB or more");
  }
  const size_t need = dlm_select_workspace_size(mode, B, S, V, max_eval);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DLM_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  REQUIRE_ALIGNED(workspace);
  float* scratch = reinterpret_cast<float*>(static_cast<char*>(workspace) + kSelectTicketBytes);
  if (mode == DLM_SCORE_COSINE) {
    float* sc = scores ? scores : scratch;
    return hip_status(dlm::launch_cosine_select(dtype, a, b, B, S, D, lo, hi, threshold, sc, idx,
                                                counts, offsets, st),
                      "cosine select");
  }
  CHECK_ROWS(eval_idx, eval_offsets, B, S, max_eval, true, stream, "confidence select");
  const int ntile = dlm::gemm_lmhead_ntile(V);
  char* wsb = static_cast<char*>(workspace) + kSelectTicketBytes + round_up((size_t)B * S * sizeof(float), 256);
  float4* part = reinterpret_cast<float4*>(wsb);
  char* gws = wsb + round_up((size_t)max_eval * ntile * sizeof(float4), 256);
  if (max_eval > 0) {
    dlm::GemmArgs g{};
    g.w = b;
    g.x = a;
    g.x_bytes = (uint32_t)((size_t)B * S * D * 2);
    g.K = D;
    g.N = V;
    g.B = B;
    g.S = S;
    g.idx = eval_idx;
    g.offsets = eval_offsets;
    g.max_rows = max_eval;
    g.lm_part = part;
    g.ntile = ntile;
    g.part = reinterpret_cast<float*>(gws);
    const int epi = mode == DLM_SCORE_MARGIN ? dlm::EPI_LMMARGIN : dlm::EPI_LMHEAD;
    int rc = hip_status(dlm::launch_gemm(DLM_BF16, epi, dlm::A_GATHER, g, st),
                        "LM-head GEMM");
    if (rc != DLM_OK) return rc;
  }
  return hip_status(dlm::launch_lmhead_combine(part, ntile, eval_idx, eval_offsets, max_eval, B, S,
                                               lo, hi, threshold, mode == DLM_SCORE_MARGIN,
                                               scores, argmax, idx, counts, offsets, st),
                    "LM-head combine");
}

// ---------------------------------------------------------------------------
size_t dlm_kl_lock_workspace_size(int B, int S, int V, int max_eval) {
  if (B <= 0 || S <= 0 || V <= 0 || max_eval <= 0) return 0;
  return round_up((size_t)max_eval * dlm::gemm_lmhead_ntile(V) * 2 * sizeof(float4), 256) +
         dlm::gemm_workspace_bytes(dlm::EPI_LMKL, max_eval, V, 0);
}

int dlm_kl_lock(const void* h_cur, const void* h_prev, const void* w_lm, int B, int S, int D, int V,
                const int32_t* eval_idx, const int32_t* eval_offsets, int max_eval, float eps,
                float gate_q, float* kl, float* maxprob, int32_t* argmax, float* locked,
                void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(B > 0 && S > 0 && D > 0, "B, S, D must be positive (B=%d S=%d D=%d)", B, S, D);
  REQUIRE(D % 64 == 0, "D=%d must be a multiple of 64", D);
  REQUIRE(V > 0 && V % 256 == 0, "V=%d must be a positive multiple of 256", V);
  REQUIRE(max_eval >= 0 && (long long)max_eval <= (long long)B * S, "max_eval=%d out of range", max_eval);
  REQUIRE(gate_q <= 1.f, "gate_q=%g must be at most 1 (<= 0: no confidence gate)", gate_q);
  REQUIRE(eps == eps, "eps must not be NaN");
  REQUIRE((long long)B * S * D * 2 < (1ll << 31), "hidden states of 2 GiB or more");
  REQUIRE((long long)V * D * 2 < (1ll << 32), "W_lm of 4 GiB or more");
  if (max_eval == 0) return DLM_OK;
  REQUIRE_PTR(h_cur);
  REQUIRE_PTR(h_prev);
  REQUIRE_PTR(w_lm);
  REQUIRE_PTR(eval_idx);
  REQUIRE_PTR(eval_offsets);
  REQUIRE_PTR(kl);
  REQUIRE_PTR(maxprob);
  REQUIRE_PTR(argmax);
  REQUIRE_PTR(locked);
  REQUIRE_ALIGNED(h_cur);
  REQUIRE_ALIGNED(h_prev);
  REQUIRE_ALIGNED(w_lm);
  const size_t need = dlm_kl_lock_workspace_size(B, S, V, max_eval);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DLM_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  REQUIRE_ALIGNED(workspace);
  CHECK_ROWS(eval_idx, eval_offsets, B, S, max_eval, true, stream, "KL lock");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ntile = dlm::gemm_lmhead_ntile(V);
  float4* part = static_cast<float4*>(workspace);
  dlm::GemmArgs g{};
  g.w = w_lm;
  g.x = h_cur;
  g.x2 = h_prev;
  g.x_bytes = (uint32_t)((size_t)B * S * D * 2);
  g.K = D;
  g.N = V;
  g.B = B;
  g.S = S;
  g.idx = eval_idx;
  g.offsets = eval_offsets;
  g.max_rows = max_eval;
  g.lm_part = part;
  g.ntile = ntile;
  g.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    round_up((size_t)max_eval * ntile * 2 * sizeof(float4), 256));
  int rc = hip_status(dlm::launch_gemm(DLM_BF16, dlm::EPI_LMKL, dlm::A_GATHER, g, st), "two-step LM head");
  if (rc != DLM_OK) return rc;
  return hip_status(dlm::launch_kl_lock(part, ntile, eval_idx, eval_offsets, max_eval, B, S, eps, gate_q,
                                        kl, maxprob, argmax, locked, st),
                    "KL lock decision");
}

// ---------------------------------------------------------------------------
size_t dlm_gather_qkv_workspace_size(int dtype, int max_rows, int D, int Hq, int Hkv, int hd) {
  if (dtype != DLM_BF16 || max_rows <= 0 || D <= 0 || Hq <= 0 || Hkv <= 0 || hd <= 0) return 0;
  return dlm::gemm_workspace_bytes(dlm::EPI_QKV, max_rows, (Hq + 2 * Hkv) * hd, D);
}

int dlm_gather_qkv_scatter_kv(int dtype, const void* x, int B, int S, int D, const int32_t* idx,
                              const int32_t* offsets, int max_rows, const void* w_qkv, int Hq,
                              int Hkv, int hd, void* q_out, void* k_cache, void* v_cache,
                              void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(dtype == DLM_F32 || dtype == DLM_BF16, "unknown dtype %d", dtype);
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_qkv);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  if (max_rows != 0) {  // with no rows to process, the row arrays may be empty (NULL)
    REQUIRE_PTR(idx);
    REQUIRE_PTR(offsets);
    REQUIRE_PTR(q_out);
  }
  REQUIRE(B > 0 && S > 0 && D > 0, "B, S, D must be positive");
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "Hq=%d must be a positive multiple of Hkv=%d", Hq,
          Hkv);
  REQUIRE(hd == 64 || hd == 128, "head dim %d not supported (64 or 128)", hd);
  REQUIRE(max_rows >= 0 && (long long)max_rows <= (long long)B * S, "max_rows=%d out of range",
          max_rows);
  REQUIRE(D % (dtype == DLM_BF16 ? 64 : 4) == 0, "D=%d must be a multiple of %d", D,
          dtype == DLM_BF16 ? 64 : 4);
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(w_qkv);
  REQUIRE_ALIGNED(q_out);
  REQUIRE_ALIGNED(k_cache);
  REQUIRE_ALIGNED(v_cache);
  if (max_rows == 0) return DLM_OK;
  if (dtype == DLM_BF16) {
    REQUIRE((long long)B * S * D * 2 < (1ll << 31), "x of 2 GiB or more is not supported");
    REQUIRE((long long)(Hq + 2 * Hkv) * hd * D * 2 < (1ll << 32), "w_qkv of 4 GiB or more");
  }
  const size_t need = dlm_gather_qkv_workspace_size(dtype, max_rows, D, Hq, Hkv, hd);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(DLM_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0) REQUIRE_ALIGNED(workspace);
  REQUIRE((long long)B * S * D < (1ll << 31), "x larger than 2^31 elements is not supported");
  CHECK_ROWS(idx, offsets, B, S, max_rows, true, stream, "gathered QKV");
  dlm::GemmArgs g{};
  g.w = w_qkv;
  g.part = static_cast<float*>(workspace);
  g.x = x;
  g.x_bytes = (uint32_t)((size_t)B * S * D * 2);
  g.K = D;
  g.N = (Hq + 2 * Hkv) * hd;
  g.B = B;
  g.S = S;
  g.idx = idx;
  g.offsets = offsets;
  g.max_rows = max_rows;
  g.q_out = q_out;
  g.k_cache = k_cache;
  g.v_cache = v_cache;
  g.nq = Hq * hd;
  g.nk = Hkv * hd;
  return hip_status(dlm::launch_gemm(dtype, dlm::EPI_QKV, dlm::A_GATHER, g,
                                     static_cast<hipStream_t>(stream)),
                    "gathered QKV GEMM");
}

// ---------------------------------------------------------------------------
size_t dlm_partial_attn_workspace_size(int dtype, int max_rows, int B, int S, int Hq, int Hkv,
                                       int hd, int D_out_wo) {
  if (max_rows <= 0 || B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || hd <= 0) return 0;
  size_t n = round_up(dlm::attn_workspace_bytes(dtype, max_rows, B, S, Hq, Hkv, hd), 256);
  if (dtype == DLM_BF16 && D_out_wo > 0)
    n += dlm::gemm_workspace_bytes(dlm::EPI_ROWS, max_rows, D_out_wo, Hq * hd);
  return n;
}

// noalloc: the split-KV partials go to the library's fixed device scratch
// instead of a caller workspace (dlm_partial_attn_noalloc)
static int partial_attn(int dtype, const void* q_sel, const int32_t* idx, const int32_t* offsets,
                        int max_rows, const void* k_cache, const void* v_cache, int B, int S, int Hq,
                        int Hkv, int hd, float scale, void* o_sel, float* lse, const void* w_o,
                        int D_out, void* out_cache, void* workspace, size_t workspace_bytes,
                        bool noalloc, void* stream) {
  REQUIRE(dtype == DLM_F32 || dtype == DLM_BF16, "unknown dtype %d", dtype);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  if (max_rows != 0) {  // with no rows to process, the row arrays may be empty (NULL)
    REQUIRE_PTR(q_sel);
    REQUIRE_PTR(idx);
    REQUIRE_PTR(offsets);
    REQUIRE_PTR(o_sel);
  }
  REQUIRE(B > 0 && S > 0, "B and S must be positive");
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "Hq=%d must be a positive multiple of Hkv=%d", Hq,
          Hkv);
  REQUIRE(hd == 64 || hd == 128, "head dim %d not supported (64 or 128)", hd);
  REQUIRE(max_rows >= 0 && (long long)max_rows <= (long long)B * S, "max_rows=%d out of range",
          max_rows);
  REQUIRE(scale > 0.f, "scale must be positive");
  REQUIRE(dtype != DLM_BF16 || (long long)(S + 64) * Hkv * hd * 2 < (1ll << 31),
          "one sequence's K or V cache slice reaches 2 GiB");
  REQUIRE_ALIGNED(q_sel);
  REQUIRE_ALIGNED(k_cache);
  REQUIRE_ALIGNED(v_cache);
  REQUIRE_ALIGNED(o_sel);
  if (w_o) {
    REQUIRE(out_cache != nullptr, "w_o given but out_cache is NULL");
    REQUIRE(D_out > 0, "D_out must be positive");
    if (dtype == DLM_BF16) {
      REQUIRE(D_out % 64 == 0 && (Hq * hd) % 64 == 0, "bf16 W_o needs D_out %% 64 == 0");
      REQUIRE((long long)D_out * Hq * hd * 2 < (1ll << 32), "W_o of 4 GiB or more");
      REQUIRE((long long)max_rows * Hq * hd * 2 < (1ll << 31), "o_sel of 2 GiB or more");
    }
    REQUIRE_ALIGNED(w_o);
  } else if (out_cache) {
    REQUIRE(D_out == Hq * hd, "without W_o, D_out (%d) must equal Hq*hd (%d)", D_out, Hq * hd);
  }
  if (out_cache) REQUIRE_ALIGNED(out_cache);
  if (noalloc) {
    // the W_o GEMM's split-K partials (loose bounds above 1024 rows) have no
    // fixed scratch; the attention's split-KV partials always fit
    if (dtype == DLM_BF16 && w_o && dlm::gemm_workspace_bytes(dlm::EPI_ROWS, max_rows, D_out, Hq * hd) > 0)
      return fail(DLM_ERR_WORKSPACE,
                  "the allocation-free call projects through W_o only for row bounds up to 1024 "
                  "(max_rows=%d); use dlm_partial_attn with a workspace", max_rows);
    if (dlm::attn_workspace_bytes(dtype, max_rows, B, S, Hq, Hkv, hd) > dlm::attn_scratch_bytes())
      return fail(DLM_ERR_WORKSPACE, "split-KV partials exceed the fixed scratch of %zu bytes",
                  dlm::attn_scratch_bytes());
  } else {
    const size_t need = dlm_partial_attn_workspace_size(dtype, max_rows, B, S, Hq, Hkv, hd, w_o ? D_out : 0);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
      return fail(DLM_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (need > 0) REQUIRE_ALIGNED(workspace);
  }
  if (max_rows == 0) return DLM_OK;
  CHECK_ROWS(idx, offsets, B, S, max_rows, true, stream, "partial attention");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (noalloc && dlm::attn_workspace_bytes(dtype, max_rows, B, S, Hq, Hkv, hd) > 0) {
    int rc = hip_status(dlm::attn_scratch_ptr(&workspace), "scratch address");
    if (rc != DLM_OK) return rc;
  }
  dlm::AttnArgs a{};
  a.q = q_sel;
  a.idx = idx;
  a.offsets = offsets;
  a.max_rows = max_rows;
  a.k = k_cache;
  a.v = v_cache;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.hd = hd;
  a.scale = scale;
  a.o = o_sel;
  a.lse = lse;
  a.ctx_out = w_o ? nullptr : out_cache;
  int rc = hip_status(dlm::launch_attn(dtype, a, workspace, st), "partial attention");
  if (rc != DLM_OK || !w_o) return rc;
  dlm::GemmArgs g{};
  g.w = w_o;
  g.x = o_sel;
  g.x_bytes = (uint32_t)((size_t)max_rows * Hq * hd * 2);
  g.K = Hq * hd;
  g.N = D_out;
  g.B = B;
  g.S = S;
  g.idx = idx;
  g.offsets = offsets;
  g.max_rows = max_rows;
  g.out = out_cache;
  g.ld_out = D_out;
  if (dtype == DLM_BF16 && !noalloc) {  // (the allocation-free call needs no GEMM partials)
    char* gws = static_cast<char*>(workspace) +
                round_up(dlm::attn_workspace_bytes(dtype, max_rows, B, S, Hq, Hkv, hd), 256);
    g.part = reinterpret_cast<float*>(gws);
  }
  return hip_status(dlm::launch_gemm(dtype, dlm::EPI_ROWS, dlm::A_COMPACT, g, st),
                    "output projection");
}

int dlm_partial_attn(int dtype, const void* q_sel, const int32_t* idx, const int32_t* offsets,
                     int max_rows, const void* k_cache, const void* v_cache, int B, int S, int Hq,
                     int Hkv, int hd, float scale, void* o_sel, float* lse, const void* w_o,
                     int D_out, void* out_cache, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return partial_attn(dtype, q_sel, idx, offsets, max_rows, k_cache, v_cache, B, S, Hq, Hkv, hd,
                      scale, o_sel, lse, w_o, D_out, out_cache, workspace, workspace_bytes, false,
                      stream);
}

int dlm_partial_attn_noalloc(int dtype, const void* q_sel, const int32_t* idx,
                             const int32_t* offsets, int max_rows, const void* k_cache,
                             const void* v_cache, int B, int S, int Hq, int Hkv, int hd,
                             float scale, void* o_sel, float* lse, const void* w_o, int D_out,
                             void* out_cache, void* stream) {
  return partial_attn(dtype, q_sel, idx, offsets, max_rows, k_cache, v_cache, B, S, Hq, Hkv, hd,
                      scale, o_sel, lse, w_o, D_out, out_cache, nullptr, 0, true, stream);
}

size_t dlm_partial_attn_noalloc_scratch_bytes(void) { return dlm::attn_scratch_bytes(); }

// ---------------------------------------------------------------------------
size_t dlm_attn_colsum_workspace_size(int B, int S, int Hkv) {
  if (B <= 0 || S <= 0 || Hkv <= 0) return 0;
  return dlm::colsum_workspace_bytes(B, S, Hkv);
}

static int attn_colsum(int dtype, const void* q_sel, const int32_t* offsets, int max_rows,
                       const void* k_cache, const float* lse, int B, int S, int Hq, int Hkv,
                       int hd, float scale, float* colsum, int key_lo, int key_hi, int k,
                       int32_t* topk_idx, float* topk_val, void* workspace,
                       size_t workspace_bytes, int window, void* stream) {
  if (dtype != DLM_BF16)
    return fail(DLM_ERR_UNSUPPORTED, "attention column sums are implemented for bf16 only");
  REQUIRE_PTR(q_sel);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(colsum);
  REQUIRE(B > 0 && S > 0, "B and S must be positive");
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "Hq=%d must be a positive multiple of Hkv=%d", Hq,
          Hkv);
  REQUIRE(hd == 64 || hd == 128, "head dim %d not supported (64 or 128)", hd);
  REQUIRE(max_rows >= 0 && (long long)max_rows <= (long long)B * S, "max_rows=%d out of range",
          max_rows);
  REQUIRE(0 <= key_lo && key_lo <= key_hi && key_hi <= S, "key window [%d,%d) outside [0,%d]",
          key_lo, key_hi, S);
  REQUIRE(k >= 0 && k <= key_hi - key_lo, "k=%d exceeds the key window", k);
  REQUIRE(k == 0 || key_hi - key_lo <= 8192, "top-k key window limited to 8192 keys");
  REQUIRE(k == 0 || topk_idx != nullptr || topk_val != nullptr, "k > 0 needs an output");
  REQUIRE_ALIGNED(q_sel);
  REQUIRE_ALIGNED(k_cache);
  const size_t need = dlm_attn_colsum_workspace_size(B, S, Hkv);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DLM_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  CHECK_ROWS(nullptr, offsets, B, S, max_rows, false, stream, "column sums");
  return hip_status(dlm::launch_colsum(q_sel, offsets, max_rows, k_cache, lse, B, S, Hq, Hkv, hd,
                                       scale, static_cast<float*>(workspace), colsum, key_lo,
                                       key_hi, k, topk_idx, topk_val, window,
                                       static_cast<hipStream_t>(stream)),
                    "attention column sums");
}

int dlm_attn_colsum(int dtype, const void* q_sel, const int32_t* offsets, int max_rows,
                    const void* k_cache, const float* lse, int B, int S, int Hq, int Hkv, int hd,
                    float scale, float* colsum, int key_lo, int key_hi, int k, int32_t* topk_idx,
                    float* topk_val, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_colsum(dtype, q_sel, offsets, max_rows, k_cache, lse, B, S, Hq, Hkv, hd, scale,
                     colsum, key_lo, key_hi, k, topk_idx, topk_val, workspace, workspace_bytes, 0,
                     stream);
}

int dlm_attn_colsum_window(int dtype, const void* q_sel, const int32_t* offsets, int max_rows,
                           const void* k_cache, const float* lse, int B, int S, int Hq, int Hkv,
                           int hd, float scale, float* colsum, int key_lo, int key_hi, int k,
                           int32_t* topk_idx, float* topk_val, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return attn_colsum(dtype, q_sel, offsets, max_rows, k_cache, lse, B, S, Hq, Hkv, hd, scale,
                     colsum, key_lo, key_hi, k, topk_idx, topk_val, workspace, workspace_bytes, 1,
                     stream);
}

// ---------------------------------------------------------------------------
int dlm_stable_prefix(const int32_t* argmax, const float* maxprob, int B, int S, int gen_lo,
                      int gen_hi, int32_t* ring, int W, int step, float conf_threshold,
                      int min_commit, int32_t* committed, void* stream) {
  REQUIRE_PTR(argmax);
  REQUIRE_PTR(maxprob);
  REQUIRE_PTR(ring);
  REQUIRE_PTR(committed);
  REQUIRE(B > 0 && S > 0, "B and S must be positive");
  REQUIRE(0 <= gen_lo && gen_lo < gen_hi && gen_hi <= S, "generated region [%d,%d) invalid",
          gen_lo, gen_hi);
  REQUIRE(W >= 1 && W <= 64, "ring depth W=%d out of range [1,64]", W);
  REQUIRE(step >= 0, "step must be non-negative");
  return hip_status(dlm::launch_stable_prefix(argmax, maxprob, B, S, gen_lo, gen_hi, ring, W, step,
                                              conf_threshold, min_commit, committed,
                                              static_cast<hipStream_t>(stream)),
                    "stable prefix");
}

// ---------------------------------------------------------------------------
size_t dlm_salient_ffn_workspace_size(int dtype, int max_rows, int D, int F) {
  if (dtype != DLM_BF16 || max_rows <= 0 || D <= 0 || F <= 0) return 0;
  const size_t h = round_up((size_t)max_rows * F * 2, 256);
  const size_t g1 = dlm::gemm_workspace_bytes(dlm::EPI_SWIGLU, max_rows, 2 * F, D);
  size_t g2 = dlm::gemm_workspace_bytes(dlm::EPI_ROWS, max_rows, D, F);
  const size_t g3 = dlm::gemm_skinny_split_bytes(max_rows, D, F);  // the down projection's K split
  if (g3 > g2) g2 = g3;
  return h + (g1 > g2 ? g1 : g2);
}

int dlm_salient_ffn(int dtype, const void* x, int B, int S, int D, const int32_t* idx,
                    const int32_t* offsets, int max_rows, const void* w_gu, int F,
                    const void* w_down, void* out_cache, void* workspace, size_t workspace_bytes,
                    void* stream) {
  REQUIRE(dtype == DLM_F32 || dtype == DLM_BF16, "unknown dtype %d", dtype);
  if (dtype != DLM_BF16) return fail(DLM_ERR_UNSUPPORTED, "the salient-row FFN is bf16 only");
  REQUIRE(B > 0 && S > 0 && D > 0 && F > 0, "B, S, D, F must be positive");
  REQUIRE(D % 64 == 0 && F % 64 == 0, "D=%d and F=%d must be multiples of 64", D, F);
  REQUIRE(max_rows >= 0 && (long long)max_rows <= (long long)B * S, "max_rows=%d out of range",
          max_rows);
  REQUIRE((long long)B * S * D * 2 < (1ll << 31), "x of 2 GiB or more is not supported");
  REQUIRE((long long)2 * F * D * 2 < (1ll << 32), "w_gu of 4 GiB or more");
  REQUIRE((long long)max_rows * F * 2 < (1ll << 31), "the FFN rows of 2 GiB or more");
  if (max_rows == 0) return DLM_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(w_gu);
  REQUIRE_PTR(w_down);
  REQUIRE_PTR(out_cache);
  REQUIRE_ALIGNED(x);
  REQUIRE_ALIGNED(w_gu);
  REQUIRE_ALIGNED(w_down);
  REQUIRE_ALIGNED(out_cache);
  const size_t need = dlm_salient_ffn_workspace_size(dtype, max_rows, D, F);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DLM_ERR_WORKSPACE, "workspace of %zu bytes required, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  REQUIRE_ALIGNED(workspace);
  CHECK_ROWS(idx, offsets, B, S, max_rows, true, stream, "salient FFN");
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* h = workspace;
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         round_up((size_t)max_rows * F * 2, 256));
  // gate and up of the gathered rows, SwiGLU in the epilogue -> h [max_rows, F]
  dlm::GemmArgs g{};
  g.w = w_gu;
  g.x = x;
  g.x_bytes = (uint32_t)((size_t)B * S * D * 2);
  g.K = D;
  g.N = 2 * F;
  g.B = B;
  g.S = S;
  g.idx = idx;
  g.offsets = offsets;
  g.max_rows = max_rows;
  g.out = h;
  g.ld_out = F;
  g.part = part;
  int rc = hip_status(dlm::launch_gemm(dtype, dlm::EPI_SWIGLU, dlm::A_GATHER, g, st), "FFN gate/up");
  if (rc != DLM_OK) return rc;
  // down projection of h, rows scattered into the output cache
  dlm::GemmArgs d{};
  d.w = w_down;
  d.x = h;
  d.x_bytes = (uint32_t)((size_t)max_rows * F * 2);
  d.K = F;
  d.N = D;
  d.B = B;
  d.S = S;
  d.idx = idx;
  d.offsets = offsets;
  d.max_rows = max_rows;
  d.out = out_cache;
  d.ld_out = D;
  d.part = part;
  d.skinny_split = 1;  // a short selection splits K over the CUs (D / 64 tiles alone leave most idle)
  return hip_status(dlm::launch_gemm(dtype, dlm::EPI_ROWS, dlm::A_COMPACT, d, st), "FFN down");
}

// ---------------------------------------------------------------------------
static int row_copy(const void* src, void* dst, const int32_t* idx, const int32_t* offsets,
                    int max_rows, int B, int S, int row_bytes, int scatter, void* stream) {
  REQUIRE(B > 0 && S > 0, "B and S must be positive");
  REQUIRE(row_bytes > 0 && row_bytes % 4 == 0, "row_bytes=%d must be a positive multiple of 4",
          row_bytes);
  REQUIRE(max_rows >= 0 && (long long)max_rows <= (long long)B * S, "max_rows=%d out of range",
          max_rows);
  if (max_rows == 0) return DLM_OK;
  REQUIRE_PTR(src);
  REQUIRE_PTR(dst);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(offsets);
  REQUIRE(((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 3u) == 0,
          "src and dst must be 4-byte aligned");
  if (row_bytes % 16 == 0) {
    REQUIRE_ALIGNED(src);
    REQUIRE_ALIGNED(dst);
  }
  CHECK_ROWS(idx, offsets, B, S, max_rows, true, stream, scatter ? "row scatter" : "row gather");
  return hip_status(dlm::launch_row_copy(src, dst, idx, offsets, max_rows, B, S, row_bytes, scatter,
                                         static_cast<hipStream_t>(stream)),
                    scatter ? "row scatter" : "row gather");
}

int dlm_gather_rows(const void* cache, int B, int S, int row_bytes, const int32_t* idx,
                    const int32_t* offsets, int max_rows, void* rows, void* stream) {
  return row_copy(cache, rows, idx, offsets, max_rows, B, S, row_bytes, 0, stream);
}

int dlm_scatter_rows(const void* rows, const int32_t* idx, const int32_t* offsets, int max_rows,
                     int B, int S, int row_bytes, void* cache, void* stream) {
  return row_copy(rows, cache, idx, offsets, max_rows, B, S, row_bytes, 1, stream);
}

int dlm_nonsalient_dv_update(int dtype, const void* q_cache, const float* lse_cache,
                             const int32_t* idx, const int32_t* offsets, int max_rows,
                             const void* k_old, const void* v_old, const void* v_cache, int B,
                             int S, int Hq, int Hkv, int hd, float scale, void* o_cache,
                             void* stream) {
  REQUIRE(dtype == DLM_F32 || dtype == DLM_BF16, "unknown dtype %d", dtype);
  REQUIRE(B > 0 && S > 0, "B and S must be positive");
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, "Hq=%d must be a positive multiple of Hkv=%d", Hq,
          Hkv);
  REQUIRE(128 % (Hq / Hkv) == 0, "query heads per KV head (%d) must divide 128", Hq / Hkv);
  REQUIRE(hd == 64 || hd == 128, "head dim %d not supported (64 or 128)", hd);
  REQUIRE(max_rows >= 0 && (long long)max_rows <= (long long)B * S, "max_rows=%d out of range",
          max_rows);
  REQUIRE(scale > 0.f, "scale must be positive");
  if (max_rows == 0) return DLM_OK;  // no salient rows: nothing changes
  REQUIRE_PTR(q_cache);
  REQUIRE_PTR(lse_cache);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(offsets);
  REQUIRE_PTR(k_old);
  REQUIRE_PTR(v_old);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(o_cache);
  REQUIRE_ALIGNED(q_cache);
  REQUIRE_ALIGNED(k_old);
  REQUIRE_ALIGNED(v_old);
  REQUIRE_ALIGNED(v_cache);
  REQUIRE_ALIGNED(o_cache);
  CHECK_ROWS(idx, offsets, B, S, max_rows, true, stream, "non-salient update");
  dlm::DvArgs a{};
  a.q = q_cache;
  a.lse = lse_cache;
  a.idx = idx;
  a.offsets = offsets;
  a.max_rows = max_rows;
  a.k_old = k_old;
  a.v_old = v_old;
  a.v = v_cache;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.hd = hd;
  a.scale = scale;
  a.o = o_cache;
  return hip_status(dlm::launch_dv_update(dtype, a, static_cast<hipStream_t>(stream)),
                    "non-salient update");
}

// ---------------------------------------------------------------------------
int dlm_lsp_adaptive_commit(const float* margin, int B, int S, int gen_lo, int gen_hi,
                            float frac_lo, float frac_hi, float margin_floor, int32_t* committed,
                            float* tau, void* stream) {
  REQUIRE_PTR(margin);
  REQUIRE_PTR(committed);
  REQUIRE(B > 0 && S > 0, "B and S must be positive");
  REQUIRE(0 <= gen_lo && gen_lo < gen_hi && gen_hi <= S, "generated region [%d,%d) invalid",
          gen_lo, gen_hi);
  REQUIRE(frac_lo > 0.f && frac_lo <= frac_hi && frac_hi <= 1.f,
          "fractions must satisfy 0 < frac_lo <= frac_hi <= 1 (got %g, %g)", frac_lo, frac_hi);
  REQUIRE(margin_floor == margin_floor, "margin_floor must not be NaN (-INFINITY: no floor)");
  return hip_status(dlm::launch_lsp_adaptive(margin, B, S, gen_lo, gen_hi, frac_lo, frac_hi,
                                             margin_floor, committed, tau,
                                             static_cast<hipStream_t>(stream)),
                    "adaptive commit");
}

// ---------------------------------------------------------------------------
int dlm_probe_mfma_bf16(int iters, int grid, float* sink, void* stream) {
  REQUIRE(iters > 0 && grid > 0, "iters=%d and grid=%d must be positive", iters, grid);
  REQUIRE_PTR(sink);
  return hip_status(dlm::launch_probe_mfma(iters, grid, sink, static_cast<hipStream_t>(stream)),
                    "MFMA probe");
}

}  // extern "C"
