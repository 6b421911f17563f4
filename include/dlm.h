/*
 * dlm.h - C ABI of the sparse-query denoising step for MI355X (gfx950).
 *
 * One denoising step of a masked diffusion LM that re-processes only the
 * tokens that are still changing:
 *   1. score every token's stability (cosine against the previous step, or the
 *      model's max-softmax confidence)                 -> dlm_saliency_select
 *   2. compact the selected positions into an index list (same call)
 *   3. recompute Q/K/V for only those rows and scatter K/V into the
 *      persistent full-length cache                     -> dlm_gather_qkv_scatter_kv
 *   4. bidirectional attention of the selected queries over all keys, with
 *      the outputs scattered back into the cached activations
 *                                                       -> dlm_partial_attn
 *      optional: per-key attention column sums + top-k  -> dlm_attn_colsum
 *      optional: longest-stable-prefix commit           -> dlm_stable_prefix
 *                (adaptive threshold on the logit margin -> dlm_lsp_adaptive_commit)
 *      optional: KL-divergence lock of converged tokens -> dlm_kl_lock
 *      optional: FFN of the salient rows                -> dlm_salient_ffn
 *      optional: value-change update of the stable rows -> dlm_nonsalient_dv_update
 *                (caches kept with dlm_gather_rows / dlm_scatter_rows)
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains caller memory.  Tensors are
 *     dense, row-major, in the layouts stated per argument, and 16-byte
 *     aligned.
 *   - `dtype` is DLM_F32 (float) or DLM_BF16 (bfloat16 storage, float32
 *     accumulation, bf16 results rounded to nearest-even).
 *   - Weights are stored output-major: row n holds the D input weights of
 *     output feature n (so y = x . W^T).
 *   - Selected rows are passed as (idx, offsets): idx int32 holds positions
 *     in ascending order per batch row, packed batch-major; offsets int32
 *     [B+1] is the exclusive prefix sum of the per-row counts.  Both live on
 *     the device; `max_rows` is a host-side upper bound on offsets[B] used to
 *     size launch grids (work beyond the device count is skipped on the GPU),
 *     so no call synchronises with the host.  With max_rows == 0 a call
 *     does nothing and its row arrays (idx, offsets, per-row outputs) may be NULL.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream), allocates nothing, and returns a status code.
 *     Argument validation happens on the host before any launch: on failure
 *     nothing has been enqueued.  dlm_last_error() gives a thread-local text
 *     describing the last failure.
 *   - `workspace` is caller-owned device scratch of at least the size the
 *     matching *_workspace_size() query returns (any contents; nothing in it
 *     survives a call).  Calls that overlap in time must not share a
 *     workspace.
 */
#ifndef DLM_H
#define DLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define DLM_OK 0
#define DLM_ERR_INVALID_ARG 1   /* null pointer, bad shape, misalignment       */
#define DLM_ERR_UNSUPPORTED 2   /* valid request this build does not implement  */
#define DLM_ERR_WORKSPACE 3     /* workspace missing or too small               */
#define DLM_ERR_HIP 4           /* a HIP launch or runtime call failed          */

/* element types */
#define DLM_F32 0
#define DLM_BF16 1

/* scoring modes of dlm_saliency_select */
#define DLM_SCORE_COSINE 0
#define DLM_SCORE_CONFIDENCE 1
#define DLM_SCORE_GIVEN 2
#define DLM_SCORE_MARGIN 3

const char* dlm_status_string(int status);
const char* dlm_last_error(void);
/* Version string of the library build. */
const char* dlm_version(void);

/* ------------------------------------------------------------------------
 * dlm_saliency_select
 *
 * Scores token stability and compacts the positions to recompute.
 * Follows: "DyLLM: Efficient Diffusion LLM Inference via Saliency-based
 * Token Selection and Partial Attention", Methodologie 1 (temporal cosine
 * similarity per token between consecutive steps; low similarity = salient
 * = recomputed); "Accelerating Diffusion Large Language Models with SlowFast
 * Sampling", Metodologia, certainty principle (max predicted confidence);
 * "Stopping Computation for Converged Tokens in Masked Diffusion-LM
 * Decoding", Methodik (unlocked positions are recomputed).
 *
 * mode DLM_SCORE_COSINE:  a = cur [B,S,D], b = prev [B,S,D] (dtype).
 *     scores[b,i] = <cur,prev> / (|cur| |prev|) for i in [lo,hi) (0 when a
 *     norm is 0), float32 accumulation.  `scores` may be NULL (then the
 *     scores live in the workspace only).  Other entries are not written.
 * mode DLM_SCORE_CONFIDENCE (dtype must be DLM_BF16):  a = hidden [B,S,D],
 *     b = W_lm [V,D].  For the rows listed by (eval_idx, eval_offsets)
 *     (at most max_eval of them) the logits z = h . W_lm^T are formed on the
 *     matrix cores and reduced on the fly (never stored): scores[b,i] =
 *     1 / sum_v exp(z_v - max z) (the max softmax probability) and
 *     argmax[b,i] = lowest v attaining max z.  `scores` [B,S] f32 and
 *     `argmax` [B,S] i32 are required and act as caches: entries of rows
 *     not evaluated keep their values.  D % 64 == 0, V % 256 == 0.
 * mode DLM_SCORE_MARGIN:  as DLM_SCORE_CONFIDENCE, with scores[b,i] = the
 *     logit margin, max z minus the second-largest logit (0 when the maximum
 *     is attained twice).  Follows "Beyond Scattered Acceptance: Fast and
 *     Coherent Inference for DLMs via Longest Stable Prefixes", Methodologie
 *     (stability diagnosis by the logit margin).
 * mode DLM_SCORE_GIVEN:  a = scores f32 [B,S] supplied by the caller
 *     (e.g. 1 = locked, 0 = unlocked); b, scores, argmax unused.
 *
 * Compaction (all modes): position i in [lo,hi) of row b is selected iff
 * score < threshold (strict).  idx int32 (capacity B*(hi-lo)) receives the
 * selected positions ascending per row, packed batch-major; counts int32 [B];
 * offsets int32 [B+1].
 * ------------------------------------------------------------------------ */
size_t dlm_select_workspace_size(int mode, int B, int S, int V, int max_eval);
int dlm_saliency_select(int mode, int dtype, const void* a, const void* b,
                        int B, int S, int D, int V,
                        const int32_t* eval_idx, const int32_t* eval_offsets, int max_eval,
                        int lo, int hi, float threshold,
                        float* scores, int32_t* argmax,
                        int32_t* idx, int32_t* counts, int32_t* offsets,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dlm_gather_qkv_scatter_kv
 *
 * Q/K/V projection of the selected rows only; K/V scattered into the
 * persistent cache.  Follows: "Stopping Computation for Converged Tokens in
 * Masked Diffusion-LM Decoding", Methodik, Kernprinzipien (locked positions
 * skip their projections, their K/V stay cached); "DyLLM ...", Methodologie 1
 * (stable tokens reuse cached activations).
 *
 * x [B,S,D]; w_qkv [(Hq+2*Hkv)*hd, D] output-major with rows [0,Hq*hd) =
 * W_q, then W_k, then W_v; head h owns rows [h*hd,(h+1)*hd) of its block.
 * For every selected row r = (b, i = idx[r]):
 *   q_out[r, :, :]       = x[b,i] . W_q^T        q_out [max_rows, Hq, hd]
 *   k_cache[b, i, :, :]  = x[b,i] . W_k^T        k_cache, v_cache [B,S,Hkv,hd]
 *   v_cache[b, i, :, :]  = x[b,i] . W_v^T
 * Cache rows that are not selected are not touched (byte-identical).
 * bf16: D % 64 == 0, hd in {64,128}, x under 2 GiB, w_qkv under 4 GiB.  The
 * workspace (size from dlm_gather_qkv_workspace_size) holds split-K partial
 * tiles; only bounds above 1024 rows with (Hq+2*Hkv)*hd % 256 == 0 and D/64 a
 * multiple of 4 need one (size 0 otherwise, and then workspace may be NULL).
 * Its size covers the most partial tiles any real row count up to the bound
 * can make the device split into: 8 per 256 x 256 output tile of the bound,
 * at most 1024 tiles of 256 KB.  f32: D % 4 == 0, no workspace.
 * ------------------------------------------------------------------------ */
size_t dlm_gather_qkv_workspace_size(int dtype, int max_rows, int D, int Hq, int Hkv, int hd);
int dlm_gather_qkv_scatter_kv(int dtype, const void* x, int B, int S, int D,
                              const int32_t* idx, const int32_t* offsets, int max_rows,
                              const void* w_qkv, int Hq, int Hkv, int hd,
                              void* q_out, void* k_cache, void* v_cache,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dlm_partial_attn
 *
 * Bidirectional (unmasked) attention of the selected queries over all S
 * keys, outputs scattered back.  Follows: "DyLLM ...", Methodologie 2 (salient
 * path: attention rows fully recomputed for the selected tokens); "Stopping
 * Computation ...", Methodik, Kernprinzipien (active tokens attend to the
 * cached K/V of locked tokens; cost O(M N d)).
 *
 * q_sel [max_rows, Hq, hd] (rows in idx order); k_cache, v_cache
 * [B,S,Hkv,hd]; query head h reads KV head h / (Hq/Hkv).  For each selected
 * row r of batch row b and head h:
 *   o_sel[r,h,:] = softmax_j(scale * q.K[b,j]) . V[b,j]   over all j < S
 *   lse[r,h]     = natural-log log-sum-exp of the scaled scores (lse may be NULL)
 * Output scatter (optional):
 *   w_o == NULL, out_cache != NULL:  out_cache[b, idx[r], :] = concat_h o_sel[r,h,:]
 *                                    (D_out must equal Hq*hd)
 *   w_o != NULL:  out_cache[b, idx[r], :] = concat_h o_sel[r,h,:] . W_o^T,
 *                 w_o [D_out, Hq*hd] output-major; out_cache required.
 * Other out_cache rows are not touched.  hd in {64,128}.  bf16: one
 * sequence's K (or V) slice plus 64 rows, (S+64)*Hkv*hd*2 bytes, stays under
 * 2 GiB, else DLM_ERR_INVALID_ARG.
 * Workspace (size from dlm_partial_attn_workspace_size, D_out_wo = D_out when
 * a W_o projection will be passed, else 0): bf16 needs split-KV partials only
 * for S >= 512 and the W_o GEMM's split-K tiles only for loose bounds above
 * 1024 rows; when the size is 0, workspace may be NULL.
 * ------------------------------------------------------------------------ */
size_t dlm_partial_attn_workspace_size(int dtype, int max_rows, int B, int S, int Hq, int Hkv,
                                       int hd, int D_out_wo);
int dlm_partial_attn(int dtype, const void* q_sel, const int32_t* idx, const int32_t* offsets,
                     int max_rows, const void* k_cache, const void* v_cache,
                     int B, int S, int Hq, int Hkv, int hd, float scale,
                     void* o_sel, float* lse,
                     const void* w_o, int D_out, void* out_cache,
                     void* workspace, size_t workspace_bytes, void* stream);

/* dlm_partial_attn_noalloc: dlm_partial_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument.  The split-KV
 * partials go to a fixed scratch array inside the library, one per GPU, of
 * dlm_partial_attn_noalloc_scratch_bytes() bytes (64.5 MiB, the largest
 * workspace dlm_partial_attn ever asks for), held until the process ends; the
 * call itself allocates nothing.  Same kernels and work plan as
 * dlm_partial_attn, so the outputs are bit-identical to it.  Limit: a bf16
 * W_o projection is accepted only for max_rows <= 1024 (larger bounds need
 * split-K partials), else DLM_ERR_WORKSPACE before any launch.  Calls that
 * overlap in time on one GPU share the scratch and race: order them on one
 * stream.  The first call on a device looks up the scratch's address there
 * (DLM_ERR_HIP if that fails). */
int dlm_partial_attn_noalloc(int dtype, const void* q_sel, const int32_t* idx,
                             const int32_t* offsets, int max_rows, const void* k_cache,
                             const void* v_cache, int B, int S, int Hq, int Hkv, int hd,
                             float scale, void* o_sel, float* lse, const void* w_o, int D_out,
                             void* out_cache, void* stream);
size_t dlm_partial_attn_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * dlm_attn_colsum
 *
 * Per-key attention column sums and the top-k keys.  Follows: "Attention-
 * Based Sampler for Diffusion Language Models", Methodologie 1-2 (decode
 * tokens in descending order of the column sums of the attention matrix,
 * aggregated over heads).
 *
 * colsum[b,j] = sum over the selected rows r of b and all heads h of
 *               exp(scale * q_sel[r,h] . K[b,j,h/(Hq/Hkv)] - lse[r,h])
 * for every j < S (bf16 only, float32 throughout).  lse [max_rows, Hq] is
 * the natural-log LSE of the same queries (from dlm_partial_attn).
 * If k > 0: topk_idx [B,k] i32 / topk_val [B,k] f32 receive the k keys of
 * [key_lo,key_hi) with the largest sums, ordered by (-colsum, j): equal sums
 * go to the lower position.  k <= key_hi-key_lo <= 8192.
 * Workspace: dlm_attn_colsum_workspace_size(B, S, Hkv) bytes, the per-key
 * float partial sums of up to 4 query ranges of every KV head (the split
 * depends on the shapes and the device's CU count; reruns are bit-identical).
 * ------------------------------------------------------------------------ */
size_t dlm_attn_colsum_workspace_size(int B, int S, int Hkv);
int dlm_attn_colsum(int dtype, const void* q_sel, const int32_t* offsets, int max_rows,
                    const void* k_cache, const float* lse,
                    int B, int S, int Hq, int Hkv, int hd, float scale,
                    float* colsum, int key_lo, int key_hi, int k,
                    int32_t* topk_idx, float* topk_val,
                    void* workspace, size_t workspace_bytes, void* stream);

/* dlm_attn_colsum_window: the same call with the work cut to the key window,
 * for block-wise use ("Attention-Based Sampler for Diffusion Language
 * Models", Methodologie 2: the scores are computed per sub-block rather than
 * over the whole sequence).  colsum[b,j] is computed for the 256-key blocks
 * that cover [key_lo, key_hi) only (so for every j in the window); entries of
 * other blocks are not touched.  Same arguments, limits and workspace. */
int dlm_attn_colsum_window(int dtype, const void* q_sel, const int32_t* offsets, int max_rows,
                           const void* k_cache, const float* lse,
                           int B, int S, int Hq, int Hkv, int hd, float scale,
                           float* colsum, int key_lo, int key_hi, int k,
                           int32_t* topk_idx, float* topk_val,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dlm_stable_prefix
 *
 * Longest-stable-prefix commit.  Follows: "Beyond Scattered Acceptance: Fast
 * and Coherent Inference for DLMs via Longest Stable Prefixes", Methodologie
 * (commit the longest contiguous stable block at the start of the remaining
 * active region in one step; commit at least one token as a fallback).
 *
 * argmax [B,S] i32 and maxprob [B,S] f32 hold each position's latest values
 * (-1 / anything before its first evaluation).  ring [B, gen_hi-gen_lo, W]
 * i32 keeps the last W pushes per generated position (initialise to -1).
 * Step `step` first pushes argmax[b, gen_lo+i] into slot step % W for every
 * generated position i, then, from the frontier L = committed[b] (a count
 * of committed generated positions), advances over positions whose W ring
 * entries are equal and not -1 and whose maxprob >= conf_threshold; if none
 * advanced, min_commit != 0 and L < gen_hi-gen_lo, it advances by one.
 * committed [B] i32 is updated in place.
 * ------------------------------------------------------------------------ */
int dlm_stable_prefix(const int32_t* argmax, const float* maxprob, int B, int S,
                      int gen_lo, int gen_hi, int32_t* ring, int W, int step,
                      float conf_threshold, int min_commit, int32_t* committed, void* stream);

/* ------------------------------------------------------------------------
 * dlm_kl_lock
 *
 * The locking criterion of "Stopping Computation for Converged Tokens in
 * Masked Diffusion-LM Decoding", 2. Methodik, Kriterium zum Sperren: a
 * position is locked (its projections and FFN are skipped from then on, its
 * K/V stay cached) when the local KL divergence between its posteriors at
 * this and the previous step, KL(p_t || p_{t-1}), falls below eps, and -
 * the optional confidence gate - its uncertainty 1 - max p_t lies at or
 * below the gate_q percentile of the uncertainties of its sequence's
 * evaluated positions.
 *
 * For the positions listed by (eval_idx, eval_offsets) (at most max_eval),
 * p_t and p_{t-1} are the softmax of the LM-head logits h . W_lm^T of the
 * position's hidden state in h_cur and in h_prev [B,S,D] bf16 (W_lm [V,D]
 * bf16), formed on the matrix cores in one pass over W_lm and reduced on the
 * fly (logits are never stored).  Writes, at the evaluated positions of the
 * [B,S] arrays: kl (f32; rounding can leave a value a few ulps below 0),
 * maxprob = max p_t (f32) and argmax of p_t (i32, lowest index on ties);
 * then sets locked[b,i] = 1.0f (f32 [B,S], 1 = locked, other values kept;
 * usable as the given scores of DLM_SCORE_GIVEN with threshold 0.5) where
 * kl < eps (strict) and, if 0 < gate_q <= 1, maxprob >= the k-th largest
 * maxprob of the sequence's evaluated positions, k = max(1, ceil(gate_q *
 * n_b)) computed in double (the nearest-rank percentile; equal values all
 * pass).  gate_q <= 0: no gate.  Other entries are not written.
 * D % 64 == 0, V % 256 == 0; workspace from dlm_kl_lock_workspace_size.
 * ------------------------------------------------------------------------ */
size_t dlm_kl_lock_workspace_size(int B, int S, int V, int max_eval);
int dlm_kl_lock(const void* h_cur, const void* h_prev, const void* w_lm, int B, int S, int D, int V,
                const int32_t* eval_idx, const int32_t* eval_offsets, int max_eval,
                float eps, float gate_q, float* kl, float* maxprob, int32_t* argmax,
                float* locked, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dlm_nonsalient_dv_update
 *
 * Value-change update of the stable rows' cached attention outputs.  Follows:
 * "DyLLM: Efficient Diffusion LLM Inference via Saliency-based Token
 * Selection and Partial Attention", Methodologie 2, non-salient path (the
 * stable tokens' attention weights are taken as unchanged; their outputs move
 * by the salient tokens' value change times those weights, cost O(N |A|)).
 *
 * For every b, every position i not in the salient set A_b (idx/offsets) and
 * every query head h, with g = h / (Hq/Hkv):
 *   o_cache[b,i,h] += sum_{r in A_b} exp(scale * q_cache[b,i,h] . k_old[r,g]
 *                                        - lse_cache[b,i,h])
 *                                    * (v_cache[b,idx[r],g] - v_old[r,g])
 * The weights are token i's softmax weights of its last computation: its
 * cached query, its cached natural-log LSE and the salient rows' K from
 * before this step's scatter.  Rows in A_b are not touched (dlm_partial_attn
 * writes them).
 *   q_cache   [B,S,Hq,hd]   dtype   queries as last computed per position
 *   lse_cache [B,S,Hq]      f32     their LSE (dlm_partial_attn's lse,
 *                                   scattered with dlm_scatter_rows)
 *   k_old, v_old [max_rows,Hkv,hd] dtype  salient rows' K/V before this
 *                                   step's dlm_gather_qkv_scatter_kv
 *                                   (dlm_gather_rows of the caches)
 *   v_cache   [B,S,Hkv,hd]  dtype   V cache after that scatter
 *   o_cache   [B,S,Hq,hd]   dtype   per-head context cache, updated in place
 *                                   (the out_cache of dlm_partial_attn
 *                                   without W_o); bf16 adds in float32 and
 *                                   rounds once.
 * hd in {64,128}; Hq/Hkv must divide 128.  bf16 rounds the weights and the
 * value change to bf16 for the matrix cores (float32 accumulation).
 * ------------------------------------------------------------------------ */
int dlm_nonsalient_dv_update(int dtype, const void* q_cache, const float* lse_cache,
                             const int32_t* idx, const int32_t* offsets, int max_rows,
                             const void* k_old, const void* v_old, const void* v_cache,
                             int B, int S, int Hq, int Hkv, int hd, float scale,
                             void* o_cache, void* stream);

/* ------------------------------------------------------------------------
 * dlm_salient_ffn
 *
 * The FFN of the salient rows only.  Follows: "DyLLM: Efficient Diffusion
 * LLM Inference via Saliency-based Token Selection and Partial Attention",
 * Methodologie 1 (the FFN is skipped for non-salient tokens, which reuse
 * their cached activations).  The pages name no FFN form; this is a SwiGLU
 * MLP (bf16 only, float32 accumulation):
 *   h[r, f]            = silu(x[b,idx[r]] . w_gu[2f]) * (x[b,idx[r]] . w_gu[2f+1])
 *   out_cache[b,idx[r]] = h[r] . w_down^T,   silu(z) = z / (1 + e^-z)
 *   x        [B,S,D]  bf16  FFN input per position (under 2 GiB)
 *   w_gu     [2F,D]   bf16  gate and up rows interleaved: row 2f = gate
 *                           feature f, row 2f+1 = up feature f
 *   w_down   [D,F]    bf16  output-major
 *   out_cache [B,S,D] bf16  selected rows replaced; others not touched
 * D and F multiples of 64.  h (rounded to bf16) lives in the workspace of
 * dlm_salient_ffn_workspace_size(dtype, max_rows, D, F) bytes, followed by
 * fp32 split-K partial tiles: long selections may split either product;
 * short ones (max_rows <= 128) split the down projection's K when it has
 * fewer than 128 output tiles of 64 features (D < 8192), so that more CUs
 * stream w_down.  dtype DLM_F32 -> DLM_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
size_t dlm_salient_ffn_workspace_size(int dtype, int max_rows, int D, int F);
int dlm_salient_ffn(int dtype, const void* x, int B, int S, int D,
                    const int32_t* idx, const int32_t* offsets, int max_rows,
                    const void* w_gu, int F, const void* w_down, void* out_cache,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dlm_gather_rows / dlm_scatter_rows
 *
 * Row copies between a per-position cache [B,S,row_bytes] and the packed
 * rows of a selection [max_rows,row_bytes] (row r <-> cache row (b, idx[r])).
 * They keep the caches of the non-salient update: the salient rows' K/V
 * before the step's scatter (gather), and the recomputed rows' queries and
 * LSE (scatter).  Follows: "DyLLM ...", Methodologie 1 (recomputed tokens
 * replace their cached activations; all others keep theirs).
 *   gather:  rows[r] = cache[b, idx[r]]     scatter: cache[b, idx[r]] = rows[r]
 * row_bytes a positive multiple of 4 (both pointers 4-byte aligned, 16-byte
 * aligned when row_bytes is a multiple of 16).  Other cache rows are not
 * touched.
 * ------------------------------------------------------------------------ */
int dlm_gather_rows(const void* cache, int B, int S, int row_bytes,
                    const int32_t* idx, const int32_t* offsets, int max_rows,
                    void* rows, void* stream);
int dlm_scatter_rows(const void* rows, const int32_t* idx, const int32_t* offsets,
                     int max_rows, int B, int S, int row_bytes, void* cache, void* stream);

/* ------------------------------------------------------------------------
 * dlm_lsp_adaptive_commit
 *
 * Commit with an adaptive threshold on the logit margin.  Follows: "Beyond
 * Scattered Acceptance: Fast and Coherent Inference for DLMs via Longest
 * Stable Prefixes", Methodologie (stability by the logit margin; the
 * threshold tau is searched so that the committed stable block covers a
 * fraction range of the active length, e.g. 25 % to 50 %; at least one
 * token is committed; structural snapping is not done).
 *
 * margin [B,S] f32 (DLM_SCORE_MARGIN scores); committed [B] i32 = generated
 * positions committed so far, updated in place.  For each b with A =
 * (gen_hi - gen_lo) - committed[b] > 0 active positions starting at
 * gen_lo + committed[b]:
 *   lo = max(1, ceil(frac_lo * A)), hi = max(lo, floor(frac_hi * A))
 *        (computed in double from the float32 fractions)
 *   tau = max(min of the first lo active margins (the largest threshold
 *         under which they are all stable), margin_floor)
 *   committed[b] += max(1, min(run of leading active margins >= tau, hi))
 * margin_floor is an absolute notion of "stable enough" for the page's
 * fallback (commit at least one when no token is stable enough): with it
 * above the first active margin exactly one position is committed.
 * -INFINITY: no floor (then the run always reaches lo).  tau [B] f32 (may be
 * NULL) receives the threshold used, or NaN where nothing is active.
 * 0 < frac_lo <= frac_hi <= 1 and margin_floor not NaN, else
 * DLM_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
int dlm_lsp_adaptive_commit(const float* margin, int B, int S, int gen_lo, int gen_hi,
                            float frac_lo, float frac_hi, float margin_floor, int32_t* committed,
                            float* tau, void* stream);

/* ------------------------------------------------------------------------
 * dlm_probe_mfma_bf16  (measurement aid, not a step of the method)
 *
 * Runs grid workgroups of 256 threads in which every wave issues `iters`
 * rounds of eight independent 32x32x16 bf16 MFMAs on register operands (no
 * memory traffic): grid * 4 * iters * 8 * 32768 flop.  Timing it gives the
 * matrix pipes' peak at the clock the chip holds under MFMA load, the
 * measured ceiling that roofline fractions are also reported against.
 * sink [grid*256] f32 (device) receives one value per thread.  iters > 0,
 * grid > 0, else DLM_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------ */
int dlm_probe_mfma_bf16(int iters, int grid, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DLM_H */
