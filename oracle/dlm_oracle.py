"""CPU float64 oracle for the sparse-query denoising step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library: it is plain NumPy written from
the method pages, slow and obviously correct, in float64 throughout (inputs are
converted exactly from their float32 / bfloat16 storage values; nothing is
rounded on the way).

Pages followed (title, section):
  [DyLLM]   "DyLLM: Efficient Diffusion LLM Inference via Saliency-based Token
            Selection and Partial Attention" - Methodologie 1 (temporal cosine
            similarity per token; low similarity = salient, recomputed; stable
            tokens reuse cached activations, the FFN included), Methodologie 2
            (salient path: full recomputation of the attention rows;
            non-salient path: existing weights times the value change),
            Methodologie 3 (adaptive input: response tokens only on most
            steps, the whole sequence every few steps).
  [SlowFast] "Accelerating Diffusion Large Language Models with SlowFast
            Sampling" - Metodologia, certainty and convergence principles
            (max predicted confidence as the stability signal).
  [AttnS]   "Attention-Based Sampler for Diffusion Language Models" -
            Methodologie 1-2 (decode in descending order of attention-matrix
            column sums, aggregated over heads).
  [SureLock] "Stopping Computation for Converged Tokens in Masked Diffusion-LM
            Decoding" - Methodik, Kernprinzipien (locked positions skip the
            query projection; their K/V stay cached and are still attended to;
            cost O(M N d)); Kriterium zum Sperren (lock when the local KL
            divergence between consecutive posteriors falls below eps,
            optionally gated by a percentile of the uncertainty 1 - max p).
  [LSP]     "Beyond Scattered Acceptance: Fast and Coherent Inference for DLMs
            via Longest Stable Prefixes" - Methodologie (commit the longest
            contiguous stable block at the start of the active region in one
            step; commit at least one token as a fallback; logit margin
            as the stability score, adaptive threshold within a fraction range
            of the active length).

Pinning status: every function here is pinned by tests/test_oracle_pins.py to
closed forms, brute force on tiny inputs or invariants (see that file).
"""
from __future__ import annotations

import math

import numpy as np

f64 = np.float64


# --------------------------------------------------------------------------
# (1) stability scores
# --------------------------------------------------------------------------
def cosine_scores(cur, prev):
    """[DyLLM] Methodologie 1: temporal cosine similarity of each token's vector
    between the current and the previous denoising step.

    cur, prev: [..., D].  Returns [...] float64.  A zero norm on either side
    gives similarity 0 (so the token is treated as changed and recomputed)."""
    c = np.asarray(cur, dtype=f64)
    p = np.asarray(prev, dtype=f64)
    dot = np.einsum("...d,...d->...", c, p)
    nc = np.sqrt(np.einsum("...d,...d->...", c, c))
    npv = np.sqrt(np.einsum("...d,...d->...", p, p))
    den = nc * npv
    out = np.zeros(dot.shape, dtype=f64)
    ok = den > 0
    out[ok] = dot[ok] / den[ok]
    return out


def confidence(rows, w_lm):
    """[SlowFast] Metodologia (certainty principle) / [SureLock] Kriterium zum
    Sperren (confidence gate 1 - max p): the model's maximum predicted
    probability per token and the token that attains it.

    rows: [n, D] hidden states; w_lm: [V, D] (row v = output weights of token v).
    Returns (maxprob [n], argmax [n] int64 - lowest index on ties,
             gap [n] = top-1 minus top-2 logit, used to flag argmaxes that
             rounding could decide either way)."""
    x = np.asarray(rows, dtype=f64)
    w = np.asarray(w_lm, dtype=f64)
    z = x @ w.T                                   # logits [n, V]
    a = np.argmax(z, axis=1)                      # first maximal index
    zmax = z[np.arange(z.shape[0]), a]
    denom = np.exp(z - zmax[:, None]).sum(axis=1)
    maxprob = 1.0 / denom
    if z.shape[1] > 1:
        part = np.partition(z, z.shape[1] - 2, axis=1)
        gap = part[:, -1] - part[:, -2]
    else:
        gap = np.full(z.shape[0], np.inf)
    return maxprob, a.astype(np.int64), gap


# --------------------------------------------------------------------------
# (2) compaction of the selected positions
# --------------------------------------------------------------------------
def compact(scores, lo, hi, threshold):
    """[DyLLM] Methodologie 1: tokens whose similarity is low are salient and
    are selected for recomputation; [SureLock] Kernprinzipien: unlocked
    positions are the ones recomputed.  A position i in [lo, hi) of batch row b
    is selected iff scores[b, i] < threshold (strict).

    Returns (idx int32 [n] ascending within each batch row, packed batch-major;
             counts int32 [B]; offsets int32 [B+1] exclusive prefix sum)."""
    sc = np.asarray(scores)
    B = sc.shape[0]
    per_b = []
    for b in range(B):
        window = sc[b, lo:hi]
        per_b.append(np.nonzero(window < threshold)[0].astype(np.int64) + lo)
    counts = np.array([len(p) for p in per_b], dtype=np.int32)
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    idx = np.concatenate(per_b).astype(np.int32) if B else np.zeros(0, np.int32)
    return idx, counts, offsets


def rows_of(idx, offsets, b):
    return np.asarray(idx[offsets[b]:offsets[b + 1]], dtype=np.int64)


# --------------------------------------------------------------------------
# (3) Q/K/V for the selected rows, K/V scattered into the persistent cache
# --------------------------------------------------------------------------
def qkv_project_scatter(x, idx, offsets, w_qkv, Hq, Hkv, hd, k_cache, v_cache):
    """[SureLock] Kernprinzipien: only active positions compute their
    projections; locked positions keep their cached K/V.  [DyLLM]
    Methodologie 1: non-salient tokens reuse cached activations.

    x: [B,S,D]; w_qkv: [(Hq+2Hkv)*hd, D] with rows [0,Hq*hd) = W_q, then W_k,
    then W_v; head h owns rows [h*hd,(h+1)*hd) of its block.
    Returns (q_sel [n,Hq,hd], k_cache', v_cache') as float64 copies; cache rows
    that are not selected are left exactly as given."""
    x = np.asarray(x, dtype=f64)
    w = np.asarray(w_qkv, dtype=f64)
    kc = np.array(k_cache, dtype=f64, copy=True)
    vc = np.array(v_cache, dtype=f64, copy=True)
    B = x.shape[0]
    n = int(offsets[B])
    q_sel = np.zeros((n, Hq, hd), dtype=f64)
    nq, nk = Hq * hd, Hkv * hd
    for b in range(B):
        rows = rows_of(idx, offsets, b)
        if rows.size == 0:
            continue
        y = x[b, rows] @ w.T                        # [n_b, (Hq+2Hkv)*hd]
        q_sel[offsets[b]:offsets[b + 1]] = y[:, :nq].reshape(-1, Hq, hd)
        kc[b, rows] = y[:, nq:nq + nk].reshape(-1, Hkv, hd)
        vc[b, rows] = y[:, nq + nk:nq + 2 * nk].reshape(-1, Hkv, hd)
    return q_sel, kc, vc


# --------------------------------------------------------------------------
# (4) bidirectional partial attention of the selected queries over all keys
# --------------------------------------------------------------------------
def partial_attention(q_sel, idx, offsets, k_cache, v_cache, Hq, Hkv, scale):
    """[DyLLM] Methodologie 2 (salient path) and [SureLock] Kernprinzipien:
    every selected query attends, without a mask (bidirectional model), to the
    keys of *all* S positions of its sequence as they stand in the cache after
    this step's scatter.  Query head h reads KV head h // (Hq // Hkv).

    Returns (o_sel [n,Hq,hd], lse [n,Hq]) with lse the natural-log
    log-sum-exp of the scaled scores."""
    q = np.asarray(q_sel, dtype=f64)
    kc = np.asarray(k_cache, dtype=f64)
    vc = np.asarray(v_cache, dtype=f64)
    B = kc.shape[0]
    G = Hq // Hkv
    n = q.shape[0]
    o = np.zeros_like(q)
    lse = np.zeros((n, Hq), dtype=f64)
    for b in range(B):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 == r0:
            continue
        for h in range(Hq):
            g = h // G
            s = scale * (q[r0:r1, h, :] @ kc[b, :, g, :].T)    # [n_b, S]
            m = s.max(axis=1, keepdims=True)
            l = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
            p = np.exp(s - l[:, None])
            o[r0:r1, h, :] = p @ vc[b, :, g, :]
            lse[r0:r1, h] = l
    return o, lse


def output_scatter(o_sel, idx, offsets, out_cache, w_o=None):
    """[DyLLM] Methodologie 1: recomputed tokens overwrite their cached
    activations; all other rows keep the cached values.  The context rows are
    the heads concatenated (optionally projected by W_o [D_out, Hq*hd])."""
    o = np.asarray(o_sel, dtype=f64)
    out = np.array(out_cache, dtype=f64, copy=True)
    B = out.shape[0]
    ctx = o.reshape(o.shape[0], int(np.prod(o.shape[1:])))
    y = ctx if w_o is None else ctx @ np.asarray(w_o, dtype=f64).T
    for b in range(B):
        rows = rows_of(idx, offsets, b)
        out[b, rows] = y[offsets[b]:offsets[b + 1]]
    return out


def salient_ffn(x, idx, offsets, w_gu, w_down, out_cache):
    """[DyLLM] Methodologie 1: the FFN is computed for the salient tokens only;
    every other token keeps its cached FFN output.

    Reading (the pages name no FFN form): a SwiGLU MLP, y = (silu(x W_g^T) *
    (x W_u^T)) W_d^T with silu(z) = z / (1 + e^-z), on the selected rows of x
    [B,S,D].  w_gu [2F, D] holds gate and up rows interleaved (row 2f = gate
    feature f, row 2f+1 = up feature f); w_down [D, F].  Returns (h [n,F], the
    output cache [B,S,D] with the selected rows replaced by y)."""
    xs = gather_rows(np.asarray(x, dtype=f64), idx, offsets)
    wgu = np.asarray(w_gu, dtype=f64)
    g = xs @ wgu[0::2].T
    u = xs @ wgu[1::2].T
    h = g / (1.0 + np.exp(-g)) * u
    y = h @ np.asarray(w_down, dtype=f64).T
    return h, scatter_rows(y, idx, offsets, np.asarray(out_cache, dtype=f64))


def gather_rows(src, idx, offsets):
    """Rows src[b, idx[r]] of every selected r, packed (row r of batch row b):
    how a caller keeps the salient rows' K/V from before this step's scatter."""
    s = np.asarray(src)
    out = np.zeros((int(offsets[-1]),) + s.shape[2:], dtype=s.dtype)
    for b in range(s.shape[0]):
        out[offsets[b]:offsets[b + 1]] = s[b, rows_of(idx, offsets, b)]
    return out


def scatter_rows(rows, idx, offsets, dst):
    """dst with dst[b, idx[r]] = rows[r] for every selected r; other rows kept."""
    out = np.array(dst, copy=True)
    for b in range(out.shape[0]):
        out[b, rows_of(idx, offsets, b)] = np.asarray(rows)[offsets[b]:offsets[b + 1]]
    return out


def nonsalient_dv_update(q_cache, lse_cache, idx, offsets, k_old, v_old, v_cache, o_cache, Hq,
                         Hkv, scale):
    """[DyLLM] Methodologie 2, non-salient path: for a stable token the
    attention weights are taken as unchanged (their change is neglected), and
    its output moves only by the change of the salient tokens' values, weighted
    by its existing attention weights:

        o_i <- o_i + sum_{j in A} P_ij (v_j^new - v_j^old)

    Reading (the page names no formula for the weights): P_ij is token i's
    softmax weight on key j as of its last computation, exp(scale q_i . k_j^old
    - lse_i), from its cached query q_i, its cached natural-log LSE lse_i and
    key j's K row from before this step's scatter.

    q_cache [B,S,Hq,hd] and lse_cache [B,S,Hq]: each position's query and LSE
    as last computed; idx/offsets: the salient set A; k_old, v_old [n,Hkv,hd]:
    the salient rows' K/V before this step's scatter (row r = idx[r]);
    v_cache [B,S,Hkv,hd] after it; o_cache [B,S,Hq,hd] the per-head context
    cache.  Returns the updated context cache: salient rows are left as given
    (their outputs come from the salient path), every other row gets the
    update.  Query head h reads KV head h // (Hq // Hkv)."""
    q = np.asarray(q_cache, dtype=f64)
    lse = np.asarray(lse_cache, dtype=f64)
    ko = np.asarray(k_old, dtype=f64)
    vo = np.asarray(v_old, dtype=f64)
    vc = np.asarray(v_cache, dtype=f64)
    out = np.array(o_cache, dtype=f64, copy=True)
    B, S = q.shape[0], q.shape[1]
    G = Hq // Hkv
    for b in range(B):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 == r0:
            continue
        sal = rows_of(idx, offsets, b)
        stable = np.setdiff1d(np.arange(S), sal)
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, stable, h, :] @ ko[r0:r1, g, :].T)     # [N - n_b, n_b]
            p = np.exp(s - lse[b, stable, h][:, None])
            dv = vc[b, sal, g, :] - vo[r0:r1, g, :]                  # [n_b, hd]
            out[b, stable, h, :] += p @ dv
    return out


# --------------------------------------------------------------------------
# (4') attention column sums and the top-k decode order
# --------------------------------------------------------------------------
def column_sums(q_sel, offsets, k_cache, lse, Hq, Hkv, scale):
    """[AttnS] Methodologie 1-2: total attention each key receives - the column
    sums of the softmax attention matrix, summed over the selected queries and
    over all heads.  p = exp(scale * q.k - lse) with the queries' own lse.

    Returns c [B,S]."""
    q = np.asarray(q_sel, dtype=f64)
    kc = np.asarray(k_cache, dtype=f64)
    ls = np.asarray(lse, dtype=f64)
    B, S = kc.shape[0], kc.shape[1]
    G = Hq // Hkv
    c = np.zeros((B, S), dtype=f64)
    for b in range(B):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 == r0:
            continue
        for h in range(Hq):
            s = scale * (q[r0:r1, h, :] @ kc[b, :, h // G, :].T)
            c[b] += np.exp(s - ls[r0:r1, h][:, None]).sum(axis=0)
    return c


def topk_keys(c, key_lo, key_hi, k):
    """[AttnS] Methodologie 1: decode in descending order of column sum.  The k
    keys of [key_lo, key_hi) with the largest sums, ordered by (-c, index):
    equal sums go to the lower position.  Returns (idx int32 [B,k], val [B,k])."""
    c = np.asarray(c, dtype=f64)
    B = c.shape[0]
    out_i = np.zeros((B, k), dtype=np.int32)
    out_v = np.zeros((B, k), dtype=f64)
    keys = np.arange(key_lo, key_hi)
    for b in range(B):
        vals = c[b, key_lo:key_hi]
        order = np.lexsort((keys, -vals))[:k]       # primary -c, secondary index
        out_i[b] = keys[order]
        out_v[b] = vals[order]
    return out_i, out_v


# --------------------------------------------------------------------------
# (5) longest stable prefix
# --------------------------------------------------------------------------
def stable_prefix_step(argmax, maxprob, ring, step, gen_lo, gen_hi, conf_threshold,
                       min_commit, committed):
    """[LSP] Methodologie: commit, in one step, the longest contiguous run of
    stable positions that starts at the current frontier of the generated
    region; if min_commit and nothing is stable, commit one position anyway.
    Stability (the workload's rule, [SlowFast] convergence principle): the
    token's per-step argmax has been the same over the last W steps and its
    max probability is >= conf_threshold.

    argmax [B,S] int (latest argmax per position, -1 before its first
    evaluation; non-evaluated positions carry their previous value forward),
    maxprob [B,S] (latest value, same carry-forward), ring [B,S_gen,W] int
    (last W pushes; -1 = empty), committed [B] = current frontier as a count of
    committed generated positions.  The comparison maxprob >= conf_threshold is
    taken in the precision of the maxprob array given.

    Returns (ring', committed') as new arrays."""
    ring = np.array(ring, copy=True)
    W = ring.shape[2]
    B = ring.shape[0]
    S_gen = gen_hi - gen_lo
    ring[:, :, step % W] = np.asarray(argmax)[:, gen_lo:gen_hi]
    mp = np.asarray(maxprob)
    thr = mp.dtype.type(conf_threshold) if np.issubdtype(mp.dtype, np.floating) else conf_threshold
    new = np.array(committed, dtype=np.int64, copy=True)
    for b in range(B):
        L = int(committed[b])
        run = 0
        while L + run < S_gen:
            i = L + run
            r = ring[b, i]
            stable = bool(np.all(r == r[0]) and r[0] != -1 and mp[b, gen_lo + i] >= thr)
            if not stable:
                break
            run += 1
        if min_commit and run == 0 and L < S_gen:
            run = 1
        new[b] = L + run
    return ring, new


def logit_margin(rows, w_lm):
    """[LSP] Methodologie, stability diagnosis: a position's logit margin, the
    top-1 minus the top-2 logit (0 when the maximum is attained twice), and the
    argmax (lowest index on ties).  rows [n, D], w_lm [V, D]."""
    z = np.asarray(rows, dtype=f64) @ np.asarray(w_lm, dtype=f64).T
    a = np.argmax(z, axis=1)
    srt = np.sort(z, axis=1)
    return srt[:, -1] - srt[:, -2], a.astype(np.int64)


def lsp_adaptive_commit(margin, gen_lo, gen_hi, committed, frac_lo=0.25, frac_hi=0.5,
                        margin_floor=-math.inf):
    """[LSP] Methodologie, adaptive sizing: the threshold tau is searched so
    that the stable block at the start of the active suffix covers a fraction
    of the active length within [frac_lo, frac_hi]; at least one token is
    committed.

    Reading: with A the active length, lo = max(1, ceil(frac_lo A)) and
    hi = max(lo, floor(frac_hi A)), tau is the largest threshold under which
    the first lo active positions are all stable (their minimum margin), and
    the block is the run of leading positions with margin >= tau, cut at hi.
    margin [B,S] (float32 values compared exactly); committed [B] = committed
    generated positions so far.

    Optional absolute floor (the page's fallback, "if no token is stable
    enough, commit at least one", needs a notion of enough): the threshold
    used is max(tau, margin_floor); when even the first active position's
    margin is below it, exactly one position is committed.  With the default
    floor (-inf) the rule above is unchanged.  Returns (new committed [B],
    threshold used [B]; nan where nothing is active)."""
    m = np.asarray(margin)
    B = m.shape[0]
    out = np.array(committed, dtype=np.int64, copy=True)
    tau = np.full(B, np.nan)
    G = gen_hi - gen_lo
    for b in range(B):
        A = G - int(out[b])
        if A <= 0:
            continue
        act = m[b, gen_lo + out[b]:gen_hi]
        lo = max(1, math.ceil(frac_lo * A))
        hi = max(lo, math.floor(frac_hi * A))
        t = max(act[:lo].min(), margin_floor)
        L = 0
        while L < A and act[L] >= t:
            L += 1
        out[b] += max(1, min(L, hi))
        tau[b] = t
    return out, tau


def kl_divergence(rows_cur, rows_prev, w_lm):
    """[SureLock] 2. Methodik, Kriterium zum Sperren (criterion 1): the local
    KL divergence D_t = KL(p_t || p_{t-1}) between a position's posterior over
    the vocabulary at this step and at the previous step, with p = softmax of
    the LM-head logits of the position's hidden state at that step.

    rows_cur, rows_prev [n, D] (the same positions at steps t and t-1), w_lm
    [V, D].  Written from the definition KL(p||q) = sum_v p_v (log p_v - log
    q_v), with log-probabilities z - logsumexp(z).  Also returns this step's
    max probability and argmax (lowest index on ties), which the confidence
    gate uses, and the top-1 minus top-2 logit gap (to flag argmaxes that
    rounding could decide either way).  Returns (kl [n], maxprob [n],
    argmax [n] int64, gap [n])."""
    w = np.asarray(w_lm, dtype=f64)
    zt = np.asarray(rows_cur, dtype=f64) @ w.T
    zp = np.asarray(rows_prev, dtype=f64) @ w.T

    def log_softmax(z):
        m = z.max(axis=1, keepdims=True)
        return z - (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))
    lt, lp = log_softmax(zt), log_softmax(zp)
    pt = np.exp(lt)
    kl = (pt * (lt - lp)).sum(axis=1)
    a = np.argmax(zt, axis=1)
    maxprob = pt[np.arange(pt.shape[0]), a]
    srt = np.sort(zt, axis=1)
    gap = srt[:, -1] - srt[:, -2] if zt.shape[1] > 1 else np.full(zt.shape[0], np.inf)
    return kl, maxprob, a.astype(np.int64), gap


def surelock_lock(kl, maxprob, eval_idx, eval_offsets, locked, eps, gate_q=0.0):
    """[SureLock] 2. Methodik, Kriterium zum Sperren: an evaluated position is
    locked when its local KL divergence falls below eps (criterion 1, strict)
    and, when the optional confidence gate is on (gate_q > 0), its uncertainty
    1 - max p lies at or below the gate_q percentile of the uncertainties of
    the positions evaluated in its sequence at this step (criterion 2).  Locks
    are permanent: locked positions stay locked.

    Reading of the percentile: the nearest-rank order statistic - with n
    evaluated positions and k = ceil(gate_q * n) (at least 1), the k-th
    smallest uncertainty.  As 1 - p falls when p rises, a position passes iff
    its max p is at least the k-th largest max p of its sequence's evaluated
    positions (compared on the max-probabilities themselves, so that no
    rounding of 1 - p decides).  k is computed in double from the float32
    gate_q, as the library does.

    kl, maxprob [B,S] (read at the evaluated positions; the comparisons are
    exact on the values given); locked [B,S] (1 = locked, 0 = active).
    Returns the new lock array."""
    kl = np.asarray(kl)
    mp = np.asarray(maxprob)
    out = np.array(locked, copy=True)
    B = out.shape[0]
    for b in range(B):
        rows = rows_of(eval_idx, eval_offsets, b)
        if rows.size == 0:
            continue
        thr = None
        if gate_q > 0:
            k = max(1, math.ceil(float(gate_q) * rows.size))
            thr = sorted(mp[b, rows].tolist(), reverse=True)[min(k, rows.size) - 1]
        for i in rows:
            if kl[b, i] < eps and (thr is None or mp[b, i] >= thr):
                out[b, i] = 1
    return out


def admissible_frontiers(prev_set, stable_state, S_gen, min_commit):
    """Set of frontiers reachable in one step when some positions' stability is
    ambiguous (a decision within the tolerance band of a float comparison).

    prev_set: set of possible previous frontiers; stable_state: int array
    [S_gen] with 1 = definitely stable, 0 = definitely not, 2 = ambiguous."""
    out = set()
    for L in prev_set:
        i = L
        stops = []
        while i < S_gen:
            st = stable_state[i]
            if st == 0:
                stops.append(i)
                break
            if st == 2:
                stops.append(i)
            i += 1
        else:
            stops.append(S_gen)
        for e in stops:
            out.add(L + 1 if (min_commit and e == L and L < S_gen) else e)
    return out


# --------------------------------------------------------------------------
# whole steps (chains of the above, as the workloads run them)
# --------------------------------------------------------------------------
def full_recompute_caches(x, w_qkv, Hq, Hkv, hd, scale, w_o=None):
    """Caches as a full (every position selected) pass on x would leave them:
    K/V caches and the output cache.  Used to build the step's input state."""
    x = np.asarray(x, dtype=f64)
    B, S, _ = x.shape
    idx = np.tile(np.arange(S, dtype=np.int32), B)
    offsets = (np.arange(B + 1) * S).astype(np.int32)
    zeros_kv = np.zeros((B, S, Hkv, hd))
    q, kc, vc = qkv_project_scatter(x, idx, offsets, w_qkv, Hq, Hkv, hd, zeros_kv, zeros_kv)
    o, _ = partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, scale)
    d_out = Hq * hd if w_o is None else np.asarray(w_o).shape[0]
    out = output_scatter(o, idx, offsets, np.zeros((B, S, d_out)), w_o)
    return kc, vc, out


def adaptive_input_window(t, prompt, S, refresh=4):
    """[DyLLM] Methodologie 3 (adaptive input): on most steps only the response
    tokens are input, so only they can be scored and selected; every
    `refresh` steps the whole sequence (prompt + response) is input to refresh
    the context, and even then only salient tokens are recomputed.

    Reading: the full sequence is input at the steps t with t % refresh == 0
    (the first step included), the response [prompt, S) at every other step.
    Returns the scoring window (lo, hi)."""
    return (0, S) if t % refresh == 0 else (prompt, S)


def cosine_step(cur, prev, w_qkv, Hq, Hkv, hd, tau, k_cache, v_cache, out_cache, w_o=None,
                lo=0, hi=None):
    """One DyLLM-style step: cosine scores -> compaction -> Q/K/V of the selected
    rows with K/V scatter -> partial attention -> output scatter."""
    S = np.asarray(cur).shape[1]
    hi = S if hi is None else hi
    scale = 1.0 / np.sqrt(hd)
    s = cosine_scores(cur, prev)
    idx, counts, offsets = compact(s, lo, hi, tau)
    q, kc, vc = qkv_project_scatter(cur, idx, offsets, w_qkv, Hq, Hkv, hd, k_cache, v_cache)
    o, lse = partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, scale)
    out = output_scatter(o, idx, offsets, out_cache, w_o)
    return dict(scores=s, idx=idx, counts=counts, offsets=offsets, q=q, k_cache=kc,
                v_cache=vc, o=o, lse=lse, out_cache=out)
