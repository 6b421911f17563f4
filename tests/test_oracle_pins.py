"""Pins for the fp64 oracle: each check ties it to something other than itself -
closed forms, pure-Python brute force on tiny inputs, independent library
routines (torch's CPU attention and softmax in float64, sorted()), invariants the
pages state, and hand-derived fixtures under tests/golden/.

The pages print no worked example with intermediate values, so no pin compares
against numbers printed on the pages; the hand fixtures are derivations from
the definitions they state."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import dlm_oracle as O
from sparse_query_attention_dlm_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# pure-Python brute force (no NumPy arithmetic)
# --------------------------------------------------------------------------
def bf_cos(a, b):
    dot = sum(x * y for x, y in zip(a, b))
    na = math.sqrt(sum(x * x for x in a))
    nb = math.sqrt(sum(y * y for y in b))
    return 0.0 if na * nb == 0 else dot / (na * nb)


def bf_attention_row(q, keys, vals, scale):
    s = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    o = [sum(e[j] / z * vals[j][d] for j in range(len(keys))) for d in range(len(vals[0]))]
    return o, m + math.log(z)


def to_list(a):
    return np.asarray(a, dtype=np.float64).tolist()


# --------------------------------------------------------------------------
# cosine
# --------------------------------------------------------------------------
def test_cosine_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5, 7))
    assert np.allclose(O.cosine_scores(x, x), 1.0, atol=1e-15)
    assert np.allclose(O.cosine_scores(x, -x), -1.0, atol=1e-15)
    assert np.allclose(O.cosine_scores(x, 3.5 * x), 1.0, atol=1e-15)   # positive scaling
    e = np.eye(4)
    assert np.allclose(O.cosine_scores(e[0], e[1]), 0.0)
    assert O.cosine_scores(np.array([1.0, 0.0]), np.array([1.0, 1.0])) == pytest.approx(1 / math.sqrt(2), abs=1e-15)
    assert O.cosine_scores(np.array([1.0, 2, 3]), np.array([4.0, 5, 6])) == pytest.approx(
        32 / (math.sqrt(14) * math.sqrt(77)), abs=1e-15)
    # a zero vector on either side scores 0
    z = np.zeros(6)
    assert O.cosine_scores(z, np.ones(6)) == 0.0 and O.cosine_scores(np.ones(6), z) == 0.0


def test_cosine_brute_force():
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal((2, 4, 9))
    got = O.cosine_scores(a[None], b[None])[0]
    for i in range(4):
        assert got[i] == pytest.approx(bf_cos(to_list(a[i]), to_list(b[i])), abs=1e-14)


def test_planted_tiny_selects_exactly_the_redrawn_rows():
    inp = W.cosine_step_inputs(W.TINY_FP32)
    s = O.cosine_scores(inp.cur, inp.prev)
    idx, counts, offsets = O.compact(s, 0, W.TINY_FP32.S, W.TINY_FP32.tau)
    assert counts.tolist() == [16]
    assert idx.tolist() == inp.redrawn[0].tolist()
    stable = np.setdiff1d(np.arange(128), inp.redrawn[0])
    assert s[0, stable].min() > 0.999 and s[0, inp.redrawn[0]].max() < 0.5


def test_planted_bf16_selects_exactly_the_redrawn_rows():
    sh = W.BF16_S1024
    inp = W.cosine_step_inputs(sh, D=512)      # reduced hidden size, same structure
    s = O.cosine_scores(inp.cur, inp.prev)
    idx, counts, _ = O.compact(s, 0, sh.S, sh.tau)
    assert counts.tolist() == [102]
    assert idx.tolist() == inp.redrawn[0].tolist()


def test_adaptive_input_window_closed_forms():
    """DyLLM, Methodologie 3: the whole sequence every `refresh` steps (from the
    first), the response alone otherwise."""
    got = [O.adaptive_input_window(t, 512, 1024) for t in range(9)]
    full, resp = (0, 1024), (512, 1024)
    assert got == [full, resp, resp, resp, full, resp, resp, resp, full]
    assert all(O.adaptive_input_window(t, 7, 20, refresh=1) == (0, 20) for t in range(5))
    assert [O.adaptive_input_window(t, 7, 20, refresh=2) for t in range(4)] == [(0, 20), (7, 20)] * 2


def test_dyllm_loop_selects_the_planted_rows_in_the_window():
    """Each step of the planted loop (every row drifts, a few prompt and
    response rows are redrawn): the oracle selects exactly the rows redrawn at
    that step that lie in the step's window - the response rows only on
    response-only steps, prompt and response rows on refresh steps."""
    sh = W.DYLLM_LOOP
    inp = W.dyllm_loop_inputs(sh, B=2, S=256, prompt=128, D=512, response_redrawn=13, prompt_redrawn=3)
    s = inp.shape
    for t in range(s.steps):
        lo, hi = O.adaptive_input_window(t, s.prompt, s.S, s.refresh)
        sc = O.cosine_scores(inp.hidden(t), inp.hidden(t - 1))
        idx, counts, off = O.compact(sc, lo, hi, s.tau)
        for b in range(s.B):
            want = [i for i in inp.redrawn(t)[b].tolist() if lo <= i < hi]
            assert O.rows_of(idx, off, b).tolist() == want, f"step {t} row {b}"
        assert counts.sum() == s.B * (s.response_redrawn + (s.prompt_redrawn if lo == 0 else 0))


def test_response_only_step_leaves_prompt_rows():
    """A step scored on [prompt, S) recomputes no prompt row: the prompt's K/V
    and output cache rows are exactly the cached ones, even where the prompt's
    hidden states changed."""
    inp = W.dyllm_loop_inputs(W.DYLLM_LOOP, B=1, S=96, prompt=40, D=128, Hq=2, Hkv=2, hd=64,
                              response_redrawn=9, prompt_redrawn=5)
    s = inp.shape
    rng = np.random.default_rng(3)
    kc, vc = rng.standard_normal((1, 96, 2, 64)), rng.standard_normal((1, 96, 2, 64))
    out = rng.standard_normal((1, 96, 128))
    r = O.cosine_step(inp.hidden(1), inp.hidden(0), inp.w_qkv, 2, 2, 64, s.tau, kc, vc, out, lo=40, hi=96)
    assert r["idx"].min() >= 40 and len(r["idx"]) == 9
    assert np.array_equal(r["k_cache"][:, :40], kc[:, :40]) and np.array_equal(r["v_cache"][:, :40], vc[:, :40])
    assert np.array_equal(r["out_cache"][:, :40], out[:, :40])


# --------------------------------------------------------------------------
# compaction
# --------------------------------------------------------------------------
def test_compact_brute_force_and_strictness():
    rng = np.random.default_rng(2)
    sc = rng.random((3, 50))
    sc[1, 7] = 0.5                                  # exactly at the threshold: not selected
    lo, hi, tau = 5, 44, 0.5
    idx, counts, offsets = O.compact(sc, lo, hi, tau)
    exp = [[i for i in range(lo, hi) if sc[b, i] < tau] for b in range(3)]
    assert counts.tolist() == [len(e) for e in exp]
    assert offsets.tolist() == [0, len(exp[0]), len(exp[0]) + len(exp[1]), sum(map(len, exp))]
    assert idx.tolist() == exp[0] + exp[1] + exp[2]
    assert 7 not in exp[1]


def test_compact_empty_and_full():
    sc = np.full((2, 10), 0.7)
    idx, counts, offsets = O.compact(sc, 0, 10, 0.7)
    assert idx.size == 0 and counts.tolist() == [0, 0] and offsets.tolist() == [0, 0, 0]
    idx, counts, offsets = O.compact(sc, 2, 6, 0.8)
    assert idx.tolist() == [2, 3, 4, 5, 2, 3, 4, 5] and offsets.tolist() == [0, 4, 8]


# --------------------------------------------------------------------------
# confidence
# --------------------------------------------------------------------------
def test_confidence_uniform_logits_tie_to_lowest_index():
    V, D = 37, 8
    mp, a, gap = O.confidence(np.ones((3, D)), np.zeros((V, D)))
    assert np.allclose(mp, 1.0 / V) and a.tolist() == [0, 0, 0] and np.all(gap == 0)


def test_confidence_closed_form_and_brute_force():
    V, D = 11, 4
    w = np.zeros((V, D))
    w[6, 0] = 1.0                      # logit of token 6 = x0, others 0
    x = np.array([[10.0, 0, 0, 0], [-3.0, 1, 2, 3]])
    mp, a, gap = O.confidence(x, w)
    assert a.tolist() == [6, 0]
    assert mp[0] == pytest.approx(math.exp(10) / (math.exp(10) + V - 1), rel=1e-14)
    assert mp[1] == pytest.approx(1.0 / (math.exp(-3) + V - 1), rel=1e-14)
    assert gap[0] == pytest.approx(10.0) and gap[1] == pytest.approx(0.0)
    rng = np.random.default_rng(3)
    x, w = rng.standard_normal((5, 6)), rng.standard_normal((9, 6))
    mp, a, _ = O.confidence(x, w)
    for r in range(5):
        z = [sum(x[r, d] * w[v, d] for d in range(6)) for v in range(9)]
        zm = max(z)
        assert a[r] == z.index(zm)
        assert mp[r] == pytest.approx(1.0 / sum(math.exp(t - zm) for t in z), rel=1e-12)


# --------------------------------------------------------------------------
# Q/K/V projection and scatter
# --------------------------------------------------------------------------
def test_qkv_identity_blocks_pin_head_and_block_order():
    B, S, Hq, Hkv, hd = 2, 6, 2, 1, 3
    D = Hq * hd
    rng = np.random.default_rng(4)
    x = rng.standard_normal((B, S, D))
    I = np.eye(D)
    w = np.concatenate([I, 2 * I[:hd], 3 * I[hd:2 * hd]])     # W_q = I, W_k = 2*(first hd dims), W_v = 3*(next hd)
    idx = np.array([1, 4, 0, 5], dtype=np.int32)
    offsets = np.array([0, 2, 4], dtype=np.int32)
    kc0 = rng.standard_normal((B, S, Hkv, hd))
    vc0 = rng.standard_normal((B, S, Hkv, hd))
    q, kc, vc = O.qkv_project_scatter(x, idx, offsets, w, Hq, Hkv, hd, kc0, vc0)
    assert np.allclose(q[0].reshape(-1), x[0, 1]) and np.allclose(q[3].reshape(-1), x[1, 5])
    assert np.allclose(q[1, 1], x[0, 4, hd:])             # head 1 = dims [hd, 2hd)
    assert np.allclose(kc[0, 4, 0], 2 * x[0, 4, :hd]) and np.allclose(vc[1, 0, 0], 3 * x[1, 0, hd:])
    untouched = np.ones((B, S), bool)
    untouched[0, [1, 4]] = untouched[1, [0, 5]] = False
    assert np.array_equal(kc[untouched], kc0[untouched]) and np.array_equal(vc[untouched], vc0[untouched])


def test_qkv_brute_force():
    B, S, D, Hq, Hkv, hd = 1, 4, 5, 2, 1, 2
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, S, D))
    w = rng.standard_normal(((Hq + 2 * Hkv) * hd, D))
    idx, offsets = np.array([0, 3], np.int32), np.array([0, 2], np.int32)
    q, kc, vc = O.qkv_project_scatter(x, idx, offsets, w, Hq, Hkv, hd,
                                      np.zeros((B, S, Hkv, hd)), np.zeros((B, S, Hkv, hd)))
    for r, i in enumerate([0, 3]):
        y = [sum(x[0, i, d] * w[n, d] for d in range(D)) for n in range(w.shape[0])]
        assert np.allclose(q[r].reshape(-1), y[:4], atol=1e-13)
        assert np.allclose(kc[0, i].reshape(-1), y[4:6], atol=1e-13)
        assert np.allclose(vc[0, i].reshape(-1), y[6:8], atol=1e-13)


# --------------------------------------------------------------------------
# partial attention
# --------------------------------------------------------------------------
def test_attention_brute_force_tiny():
    B, S, Hq, Hkv, hd = 2, 7, 4, 2, 3
    rng = np.random.default_rng(6)
    kc, vc = rng.standard_normal((2, B, S, Hkv, hd))
    idx = np.array([2, 6, 0, 1, 3], np.int32)
    offsets = np.array([0, 2, 5], np.int32)
    q = rng.standard_normal((5, Hq, hd))
    scale = 0.61
    o, lse = O.partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, scale)
    for b in range(B):
        for r in range(offsets[b], offsets[b + 1]):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                ob, lb = bf_attention_row(to_list(q[r, h]), to_list(kc[b, :, g]), to_list(vc[b, :, g]), scale)
                assert np.allclose(o[r, h], ob, atol=1e-13) and lse[r, h] == pytest.approx(lb, abs=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    hd = 4
    # one key: o = v, lse = scale * q.k
    k, v, q = rng.standard_normal((3, hd))
    o, lse = O.partial_attention(q[None, None], [0], [0, 1], k[None, None, None], v[None, None, None], 1, 1, 0.5)
    assert np.allclose(o[0, 0], v) and lse[0, 0] == pytest.approx(0.5 * q @ k)
    # identical keys: o = mean(V), lse = s + log S
    S = 6
    kc = np.tile(k, (1, S, 1, 1))
    vc = rng.standard_normal((1, S, 1, hd))
    o, lse = O.partial_attention(q[None, None], [0], [0, 1], kc, vc, 1, 1, 0.5)
    assert np.allclose(o[0, 0], vc[0, :, 0].mean(0)) and lse[0, 0] == pytest.approx(0.5 * q @ k + math.log(S))
    # q = 0: uniform weights, lse = log S
    o, lse = O.partial_attention(np.zeros((1, 1, hd)), [0], [0, 1], rng.standard_normal((1, S, 1, hd)), vc, 1, 1, 0.5)
    assert np.allclose(o[0, 0], vc[0, :, 0].mean(0)) and lse[0, 0] == pytest.approx(math.log(S))


def test_attention_gqa_head_map():
    # KV head 0 values all 1, KV head 1 values all 2: query heads 0,1 -> 1 and 2,3 -> 2
    B, S, Hq, Hkv, hd = 1, 5, 4, 2, 2
    rng = np.random.default_rng(8)
    kc = rng.standard_normal((B, S, Hkv, hd))
    vc = np.zeros((B, S, Hkv, hd))
    vc[:, :, 0] = 1.0
    vc[:, :, 1] = 2.0
    o, _ = O.partial_attention(rng.standard_normal((1, Hq, hd)), [3], [0, 1], kc, vc, Hq, Hkv, 1.0)
    assert np.allclose(o[0, :2], 1.0) and np.allclose(o[0, 2:], 2.0)


def test_full_selection_equals_library_dense_attention():
    """All positions selected: the step equals plain dense bidirectional attention
    computed by torch's CPU scaled_dot_product_attention in float64."""
    B, S, D, Hq, Hkv, hd = 2, 9, 12, 4, 2, 3
    rng = np.random.default_rng(9)
    x = rng.standard_normal((B, S, D))
    w = rng.standard_normal(((Hq + 2 * Hkv) * hd, D)) / 3
    idx = np.tile(np.arange(S, dtype=np.int32), B)
    offsets = np.arange(B + 1, dtype=np.int32) * S
    z = np.zeros((B, S, Hkv, hd))
    q, kc, vc = O.qkv_project_scatter(x, idx, offsets, w, Hq, Hkv, hd, z, z)
    o, _ = O.partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, 1 / math.sqrt(hd))
    xt = torch.tensor(x)
    y = xt @ torch.tensor(w).T
    Q = y[..., :Hq * hd].reshape(B, S, Hq, hd).transpose(1, 2)
    K = y[..., Hq * hd:(Hq + Hkv) * hd].reshape(B, S, Hkv, hd).transpose(1, 2)
    V = y[..., (Hq + Hkv) * hd:].reshape(B, S, Hkv, hd).transpose(1, 2)
    K = K.repeat_interleave(Hq // Hkv, dim=1)
    V = V.repeat_interleave(Hq // Hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).transpose(1, 2).reshape(B * S, Hq, hd)
    assert np.allclose(o, ref.numpy(), atol=1e-12)


def test_zero_selection_returns_cache():
    rng = np.random.default_rng(10)
    B, S, D, Hq, Hkv, hd = 1, 8, 6, 2, 2, 3
    cur = rng.standard_normal((B, S, D))
    w = rng.standard_normal(((Hq + 2 * Hkv) * hd, D))
    kc, vc, out = (rng.standard_normal((B, S, Hkv, hd)), rng.standard_normal((B, S, Hkv, hd)),
                   rng.standard_normal((B, S, Hq * hd)))
    r = O.cosine_step(cur, cur, w, Hq, Hkv, hd, tau=0.5, k_cache=kc, v_cache=vc, out_cache=out)
    assert r["idx"].size == 0
    assert np.array_equal(r["k_cache"], kc) and np.array_equal(r["v_cache"], vc) and np.array_equal(r["out_cache"], out)


def test_full_selection_step_equals_full_recompute():
    rng = np.random.default_rng(11)
    B, S, D, Hq, Hkv, hd = 2, 6, 8, 2, 1, 4
    cur = rng.standard_normal((B, S, D))
    w = rng.standard_normal(((Hq + 2 * Hkv) * hd, D)) / 2
    wo = rng.standard_normal((5, Hq * hd))
    junk = lambda *s: rng.standard_normal(s)
    r = O.cosine_step(cur, -cur, w, Hq, Hkv, hd, tau=0.5, k_cache=junk(B, S, Hkv, hd),
                      v_cache=junk(B, S, Hkv, hd), out_cache=junk(B, S, 5), w_o=wo)
    kc, vc, out = O.full_recompute_caches(cur, w, Hq, Hkv, hd, 1 / math.sqrt(hd), wo)
    assert r["counts"].tolist() == [S, S]
    assert np.allclose(r["k_cache"], kc) and np.allclose(r["out_cache"], out, atol=1e-12)


def test_output_scatter_with_wo_brute_force():
    rng = np.random.default_rng(12)
    o = rng.standard_normal((2, 2, 3))
    wo = rng.standard_normal((4, 6))
    out0 = rng.standard_normal((1, 5, 4))
    out = O.output_scatter(o, np.array([1, 3], np.int32), np.array([0, 2], np.int32), out0, wo)
    for r, i in enumerate([1, 3]):
        ctx = o[r].reshape(-1).tolist()
        y = [sum(ctx[c] * wo[n, c] for c in range(6)) for n in range(4)]
        assert np.allclose(out[0, i], y, atol=1e-13)
    assert np.array_equal(out[0, [0, 2, 4]], out0[0, [0, 2, 4]])


# --------------------------------------------------------------------------
# column sums and top-k
# --------------------------------------------------------------------------
def _attn_inputs(B, S, nq, Hq, Hkv, hd, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B * nq, Hq, hd))
    kc = rng.standard_normal((B, S, Hkv, hd))
    vc = rng.standard_normal((B, S, Hkv, hd))
    idx = np.tile(np.arange(S - nq, S, dtype=np.int32), B)
    offsets = np.arange(B + 1, dtype=np.int32) * nq
    return q, kc, vc, idx, offsets


def _dv_case(seed, B=2, S=7, Hq=4, Hkv=2, hd=3, sal=((1, 4), (0, 2, 6))):
    """Previous step: every position computed exactly (pure-Python softmax over
    the old K/V).  This step: the salient rows A get new K and new V."""
    rng = np.random.default_rng(seed)
    k_old_c, v_old_c = rng.standard_normal((2, B, S, Hkv, hd))
    q = rng.standard_normal((B, S, Hq, hd))
    scale = 0.7
    G = Hq // Hkv
    o = np.zeros((B, S, Hq, hd))
    lse = np.zeros((B, S, Hq))
    for b in range(B):
        for i in range(S):
            for h in range(Hq):
                ob, lb = bf_attention_row(to_list(q[b, i, h]), to_list(k_old_c[b, :, h // G]),
                                          to_list(v_old_c[b, :, h // G]), scale)
                o[b, i, h], lse[b, i, h] = ob, lb
    idx = np.concatenate([np.array(a, np.int32) for a in sal])
    offsets = np.concatenate([[0], np.cumsum([len(a) for a in sal])]).astype(np.int32)
    k_new_c, v_new_c = k_old_c.copy(), v_old_c.copy()
    for b in range(B):
        for i in sal[b]:
            k_new_c[b, i] = rng.standard_normal((Hkv, hd))
            v_new_c[b, i] = rng.standard_normal((Hkv, hd))
    k_old = O.gather_rows(k_old_c, idx, offsets)
    v_old = O.gather_rows(v_old_c, idx, offsets)
    return dict(q=q, lse=lse, o=o, idx=idx, offsets=offsets, k_old=k_old, v_old=v_old, k_old_c=k_old_c,
                v_new_c=v_new_c, k_new_c=k_new_c, scale=scale, Hq=Hq, Hkv=Hkv, sal=sal)


def _dv(c, v_cache=None, idx=None, offsets=None, k_old=None, v_old=None):
    return O.nonsalient_dv_update(c["q"], c["lse"], c["idx"] if idx is None else idx,
                                  c["offsets"] if offsets is None else offsets,
                                  c["k_old"] if k_old is None else k_old,
                                  c["v_old"] if v_old is None else v_old,
                                  c["v_new_c"] if v_cache is None else v_cache, c["o"], c["Hq"], c["Hkv"],
                                  c["scale"])


def test_dv_update_equals_old_weights_on_new_values():
    """With its existing weights (the old keys' softmax) held fixed, a stable
    row's exact output on the new values is sum_j P_old(j) v_new(j) over all
    keys; the update reaches exactly that, although the salient rows' K changed
    too (pure-Python softmax per row).  Salient rows are left as given."""
    c = _dv_case(12)
    out = _dv(c)
    G = c["Hq"] // c["Hkv"]
    for b, sal in enumerate(c["sal"]):
        for i in range(out.shape[1]):
            for h in range(c["Hq"]):
                if i in sal:
                    assert np.array_equal(out[b, i, h], c["o"][b, i, h])
                    continue
                ref, _ = bf_attention_row(to_list(c["q"][b, i, h]), to_list(c["k_old_c"][b, :, h // G]),
                                          to_list(c["v_new_c"][b, :, h // G]), c["scale"])
                assert np.allclose(out[b, i, h], ref, atol=1e-12)
    # the new keys are not what the weights use: with them the result differs
    k_new = O.gather_rows(c["k_new_c"], c["idx"], c["offsets"])
    assert not np.allclose(_dv(c, k_old=k_new), out, atol=1e-6)


def test_dv_update_invariants():
    c = _dv_case(13)
    # unchanged values: nothing moves, whatever the keys did
    v_same = O.scatter_rows(c["v_old"], c["idx"], c["offsets"], c["v_new_c"])
    assert np.allclose(_dv(c, v_cache=v_same), c["o"], atol=1e-15)
    # empty salient set: nothing moves
    e = np.zeros(0, np.int32)
    assert np.array_equal(_dv(c, idx=e, offsets=np.zeros(3, np.int32), k_old=np.zeros((0, 2, 3)),
                              v_old=np.zeros((0, 2, 3))), c["o"])
    # linear in the value change: two halves of the change add up
    v_half = O.scatter_rows(0.5 * (O.gather_rows(c["v_new_c"], c["idx"], c["offsets"]) + c["v_old"]),
                            c["idx"], c["offsets"], c["v_new_c"])
    d_full = _dv(c) - c["o"]
    d_half = _dv(c, v_cache=v_half) - c["o"]
    assert np.allclose(d_full, 2 * d_half, atol=1e-12)
    # GQA head map: a change on KV head 1 only moves query heads 2 and 3
    v1 = v_same.copy()
    for b, sal in enumerate(c["sal"]):
        v1[b, list(sal), 1] += 1.0
    d = _dv(c, v_cache=v1) - c["o"]
    assert np.array_equal(d[:, :, :2], np.zeros_like(d[:, :, :2])) and np.abs(d[:, :, 2:]).max() > 1e-3


def test_gather_scatter_rows_brute_force():
    rng = np.random.default_rng(14)
    B, S, W = 3, 6, 5
    src = rng.standard_normal((B, S, W))
    idx = np.array([5, 0, 2, 3], np.int32)
    offsets = np.array([0, 1, 1, 4], np.int32)
    g = O.gather_rows(src, idx, offsets)
    assert g.shape == (4, W)
    for r, (b, i) in enumerate([(0, 5), (2, 0), (2, 2), (2, 3)]):
        assert to_list(g[r]) == to_list(src[b, i])
    dst = rng.standard_normal((B, S, W))
    out = O.scatter_rows(g, idx, offsets, dst)
    for b in range(B):
        for i in range(S):
            want = src[b, i] if (b, i) in [(0, 5), (2, 0), (2, 2), (2, 3)] else dst[b, i]
            assert to_list(out[b, i]) == to_list(want)


def test_salient_ffn_brute_force_and_library():
    """Pure-Python brute force on a tiny case, and torch's CPU silu/matmul in
    float64 with all rows selected; unselected rows keep the cache."""
    rng = np.random.default_rng(15)
    B, S, D, F = 2, 5, 4, 3
    x = rng.standard_normal((B, S, D))
    wgu = rng.standard_normal((2 * F, D))
    wd = rng.standard_normal((D, F))
    cache = rng.standard_normal((B, S, D))
    idx = np.array([4, 1, 3], np.int32)
    offsets = np.array([0, 1, 3], np.int32)
    h, out = O.salient_ffn(x, idx, offsets, wgu, wd, cache)
    sel = [(0, 4), (1, 1), (1, 3)]
    for r, (b, i) in enumerate(sel):
        xr = to_list(x[b, i])
        hh = []
        for f in range(F):
            gte = sum(a * w for a, w in zip(xr, to_list(wgu[2 * f])))
            up = sum(a * w for a, w in zip(xr, to_list(wgu[2 * f + 1])))
            hh.append(gte / (1 + math.exp(-gte)) * up)
        assert np.allclose(h[r], hh, atol=1e-13)
        y = [sum(hh[f] * wd[d, f] for f in range(F)) for d in range(D)]
        assert np.allclose(out[b, i], y, atol=1e-12)
    for b in range(B):
        for i in range(S):
            if (b, i) not in sel:
                assert np.array_equal(out[b, i], cache[b, i])
    # every row selected: torch's silu and matmul on the whole batch
    idx_all = np.tile(np.arange(S, dtype=np.int32), B)
    off_all = np.arange(B + 1, dtype=np.int32) * S
    _, out_all = O.salient_ffn(x, idx_all, off_all, wgu, wd, cache)
    xt = torch.tensor(x)
    ref = (torch.nn.functional.silu(xt @ torch.tensor(wgu[0::2]).T) * (xt @ torch.tensor(wgu[1::2]).T)) @ torch.tensor(wd).T
    assert np.allclose(out_all, ref.numpy(), atol=1e-12)


def test_salient_ffn_closed_forms():
    """silu(0) = 0 (a zero gate zeroes the row); a unit up row and identity-like
    down weights make y_d = silu(g_d); an empty selection returns the cache."""
    rng = np.random.default_rng(16)
    B, S, D = 1, 3, 2
    x = rng.standard_normal((B, S, D))
    cache = rng.standard_normal((B, S, D))
    wgu = np.zeros((4, D))
    wgu[1] = rng.standard_normal(D)
    wgu[3] = rng.standard_normal(D)
    h, _ = O.salient_ffn(x, [0, 1, 2], [0, 3], wgu, np.eye(D), cache)
    assert np.array_equal(h, np.zeros_like(h))
    # gate f = x_f, up = 1 (a constant input column), down = identity
    x1 = np.concatenate([x, np.ones((B, S, 1))], axis=2)
    wgu = np.zeros((2 * D, D + 1))
    for f in range(D):
        wgu[2 * f, f] = 1.0
        wgu[2 * f + 1, D] = 1.0
    wd = np.zeros((D + 1, D))
    wd[:D, :D] = np.eye(D)
    _, out = O.salient_ffn(x1, [0, 2], [0, 2], wgu, wd, np.zeros((B, S, D + 1)))
    for i in (0, 2):
        assert np.allclose(out[0, i, :D], x[0, i] / (1 + np.exp(-x[0, i])), atol=1e-15)
    assert np.array_equal(out[0, 1], np.zeros(D + 1))
    _, out = O.salient_ffn(x, np.zeros(0, np.int32), [0, 0], np.ones((4, D)), np.ones((D, 2)), cache)
    assert np.array_equal(out, cache)


def test_logit_margin_brute_force_and_ties():
    rng = np.random.default_rng(17)
    rows = rng.standard_normal((5, 6))
    w = rng.standard_normal((9, 6))
    m, a = O.logit_margin(rows, w)
    for r in range(5):
        z = [sum(x * y for x, y in zip(to_list(rows[r]), to_list(w[v]))) for v in range(9)]
        zs = sorted(z, reverse=True)
        assert m[r] == pytest.approx(zs[0] - zs[1], abs=1e-13) and a[r] == z.index(zs[0])
    # a maximum attained twice: margin 0, argmax the lower index
    w2 = np.zeros((4, 2))
    w2[1] = w2[3] = [1.0, 0.0]
    m, a = O.logit_margin(np.array([[2.0, 1.0]]), w2)
    assert m[0] == 0.0 and a[0] == 1


def bf_lsp(margins, committed, G, frac_lo, frac_hi):
    """Brute force: try every candidate threshold (each margin value) and keep
    the largest one whose leading stable run reaches lo."""
    A = G - committed
    if A <= 0:
        return committed, None
    act = margins[committed:]
    lo = max(1, math.ceil(frac_lo * A))
    hi = max(lo, math.floor(frac_hi * A))
    best = None
    for t in sorted(set(act), reverse=True):
        run = 0
        while run < A and act[run] >= t:
            run += 1
        if run >= lo:
            best = (t, run)
            break
    return committed + min(best[1], hi), best[0]


def test_lsp_adaptive_commit_brute_force():
    rng = np.random.default_rng(18)
    B, S, lo_g = 6, 40, 8
    G = S - lo_g
    for trial in range(20):
        m = np.round(rng.standard_normal((B, S)) * 3, 1).astype(np.float32)   # ties on purpose
        com = rng.integers(0, G + 1, B)
        fl, fh = [(0.25, 0.5), (0.1, 0.3), (0.5, 0.5)][trial % 3]
        out, tau = O.lsp_adaptive_commit(m, lo_g, S, com, fl, fh)
        for b in range(B):
            want, t = bf_lsp([float(x) for x in m[b, lo_g:]], int(com[b]), G, fl, fh)
            assert out[b] == want
            assert (t is None and np.isnan(tau[b])) or tau[b] == t


def test_lsp_adaptive_commit_closed_forms():
    # strictly decreasing margins over A = 8 active: tau = 2nd margin, block = lo = 2
    m = np.array([[9.0, 8, 7, 6, 5, 4, 3, 2]], np.float32)
    out, tau = O.lsp_adaptive_commit(m, 0, 8, [0])
    assert out[0] == 2 and tau[0] == 8.0
    # all equal: every position is stable under tau, the block is cut at hi = 4
    out, _ = O.lsp_adaptive_commit(np.ones((1, 8), np.float32), 0, 8, [0])
    assert out[0] == 4
    # one active position: it is committed (the fallback); none active: unchanged
    out, tau = O.lsp_adaptive_commit(np.zeros((1, 8), np.float32), 0, 8, [7])
    assert out[0] == 8
    out, tau = O.lsp_adaptive_commit(np.zeros((1, 8), np.float32), 0, 8, [8])
    assert out[0] == 8 and np.isnan(tau[0])
    # the geometric shrink: repeated commits on equal margins take half each time
    c, seen = 0, []
    while c < 64:
        c = int(O.lsp_adaptive_commit(np.ones((1, 64), np.float32), 0, 64, [c])[0][0])
        seen.append(c)
    assert seen[:4] == [32, 48, 56, 60]


def test_lsp_margin_floor():
    """The optional floor: below every margin it changes nothing; above the
    first active margin only the fallback commits (exactly one position); in
    between it cuts the block at the first margin under it (fewer than lo
    positions can then be committed), against a brute force over every
    candidate threshold that counts only margins at or above the floor as
    stable."""
    def bf_floor(margins, committed, G, fl, fh, floor):
        A = G - committed
        if A <= 0:
            return committed, None
        act = margins[committed:]
        lo, hi = max(1, math.ceil(fl * A)), max(max(1, math.ceil(fl * A)), math.floor(fh * A))
        for t in sorted(set(act), reverse=True):
            run = 0
            while run < A and act[run] >= t:
                run += 1
            if run >= lo:
                break
        if t >= floor:
            return committed + min(run, hi), t
        run = 0
        while run < A and act[run] >= floor:
            run += 1
        return committed + max(1, min(run, hi)), floor

    rng = np.random.default_rng(19)
    B, S, g0 = 6, 40, 8
    G = S - g0
    for trial in range(30):
        m = np.round(np.abs(rng.standard_normal((B, S))) * 3, 1).astype(np.float32)
        com = rng.integers(0, G + 1, B)
        fl, fh = [(0.25, 0.5), (0.1, 0.3), (0.5, 0.5)][trial % 3]
        floor = float([0.0, 1.5, 2.5, 9.0][trial % 4])
        out, tau = O.lsp_adaptive_commit(m, g0, S, com, fl, fh, margin_floor=floor)
        for b in range(B):
            want, t = bf_floor([float(x) for x in m[b, g0:]], int(com[b]), G, fl, fh, floor)
            assert out[b] == want and ((t is None and np.isnan(tau[b])) or tau[b] == t)
    m = np.array([[9.0, 8, 7, 6, 5, 4, 3, 2]], np.float32)
    assert O.lsp_adaptive_commit(m, 0, 8, [0], margin_floor=1.0)[0][0] == 2        # below every margin
    assert O.lsp_adaptive_commit(m, 0, 8, [0], margin_floor=100.0)[0][0] == 1      # only the fallback
    m2 = np.array([[9.0, 1, 9, 9, 9, 9, 9, 9]], np.float32)
    assert O.lsp_adaptive_commit(m2, 0, 8, [0], margin_floor=5.0)[0][0] == 1       # cut by the floor
    assert O.lsp_adaptive_commit(m2, 0, 8, [0])[0][0] == 4                          # no floor: tau = 1


def test_colsum_sum_invariant_and_library_softmax():
    B, S, nq, Hq, Hkv, hd = 2, 11, 6, 4, 2, 3
    q, kc, vc, idx, offsets = _attn_inputs(B, S, nq, Hq, Hkv, hd, 13)
    scale = 0.7
    _, lse = O.partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, scale)
    c = O.column_sums(q, offsets, kc, lse, Hq, Hkv, scale)
    assert np.allclose(c.sum(axis=1), Hq * nq, atol=1e-12)          # each query row sums to 1 per head
    for b in range(B):
        Q = torch.tensor(q[b * nq:(b + 1) * nq]).transpose(0, 1)      # [Hq, nq, hd]
        K = torch.tensor(kc[b]).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)
        P = torch.softmax(scale * Q @ K.transpose(1, 2), dim=-1)      # [Hq, nq, S]
        assert np.allclose(c[b], P.sum(dim=(0, 1)).numpy(), atol=1e-12)


def test_colsum_zero_queries_uniform_and_topk_tiebreak():
    B, S, nq, Hq, Hkv, hd = 2, 16, 12, 3, 3, 4
    q, kc, vc, idx, offsets = _attn_inputs(B, S, nq, Hq, Hkv, hd, 14)
    q[:] = 0.0
    _, lse = O.partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, 0.5)
    c = O.column_sums(q, offsets, kc, lse, Hq, Hkv, 0.5)
    assert np.allclose(c, Hq * nq / S, atol=1e-13)
    ti, tv = O.topk_keys(np.full((B, S), Hq * nq / S), 4, 16, 5)       # all equal -> lowest indices
    assert ti.tolist() == [[4, 5, 6, 7, 8]] * 2


def test_topk_brute_force():
    rng = np.random.default_rng(15)
    c = rng.integers(0, 4, size=(3, 20)).astype(np.float64)          # many ties
    ti, tv = O.topk_keys(c, 3, 18, 7)
    for b in range(3):
        exp = sorted(range(3, 18), key=lambda j: (-c[b, j], j))[:7]
        assert ti[b].tolist() == exp and tv[b].tolist() == [c[b, j] for j in exp]


# --------------------------------------------------------------------------
# stable prefix
# --------------------------------------------------------------------------
def bf_prefix(argmax_hist, maxprob, L, conf, min_commit, S_gen, W):
    """Brute force: argmax_hist is the list of per-step argmax rows (carry-forward
    already applied), newest last."""
    last = argmax_hist[-W:]
    if len(last) < W:
        last = [[-1] * S_gen] * (W - len(last)) + last
    i = L
    while i < S_gen:
        col = [row[i] for row in last]
        if not (all(v == col[0] for v in col) and col[0] != -1 and maxprob[i] >= conf):
            break
        i += 1
    if min_commit and i == L and L < S_gen:
        i = L + 1
    return i


def test_stable_prefix_brute_force_random_histories():
    rng = np.random.default_rng(16)
    B, S, gen_lo, W = 4, 30, 6, 3
    S_gen = S - gen_lo
    for trial in range(20):
        ring = np.full((B, S_gen, W), -1, np.int64)
        committed = np.zeros(B, np.int64)
        hist = [[] for _ in range(B)]
        min_commit = trial % 2
        for t in range(6):
            am = rng.integers(0, 2, size=(B, S)).astype(np.int64)     # few tokens -> frequent repeats
            mp = rng.choice([0.5, 0.9, 0.95], size=(B, S))
            ring, new = O.stable_prefix_step(am, mp, ring, t, gen_lo, S, 0.9, min_commit, committed)
            for b in range(B):
                hist[b].append(am[b, gen_lo:].tolist())
                exp = bf_prefix(hist[b], mp[b, gen_lo:].tolist(), int(committed[b]), 0.9, min_commit, S_gen, W)
                assert new[b] == exp
            committed = new


def test_stable_prefix_closed_forms():
    B, S, W = 2, 10, 3
    ring = np.full((B, S, W), 7, np.int64)
    am = np.full((B, S), 7)
    mp = np.full((B, S), 0.95)
    _, new = O.stable_prefix_step(am, mp, ring, 5, 0, S, 0.9, 0, np.array([0, 4]))
    assert new.tolist() == [S, S]                                    # all stable
    mp[:] = 0.5
    _, new = O.stable_prefix_step(am, mp, ring, 5, 0, S, 0.9, 0, np.array([3, S]))
    assert new.tolist() == [3, S]                                    # none stable
    _, new = O.stable_prefix_step(am, mp, ring, 5, 0, S, 0.9, 1, np.array([3, S]))
    assert new.tolist() == [4, S]                                    # fallback commits one, never past S_gen
    mp[:] = 0.9
    _, new = O.stable_prefix_step(am, mp, ring, 5, 0, S, 0.9, 0, np.array([0, 0]))
    assert new.tolist() == [S, S]                                    # >= is inclusive


def test_admissible_frontiers():
    st = np.array([1, 1, 2, 1, 0, 1])
    assert O.admissible_frontiers({0}, st, 6, 0) == {2, 4}
    assert O.admissible_frontiers({4}, st, 6, 1) == {5}
    assert O.admissible_frontiers({5}, st, 6, 0) == {6}


def test_lsp_planted_closed_form():
    """Planted rows before P_b have a dominant token: argmax = target and
    max-prob >= 0.9; row P_b is diffuse.  Then L_t = min(P_b, first i >= L_{t-1}
    whose first evaluation step e_i > t-2)."""
    D = 256
    sh = W.LspShape(**{**W.LSP_COMMIT.__dict__, "B": 3, "S": 160, "prompt": 32, "D": D, "V": 2048,
                       "w_std": 0.02 * math.sqrt(4096 / D), "steps": 8})
    inp = W.lsp_inputs(sh)
    S_gen = inp.S_gen
    ring = np.full((sh.B, S_gen, sh.W), -1, np.int64)
    argmax = np.full((sh.B, sh.S), -1, np.int64)
    maxprob = np.zeros((sh.B, sh.S))
    committed = np.zeros(sh.B, np.int64)
    first_eval = np.full((sh.B, S_gen), 10 ** 9)
    for t in range(sh.steps):
        h = inp.hidden(t)
        rows = inp.active_rows(t)
        for b in range(sh.B):
            mp, a, _ = O.confidence(h[b, rows[b]], inp.w_lm)
            argmax[b, rows[b]] = a
            maxprob[b, rows[b]] = mp
            g = rows[b] - sh.prompt
            first_eval[b, g] = np.minimum(first_eval[b, g], t)
            planted = g < inp.frontier[b]
            assert np.array_equal(a[planted], inp.targets[b, g[planted]])
            assert np.all(mp[planted] >= 0.9)
            assert np.all(mp[g == inp.frontier[b]] < 0.9)
        ring, new = O.stable_prefix_step(argmax, maxprob, ring, t, sh.prompt, sh.S, sh.conf, 0, committed)
        for b in range(sh.B):
            i = int(committed[b])
            while i < S_gen and first_eval[b, i] <= t - 2:
                i += 1
            assert new[b] == min(int(inp.frontier[b]), i)
        committed = new
    assert committed.max() > 0


# --------------------------------------------------------------------------
# hand-derived fixtures
# --------------------------------------------------------------------------
def test_golden_hand_fixtures():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        cases = json.load(f)
    for c in cases["attention"]:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, :, None]
        v = np.array(c["v"], dtype=np.float64)[None, :, None]
        o, lse = O.partial_attention(q, [0], [0, 1], k, v, 1, 1, c["scale"])
        assert np.allclose(o[0, 0], c["o"], atol=1e-12), c["name"]
        assert lse[0, 0] == pytest.approx(c["lse"], abs=1e-12), c["name"]
    for c in cases["cosine"]:
        assert O.cosine_scores(np.array(c["a"]), np.array(c["b"])) == pytest.approx(c["cos"], abs=1e-15)
    for c in cases["colsum"]:
        q = np.array(c["q"], dtype=np.float64)[:, None]
        k = np.array(c["k"], dtype=np.float64)[None, :, None]
        nq = q.shape[0]
        v = np.zeros_like(k)
        _, lse = O.partial_attention(q, list(range(nq)), [0, nq], k, v, 1, 1, c["scale"])
        col = O.column_sums(q, [0, nq], k, lse, 1, 1, c["scale"])
        assert np.allclose(col[0], c["c"], atol=1e-12), c["name"]


# --------------------------------------------------------------------------
# SureLock: local KL divergence and the lock decision
# --------------------------------------------------------------------------
def _kl_brute(zt, zp):
    """Pure-Python KL(p_t || p_p) of one position's logit lists."""
    mt, mp_ = max(zt), max(zp)
    st = sum(math.exp(z - mt) for z in zt)
    sp = sum(math.exp(z - mp_) for z in zp)
    out = 0.0
    for a, b in zip(zt, zp):
        lpa = a - mt - math.log(st)
        lpb = b - mp_ - math.log(sp)
        out += math.exp(lpa) * (lpa - lpb)
    return out


def test_kl_brute_force_and_library():
    """Against a pure-Python sum over the vocabulary and scipy's relative
    entropy of the two softmax distributions (argument order matters)."""
    from scipy.special import softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(81)
    n, D, V = 6, 16, 40
    xt, xp = rng.standard_normal((n, D)), rng.standard_normal((n, D))
    xp[0] = xt[0] + 0.05 * rng.standard_normal(D)
    w = rng.standard_normal((V, D)) * 0.5
    kl, mp, a, gap = O.kl_divergence(xt, xp, w)
    zt, zp = xt @ w.T, xp @ w.T
    for r in range(n):
        assert abs(kl[r] - _kl_brute(zt[r].tolist(), zp[r].tolist())) < 1e-12
        assert abs(kl[r] - entropy(softmax(zt[r]), softmax(zp[r]))) < 1e-12
        assert a[r] == int(np.argmax(zt[r])) and abs(mp[r] - softmax(zt[r]).max()) < 1e-15
    rev, _, _, _ = O.kl_divergence(xp, xt, w)
    assert np.all(kl >= 0) and np.max(np.abs(kl - rev)) > 1e-3   # asymmetric: the order is pinned
    assert kl[0] < kl[1:].min()


def test_kl_closed_forms():
    """Equal posteriors give 0 (also when every logit moves by one constant);
    two tokens with logits (a, 0) against (0, 0): KL = p log 2p + (1-p) log 2(1-p)
    with p = sigmoid(a)."""
    rng = np.random.default_rng(82)
    D, V = 8, 30
    w = rng.standard_normal((V, D))
    w[:, 0] = 1.0                                    # a constant column: x + c e0 shifts every logit by c
    x = rng.standard_normal((3, D))
    xs = x.copy()
    xs[:, 0] += np.array([0.0, 2.5, -7.0])
    kl, _, _, _ = O.kl_divergence(x, x, w)
    assert np.all(kl == 0.0)
    kl, _, _, _ = O.kl_divergence(x, xs, w)
    assert np.max(np.abs(kl)) < 1e-12
    for a in (0.3, 2.0, -4.0):
        w2 = np.array([[1.0], [0.0]])
        kl, mp, am, _ = O.kl_divergence(np.array([[a]]), np.array([[0.0]]), w2)
        p = 1.0 / (1.0 + math.exp(-a))
        assert abs(kl[0] - (p * math.log(2 * p) + (1 - p) * math.log(2 * (1 - p)))) < 1e-14
        assert abs(mp[0] - max(p, 1 - p)) < 1e-15 and am[0] == (0 if a > 0 else 1)


def _lock_brute(kl, mp, rows_per_b, locked, eps, q):
    """The lock rule with the uncertainties 1 - p in exact rational arithmetic
    and the nearest-rank percentile taken on them."""
    from fractions import Fraction
    out = np.array(locked, copy=True)
    for b, rows in enumerate(rows_per_b):
        if len(rows) == 0:
            continue
        u = {i: 1 - Fraction(float(mp[b, i])) for i in rows}
        if q > 0:
            k = max(1, math.ceil(float(q) * len(rows)))
            pq = sorted(u.values())[min(k, len(rows)) - 1]
        for i in rows:
            if kl[b, i] < eps and (q <= 0 or u[i] <= pq):
                out[b, i] = 1
    return out


def test_surelock_lock_brute_force():
    rng = np.random.default_rng(83)
    B, S = 4, 60
    for q in (0.0, 0.3, 0.5, 1.0, np.float32(0.7)):
        kl = rng.choice(np.array([0.0, 0.01, 0.02, 0.05, 0.3], np.float32), size=(B, S))
        mp = rng.choice(np.array([0.2, 0.5, 0.9, 0.95, 0.999], np.float32), size=(B, S))
        rows = [np.sort(rng.choice(S, m, replace=False)) for m in (20, 0, 33, 7)]
        idx, off = W.pack_rows(rows)
        locked = (rng.random((B, S)) < 0.2).astype(np.float32)
        got = O.surelock_lock(kl, mp, idx, off, locked, np.float32(0.02), q)
        want = _lock_brute(kl, mp, rows, locked, np.float32(0.02), q)
        assert np.array_equal(got, want), f"q={q}"
        assert np.all(got >= locked)                                  # locks are permanent
        mask = np.zeros((B, S), bool)
        for b, r in enumerate(rows):
            mask[b, r] = True
        assert np.array_equal(got[~mask], locked[~mask])              # only evaluated positions move


def test_surelock_lock_closed_forms():
    """Strict KL threshold; no gate: lock iff kl < eps; q = 1: the gate passes
    everything; a small q: only the most confident position(s) pass (ties at
    the percentile value all pass)."""
    kl = np.array([[0.0, 0.01, 0.02, 0.03, 0.0, 0.0]], np.float32)
    mp = np.array([[0.9, 0.99, 0.5, 0.99, 0.99, 0.7]], np.float32)
    idx, off = W.pack_rows([np.arange(6)])
    z = np.zeros((1, 6), np.float32)
    eps = np.float32(0.02)
    assert O.surelock_lock(kl, mp, idx, off, z, eps, 0.0).tolist() == [[1, 1, 0, 0, 1, 1]]
    assert O.surelock_lock(kl, mp, idx, off, z, eps, 1.0).tolist() == [[1, 1, 0, 0, 1, 1]]
    # k = ceil(0.1 * 6) = 1: the largest max p is 0.99 (three positions tie)
    assert O.surelock_lock(kl, mp, idx, off, z, eps, 0.1).tolist() == [[0, 1, 0, 0, 1, 0]]
    # k = 4: the 4th largest is 0.9
    assert O.surelock_lock(kl, mp, idx, off, z, eps, 0.6).tolist() == [[1, 1, 0, 0, 1, 0]]
