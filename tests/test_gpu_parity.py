"""Parity of the HIP path (through the C ABI) with the fp64 oracle on the same
seeded inputs, element by element.

Bars: index sets exact outside the 1e-4 threshold band; float outputs within
1e-4 (fp32 storage) or 2e-2 (bf16 storage) max-abs; cache rows that a step does
not select must be byte-identical.  Downstream calls receive the oracle's index
set, so each stage is compared on identical inputs."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import dlm_oracle as O
from sparse_query_attention_dlm_amd import workloads as W
from helpers import (BAND, TOL, check_selection, check_topk, dev, host, i32, maxabs, rows_mask,
                     workspace)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dlm():
    from sparse_query_attention_dlm_amd import binding
    return binding


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# cosine-selected single steps (tiny fp32 layer, bf16 S=1024 layer)
# ---------------------------------------------------------------------------
def run_cosine_step(dlm, shape, tau=None, bound=None, lo=0, hi=None, **override):
    """One cosine-selected step (select -> Q/K/V + K/V scatter -> partial
    attention + output scatter) against the oracle.  bound: the host-side row
    bound passed to the Q/K/V and attention calls (None = the exact count;
    "loose" = B*S, as a caller that does not know the count passes it).
    [lo, hi): the scored window."""
    inp = W.cosine_step_inputs(shape, **override)
    s = inp.shape
    dt = s.dtype
    tau = s.tau if tau is None else tau
    scale = 1.0 / math.sqrt(s.hd)
    hi = s.S if hi is None else hi
    say(f"[cosine step] {s.name} B={s.B} S={s.S} D={s.D} Hq={s.Hq} Hkv={s.Hkv} tau={tau} "
        f"bound={bound} window=[{lo},{hi})")
    kc0, vc0, out0 = O.full_recompute_caches(inp.prev, inp.w_qkv, s.Hq, s.Hkv, s.hd, scale, inp.w_o)
    kc0, vc0, out0 = (W.to_storage(a, dt) for a in (kc0, vc0, out0))
    ref = O.cosine_step(inp.cur, inp.prev, inp.w_qkv, s.Hq, s.Hkv, s.hd, tau, kc0, vc0, out0, w_o=inp.w_o,
                        lo=lo, hi=hi)

    cur, prev = dev(inp.cur, dt), dev(inp.prev, dt)
    B, S = s.B, s.S
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    ws = workspace(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_COSINE, B, S))
    scores.fill_(-7.0)
    dlm.dlm_saliency_select(dlm.DLM_SCORE_COSINE, cur, prev, lo=lo, hi=hi, threshold=tau, idx=idx,
                            counts=counts, offsets=offsets, scores=scores, workspace=ws)
    torch.cuda.synchronize()
    sc_g = host(scores)
    assert maxabs(sc_g[:, lo:hi], ref["scores"][:, lo:hi]) <= 1e-5
    assert np.all(sc_g[:, :lo] == -7.0) and np.all(sc_g[:, hi:] == -7.0), "scores written outside the window"
    off_g = offsets.cpu().numpy()
    check_selection(idx.cpu().numpy(), counts.cpu().numpy(), off_g, ref["scores"], lo, hi, tau)

    n = int(ref["offsets"][-1])
    max_rows = n if bound is None else (B * S if bound == "loose" else int(bound))
    idx_o, off_o = i32(ref["idx"]), i32(ref["offsets"])
    q = torch.zeros(max(max_rows, 1), s.Hq, s.hd, dtype=cur.dtype, device="cuda")
    kc, vc = dev(kc0, dt), dev(vc0, dt)
    dcode = dlm.DLM_BF16 if dt == "bf16" else dlm.DLM_F32
    wsq = workspace(dlm.dlm_gather_qkv_workspace_size(dcode, max_rows, s.D, s.Hq, s.Hkv, s.hd))
    dlm.dlm_gather_qkv_scatter_kv(cur, idx_o, off_o, max_rows, dev(inp.w_qkv, dt), s.Hq, s.Hkv, s.hd, q, kc, vc,
                                  workspace=wsq)
    o = torch.zeros_like(q)
    lse = torch.zeros(max(max_rows, 1), s.Hq, dtype=torch.float32, device="cuda")
    out = dev(out0, dt)
    wo = dev(inp.w_o, dt) if inp.w_o is not None else None
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(
        dcode, max(max_rows, 1), B, S, s.Hq, s.Hkv, s.hd, out0.shape[-1] if inp.w_o is not None else 0))
    dlm.dlm_partial_attn(q, idx_o, off_o, max_rows, kc, vc, scale, o, lse, w_o=wo, out_cache=out, workspace=wsa)
    torch.cuda.synchronize()

    tol = TOL[dt]
    sel = rows_mask(B, S, ref["idx"], ref["offsets"])
    errs = {
        "q": maxabs(host(q)[:n], ref["q"]),
        "k": maxabs(host(kc)[sel], ref["k_cache"][sel]),
        "v": maxabs(host(vc)[sel], ref["v_cache"][sel]),
        "o": maxabs(host(o)[:n], ref["o"]),
        "lse": maxabs(host(lse)[:n], ref["lse"]),
        "out": maxabs(host(out)[sel], ref["out_cache"][sel]),
    }
    say(f"  n={n} max-abs errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= tol, f"{k_}: {v_} > {tol}"
    # untouched rows byte-identical
    k_ref, v_ref, out_ref = dev(kc0, dt), dev(vc0, dt), dev(out0, dt)
    keep = torch.from_numpy(~sel).cuda()
    assert torch.equal(kc[keep], k_ref[keep]) and torch.equal(vc[keep], v_ref[keep])
    assert torch.equal(out[keep], out_ref[keep])
    return ref, n


def test_tiny_fp32_step(dlm):
    ref, n = run_cosine_step(dlm, W.TINY_FP32)
    assert n == 16


def test_bf16_s1024_step_full_size(dlm):
    ref, n = run_cosine_step(dlm, W.BF16_S1024)
    assert n == 102


def test_bf16_s1024_step_bench_launch(dlm):
    """The one-layer step exactly as the benchmark launches it: the host passes
    the loose row bound B*S = 1024 to the Q/K/V and attention calls, so the
    Q/K/V GEMM is the single dual launch whose device count (102) picks the
    48-weight-row streaming body at K = 4096, N = 12288, and attention sizes
    its grid for 1024 rows.  Every Q/K/V/O/LSE/output element against the
    oracle; unselected cache rows byte-identical."""
    ref, n = run_cosine_step(dlm, W.BF16_S1024, bound="loose")
    assert n == 102


def test_bf16_step_response_window(dlm):
    """Scoring restricted to a window [lo, hi) with lo > 0 (DyLLM's
    response-only input): scores outside the window are not written, and only
    window positions can be selected; the step's outputs against the oracle."""
    ref, n = run_cosine_step(dlm, W.BF16_S1024, lo=75, hi=190, B=2, S=200, D=512, Hq=4, Hkv=2, hd=128,
                             n_redrawn=60)
    assert 0 < n and np.all((ref["idx"] >= 75) & (ref["idx"] < 190))


def test_bf16_step_ragged_multi_batch(dlm):
    # several batch rows, a ragged selection count and tiles that do not divide evenly
    run_cosine_step(dlm, W.BF16_S1024, B=3, S=200, D=512, Hq=4, Hkv=2, hd=128, n_redrawn=37)


def test_bf16_step_head_dim_64(dlm):
    run_cosine_step(dlm, W.BF16_S1024, B=2, S=130, D=256, Hq=4, Hkv=4, hd=64, n_redrawn=19)


def test_bf16_step_deep_split_k(dlm):
    # few output tiles and a long reduction (D = 4096 over N = 1536 features),
    # with the exact count: the weight-streaming tiling with two k-halves per
    # workgroup; with the loose bound (256 rows): the dual launch
    run_cosine_step(dlm, W.BF16_S1024, B=1, S=256, D=4096, Hq=4, Hkv=4, hd=128, n_redrawn=40)
    run_cosine_step(dlm, W.BF16_S1024, B=1, S=256, D=4096, Hq=4, Hkv=4, hd=128, n_redrawn=40, bound="loose")


def test_bf16_step_with_output_projection(dlm):
    # bf16 layer with a W_o projection before the output scatter (ragged, two batch rows)
    run_cosine_step(dlm, W.BF16_S1024, B=2, S=150, D=256, Hq=4, Hkv=4, hd=64, n_redrawn=23, with_wo=True)


def test_all_selected_equals_full_recompute(dlm):
    # tau above every cosine: all rows recomputed -> the step equals a full pass on cur
    ref, n = run_cosine_step(dlm, W.BF16_S1024, tau=2.0, B=1, S=96, D=256, Hq=2, Hkv=2, hd=128, n_redrawn=5)
    assert n == 96


def test_none_selected_returns_cache(dlm):
    ref, n = run_cosine_step(dlm, W.BF16_S1024, tau=-2.0, B=2, S=64, D=256, Hq=2, Hkv=2, hd=128, n_redrawn=5)
    assert n == 0


def test_dyllm_adaptive_input_loop(dlm):
    """DyLLM's adaptive input over 8 steps of the one-layer bf16 workload (1024
    positions: a 512-token prompt and a 512-token response; every row drifts,
    51 response rows and 4 prompt rows are redrawn per step): steps with
    t % 4 == 0 score the whole sequence, the others the response [512, 1024)
    only; each step selects by cosine < 0.95 inside its window and recomputes
    the selected rows' Q/K/V (K/V scatter) and attention over all 1024 keys
    (context scatter), with the loose row bound the benchmark passes.  Each
    step against the oracle, which carries its own caches: the scores in the
    window (none written outside), the index set, Q, K/V and output rows, O,
    LSE; every row not selected keeps the step's input cache bytes."""
    inp = W.dyllm_loop_inputs(W.DYLLM_LOOP)
    s = inp.shape
    B, S = s.B, s.S
    scale = 1.0 / math.sqrt(s.hd)
    say(f"[dyllm loop] B={B} S={S} prompt={s.prompt} D={s.D} steps={s.steps} refresh={s.refresh}")
    kc_o, vc_o, out_o = (W.round_bf16(a) for a in
                         O.full_recompute_caches(inp.hidden(-1), inp.w_qkv, s.Hq, s.Hkv, s.hd, scale))
    kc, vc, out = dev(kc_o, "bf16"), dev(vc_o, "bf16"), dev(out_o, "bf16")
    w = dev(inp.w_qkv, "bf16")
    max_rows = B * S
    q = torch.zeros(max_rows, s.Hq, s.hd, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    lse = torch.zeros(max_rows, s.Hq, dtype=torch.float32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    ws = workspace(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_COSINE, B, S))
    wsq = workspace(dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, max_rows, s.D, s.Hq, s.Hkv, s.hd))
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, max_rows, B, S, s.Hq, s.Hkv, s.hd))
    for t in range(s.steps):
        lo, hi = O.adaptive_input_window(t, s.prompt, S, s.refresh)
        cur, prev = inp.hidden(t), inp.hidden(t - 1)
        ref = O.cosine_step(cur, prev, inp.w_qkv, s.Hq, s.Hkv, s.hd, s.tau, kc_o, vc_o, out_o, lo=lo, hi=hi)
        before = [x.clone() for x in (kc, vc, out)]
        scores.fill_(-7.0)
        curd = dev(cur, "bf16")
        dlm.dlm_saliency_select(dlm.DLM_SCORE_COSINE, curd, dev(prev, "bf16"), lo=lo, hi=hi, threshold=s.tau,
                                idx=idx, counts=counts, offsets=offsets, scores=scores, workspace=ws)
        torch.cuda.synchronize()
        sc_g = host(scores)
        assert maxabs(sc_g[:, lo:hi], ref["scores"][:, lo:hi]) <= 1e-5
        assert np.all(sc_g[:, :lo] == -7.0)
        check_selection(idx.cpu().numpy(), counts.cpu().numpy(), offsets.cpu().numpy(), ref["scores"], lo, hi,
                        s.tau)
        n = int(ref["offsets"][-1])
        idx_o, off_o = i32(ref["idx"]), i32(ref["offsets"])
        dlm.dlm_gather_qkv_scatter_kv(curd, idx_o, off_o, max_rows, w, s.Hq, s.Hkv, s.hd, q, kc, vc, workspace=wsq)
        dlm.dlm_partial_attn(q, idx_o, off_o, max_rows, kc, vc, scale, o, lse, out_cache=out, workspace=wsa)
        torch.cuda.synchronize()
        sel = rows_mask(B, S, ref["idx"], ref["offsets"])
        errs = dict(q=maxabs(host(q)[:n], ref["q"]), k=maxabs(host(kc)[sel], ref["k_cache"][sel]),
                    v=maxabs(host(vc)[sel], ref["v_cache"][sel]), o=maxabs(host(o)[:n], ref["o"]),
                    lse=maxabs(host(lse)[:n], ref["lse"]), out=maxabs(host(out)[sel], ref["out_cache"][sel]))
        say(f"  step {t} window [{lo},{hi}) n={n} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k_, v_ in errs.items():
            assert v_ <= TOL["bf16"], f"step {t} {k_}: {v_}"
        keep = torch.from_numpy(~sel).cuda()
        for x, x0 in zip((kc, vc, out), before):
            assert torch.equal(x[keep], x0[keep]), f"step {t}: an unselected row changed"
        if lo > 0:
            assert ref["idx"].min() >= lo
        kc_o, vc_o, out_o = ref["k_cache"], ref["v_cache"], ref["out_cache"]


# ---------------------------------------------------------------------------
# lock loop (GQA, given scores, several steps carrying the caches)
# ---------------------------------------------------------------------------
def test_gqa_lock_loop_reduced(dlm):
    inp = W.lock_loop_inputs(W.GQA_LOCK_LOOP, B=2, S=320, D=512, Hq=8, Hkv=2, steps=5)
    s = inp.shape
    B, S = s.B, s.S
    scale = 1.0 / math.sqrt(s.hd)
    say(f"[lock loop] B={B} S={S} D={s.D} Hq={s.Hq} Hkv={s.Hkv} steps={s.steps}")
    kc_o = np.zeros((B, S, s.Hkv, s.hd))
    vc_o = np.zeros_like(kc_o)
    out_o = np.zeros((B, S, s.Hq * s.hd))
    kc = torch.zeros(B, S, s.Hkv, s.hd, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    out = torch.zeros(B, S, s.Hq * s.hd, dtype=torch.bfloat16, device="cuda")
    w = dev(inp.w_qkv, "bf16")
    max_rows = B * S
    q = torch.zeros(max_rows, s.Hq, s.hd, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    lse = torch.zeros(max_rows, s.Hq, dtype=torch.float32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, max_rows, B, S, s.Hq, s.Hkv, s.hd))
    wsq = workspace(dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, max_rows, s.D, s.Hq, s.Hkv, s.hd))
    for t in range(s.steps):
        sc = inp.unlocked_scores(t)
        x = inp.hidden(t)
        ridx, rcounts, roff = O.compact(sc, 0, S, 0.5)
        q_o, kc_o, vc_o = O.qkv_project_scatter(x, ridx, roff, inp.w_qkv, s.Hq, s.Hkv, s.hd, kc_o, vc_o)
        o_o, lse_o = O.partial_attention(q_o, ridx, roff, kc_o, vc_o, s.Hq, s.Hkv, scale)
        out_o = O.output_scatter(o_o, ridx, roff, out_o)

        dlm.dlm_saliency_select(dlm.DLM_SCORE_GIVEN, dev(sc, "f32"), None, lo=0, hi=S, threshold=0.5,
                                idx=idx, counts=counts, offsets=offsets)
        xd = dev(x, "bf16")
        dlm.dlm_gather_qkv_scatter_kv(xd, idx, offsets, max_rows, w, s.Hq, s.Hkv, s.hd, q, kc, vc,
                                      workspace=wsq)
        dlm.dlm_partial_attn(q, idx, offsets, max_rows, kc, vc, scale, o, lse, out_cache=out, workspace=wsa)
        torch.cuda.synchronize()
        n = int(roff[-1])
        assert np.array_equal(offsets.cpu().numpy(), roff) and np.array_equal(idx.cpu().numpy()[:n], ridx)
        errs = dict(q=maxabs(host(q)[:n], q_o), k=maxabs(host(kc), kc_o), v=maxabs(host(vc), vc_o),
                    o=maxabs(host(o)[:n], o_o), lse=maxabs(host(lse)[:n], lse_o), out=maxabs(host(out), out_o))
        say(f"  step {t}: n={n} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k_, v_ in errs.items():
            assert v_ <= TOL["bf16"], f"step {t} {k_}: {v_}"


@pytest.mark.parametrize("t,bound", [(0, "exact"), (32, "exact"), (40, "exact"), (62, "exact"), (63, "exact"),
                                     (63, "loose")])
def test_gqa_lock_loop_step_full_size(dlm, t, bound):
    """One step of the 64-step GQA lock loop at its full size (B = 8, S = 2048,
    D = 4096, 32 query / 8 KV heads of 128), with the row bound the benchmark's
    loop passes (the exact count) and, for the last step, the loose bound B*S.
    The launches differ by step: t = 0 (16384 rows, 1536 tiles of 256 x 256:
    six whole rounds of the 256-workgroup grid) runs the GEMM unsplit, its
    Q/K/V epilogue inside the GEMM kernel, and 128-vector attention
    workgroups (GQA 4:1); t = 32 (8480 rows, 816 tiles) splits the 48 tiles
    of its last round 4 ways (their epilogue in the reduce pass) and t = 40
    (6504 rows, 624 tiles) leaves the 112 of its last round unsplit; t = 62
    (1072 rows, 120 tiles) splits K 2 ways over spare workgroups; t = 63 (824 rows) runs
    the 128 x 128 body of the dual launch (the loose bound the 256 x 256
    tiling), and its 256 attention units, one per CU, leave the keys unsplit.
    The caches hold seeded earlier rows.  Every
    Q row, every cache row (selected against the oracle, others
    byte-identical) and O/LSE of 48 sampled rows against the oracle."""
    inp = W.lock_loop_inputs(W.GQA_LOCK_LOOP)
    s = inp.shape
    B, S = s.B, s.S
    scale = 1.0 / math.sqrt(s.hd)
    rng = np.random.default_rng(77)
    kc0 = W.round_bf16(rng.standard_normal((B, S, s.Hkv, s.hd), dtype=np.float32))
    vc0 = W.round_bf16(rng.standard_normal((B, S, s.Hkv, s.hd), dtype=np.float32))
    sc, x = inp.unlocked_scores(t), inp.hidden(t)
    ridx, _, roff = O.compact(sc, 0, S, 0.5)
    n = int(roff[-1])
    max_rows = n if bound == "exact" else B * S
    say(f"[lock loop full size] B={B} S={S} D={s.D} Hq={s.Hq} Hkv={s.Hkv} t={t} n={n} max_rows={max_rows}")
    q_o, kc_o, vc_o = O.qkv_project_scatter(x, ridx, roff, inp.w_qkv, s.Hq, s.Hkv, s.hd, kc0, vc0)
    pick = np.unique(np.linspace(0, n - 1, 48).astype(np.int64))
    counts = np.array([np.sum((pick >= roff[b]) & (pick < roff[b + 1])) for b in range(B)])
    poff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    o_o, lse_o = O.partial_attention(q_o[pick], ridx[pick], poff, kc_o, vc_o, s.Hq, s.Hkv, scale)

    kc, vc = dev(kc0, "bf16"), dev(vc0, "bf16")
    kc_before, vc_before = kc.clone(), vc.clone()
    q = torch.zeros(max_rows, s.Hq, s.hd, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    lse = torch.zeros(max_rows, s.Hq, dtype=torch.float32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, max_rows, B, S, s.Hq, s.Hkv, s.hd))
    wsq = workspace(dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, max_rows, s.D, s.Hq, s.Hkv, s.hd))
    dlm.dlm_saliency_select(dlm.DLM_SCORE_GIVEN, dev(sc, "f32"), None, lo=0, hi=S, threshold=0.5,
                            idx=idx, counts=cnt, offsets=offsets)
    dlm.dlm_gather_qkv_scatter_kv(dev(x, "bf16"), idx, offsets, max_rows, dev(inp.w_qkv, "bf16"), s.Hq,
                                  s.Hkv, s.hd, q, kc, vc, workspace=wsq)
    dlm.dlm_partial_attn(q, idx, offsets, max_rows, kc, vc, scale, o, lse, workspace=wsa)
    torch.cuda.synchronize()
    assert np.array_equal(offsets.cpu().numpy(), roff) and np.array_equal(idx.cpu().numpy()[:n], ridx)
    sel = torch.from_numpy(rows_mask(B, S, ridx, roff)).cuda()
    assert torch.equal(kc[~sel], kc_before[~sel]) and torch.equal(vc[~sel], vc_before[~sel])
    errs = dict(q=maxabs(host(q[:n]), q_o), k=maxabs(host(kc), kc_o), v=maxabs(host(vc), vc_o),
                o=maxabs(host(o)[pick], o_o), lse=maxabs(host(lse)[pick], lse_o))
    say(f"  n={n} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL["bf16"], f"{k_}: {v_}"


def test_loose_row_bound_picks_every_tiling(dlm):
    """The host passes max_rows = B*S > 1024 while the device count is 50, 600
    or 2000: the one GEMM launch must take the weight-streaming tiling, then
    the 256 x 256 tiling with K split over spare workgroups, and the attention
    its matching plans; every result against the oracle."""
    B, S, D, Hq, Hkv, hd = 2, 1100, 1024, 4, 2, 64
    N = (Hq + 2 * Hkv) * hd
    scale = 1.0 / math.sqrt(hd)
    rng = np.random.default_rng(11)
    x = W.round_bf16(rng.standard_normal((B, S, D)))
    w = W.round_bf16(rng.standard_normal((N, D)) / 32.0)
    kc0 = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    vc0 = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    out0 = W.round_bf16(rng.standard_normal((B, S, Hq * hd)))
    max_rows = B * S
    q = torch.zeros(max_rows, Hq, hd, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    lse = torch.zeros(max_rows, Hq, dtype=torch.float32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    wsq = workspace(dlm.dlm_gather_qkv_workspace_size(dlm.DLM_BF16, max_rows, D, Hq, Hkv, hd))
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, max_rows, B, S, Hq, Hkv, hd))
    xd, wd = dev(x, "bf16"), dev(w, "bf16")
    for per_b in (25, 300, 1000):
        sc = np.ones((B, S))
        for b in range(B):
            sc[b, rng.choice(S, per_b, replace=False)] = 0.0
        ridx, _, roff = O.compact(sc, 0, S, 0.5)
        q_o, kc_o, vc_o = O.qkv_project_scatter(x, ridx, roff, w, Hq, Hkv, hd, kc0, vc0)
        o_o, lse_o = O.partial_attention(q_o, ridx, roff, kc_o, vc_o, Hq, Hkv, scale)
        out_o = O.output_scatter(o_o, ridx, roff, out0)
        say(f"[loose bound] max_rows={max_rows} n={int(roff[-1])} D={D} N={N}")
        kc, vc, out = dev(kc0, "bf16"), dev(vc0, "bf16"), dev(out0, "bf16")
        dlm.dlm_saliency_select(dlm.DLM_SCORE_GIVEN, dev(sc, "f32"), None, lo=0, hi=S, threshold=0.5,
                                idx=idx, counts=counts, offsets=offsets)
        dlm.dlm_gather_qkv_scatter_kv(xd, idx, offsets, max_rows, wd, Hq, Hkv, hd, q, kc, vc,
                                      workspace=wsq)
        dlm.dlm_partial_attn(q, idx, offsets, max_rows, kc, vc, scale, o, lse, out_cache=out, workspace=wsa)
        torch.cuda.synchronize()
        n = int(roff[-1])
        assert np.array_equal(idx.cpu().numpy()[:n], ridx)
        errs = dict(q=maxabs(host(q)[:n], q_o), k=maxabs(host(kc), kc_o), v=maxabs(host(vc), vc_o),
                    o=maxabs(host(o)[:n], o_o), lse=maxabs(host(lse)[:n], lse_o), out=maxabs(host(out), out_o))
        say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        for k_, v_ in errs.items():
            assert v_ <= TOL["bf16"], f"n={n} {k_}: {v_}"


def run_attention_plan(dlm, B, S, Hq, Hkv, hd, rows_per_b, sample=None, seed=21, late_keys=None):
    """Partial attention on given q/k/v (bf16) against the oracle; with
    `sample`, only that many selected rows (spread over the batch rows) are
    recomputed by the oracle, over all S keys.  `late_keys` (positions): those
    keys are set to 200 times a unit direction u and every query gets +3 u,
    so their scaled scores exceed the early keys' by ~75 in log2 units."""
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(hd)
    kc = rng.standard_normal((B, S, Hkv, hd))
    u = np.ones(hd) / math.sqrt(hd)
    if late_keys is not None:
        kc[:, late_keys] = 200.0 * u
    kc = W.round_bf16(kc)
    vc = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    sc = np.ones((B, S))
    for b in range(B):
        sc[b, rng.choice(S, rows_per_b[b], replace=False)] = 0.0
    ridx, _, roff = O.compact(sc, 0, S, 0.5)
    n = int(roff[-1])
    q = rng.standard_normal((n, Hq, hd))
    if late_keys is not None:
        q = q + 3.0 * u
    q = W.round_bf16(q)
    say(f"[attention plan] B={B} S={S} Hq={Hq} Hkv={Hkv} hd={hd} n={n} sample={sample}")
    o = torch.zeros(n, Hq, hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(n, Hq, dtype=torch.float32, device="cuda")
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, n, B, S, Hq, Hkv, hd))
    dlm.dlm_partial_attn(dev(q, "bf16"), i32(ridx), i32(roff), n, dev(kc, "bf16"), dev(vc, "bf16"), scale,
                         o, lse, workspace=wsa)
    torch.cuda.synchronize()
    if sample is None:
        pick = np.arange(n)
    else:
        pick = np.unique(np.linspace(0, n - 1, sample).astype(np.int64))
    # the oracle on the picked rows only: each keeps its own batch row
    counts = np.array([np.sum((pick >= roff[b]) & (pick < roff[b + 1])) for b in range(B)])
    poff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    o_o, lse_o = O.partial_attention(q[pick], ridx[pick], poff, kc, vc, Hq, Hkv, scale)
    eo, el = maxabs(host(o)[pick], o_o), maxabs(host(lse)[pick], lse_o)
    say(f"  rows checked {len(pick)}: o={eo:.2e} lse={el:.2e}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 16)])
def test_attention_many_tiles_gqa_ragged(dlm, hd, Hq, Hkv):
    """>= 512 tiles of 128 query vectors: no key split; GQA 4:1 runs 128-vector
    workgroups (two per CU), GQA 2:1 the 256-vector ones; ragged last query
    tile and last 64-key tile; sampled rows against the oracle."""
    run_attention_plan(dlm, B=2, S=1500, Hq=Hq, Hkv=Hkv, hd=hd, rows_per_b=[1500, 1436], sample=48)


@pytest.mark.parametrize("hd", [64, 128])
def test_attention_few_tiles_split_keys(dlm, hd):
    """Four query tiles over S = 4200 keys: the keys split over 14 workgroups
    (more than 8, the merge's second register layout) and the LSE merge pass;
    every row against the oracle."""
    run_attention_plan(dlm, B=2, S=4200, Hq=4, Hkv=2, hd=hd, rows_per_b=[37, 5])


def test_attention_two_key_splits(dlm):
    """128 query tiles (B = 8, 33-64 rows each, GQA 4:1) on 256 CUs: the keys
    split exactly 2 ways (the merge's two-slot layout); sampled rows against
    the oracle."""
    run_attention_plan(dlm, B=8, S=2048, Hq=32, Hkv=8, hd=128, rows_per_b=[64, 40, 33, 50, 64, 61, 37, 48],
                       sample=64)


@pytest.mark.parametrize("rows_per_b", [[40, 17], [2048, 1900]])
@pytest.mark.parametrize("Hq,Hkv", [(8, 4), (32, 8)])
def test_attention_rescale_on_late_large_scores(dlm, rows_per_b, Hq, Hkv):
    """Keys far above every earlier score appear after the first tiles (and in
    a later split): the running reference must move mid-sequence (a lane's
    tile sum of probabilities against the old reference would pass 2^64).
    The 57-row selections split their keys; GQA 2:1 at 3,948 rows stays on
    the 64-key tiles unsplit (a short row bound: 252 tiles), GQA 4:1 at 3,948
    rows takes the 32-key tiles (1,000 tiles); outputs and LSE against the
    oracle."""
    run_attention_plan(dlm, B=2, S=2048, Hq=Hq, Hkv=Hkv, hd=128, rows_per_b=rows_per_b, sample=64,
                       late_keys=[700, 701, 1500, 2040])


def test_attention_short_sequence(dlm):
    """S = 70: one ragged 64-key tile and a 6-key tail tile, never split."""
    run_attention_plan(dlm, B=3, S=70, Hq=4, Hkv=4, hd=128, rows_per_b=[70, 1, 33])


# ---------------------------------------------------------------------------
# attention column sums + top-k
# ---------------------------------------------------------------------------
def run_colsum(dlm, zero_q=False, **override):
    inp = W.colsum_inputs(W.COLSUM_TOP64, zero_q=zero_q, **override)
    s = inp.shape
    B, S, nq = s.B, s.S, s.S - s.prompt
    scale = 1.0 / math.sqrt(s.hd)
    say(f"[colsum] B={B} S={S} prompt={s.prompt} Hq={s.Hq} Hkv={s.Hkv} k={s.k} zero_q={zero_q}")
    sc = inp.masked_scores()
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    dlm.dlm_saliency_select(dlm.DLM_SCORE_GIVEN, dev(sc), None, lo=0, hi=S, threshold=0.5, idx=idx,
                            counts=counts, offsets=offsets)
    ridx, _, roff = O.compact(sc, 0, S, 0.5)
    q_np = inp.q.reshape(B * nq, s.Hq, s.hd)
    o_o, lse_o = O.partial_attention(q_np, ridx, roff, inp.k_cache, inp.v_cache, s.Hq, s.Hkv, scale)
    c_o = O.column_sums(q_np, roff, inp.k_cache, lse_o, s.Hq, s.Hkv, scale)
    q = dev(q_np, "bf16")
    kc, vc = dev(inp.k_cache, "bf16"), dev(inp.v_cache, "bf16")
    n = B * nq
    o = torch.zeros_like(q)
    lse = torch.zeros(n, s.Hq, dtype=torch.float32, device="cuda")
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, n, B, S, s.Hq, s.Hkv, s.hd))
    dlm.dlm_partial_attn(q, idx, offsets, n, kc, vc, scale, o, lse, workspace=wsa)
    colsum = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    ti = torch.zeros(B, s.k, dtype=torch.int32, device="cuda")
    tv = torch.zeros(B, s.k, dtype=torch.float32, device="cuda")
    wsc = workspace(dlm.dlm_attn_colsum_workspace_size(B, S, s.Hkv))
    dlm.dlm_attn_colsum(q, offsets, n, kc, lse, scale, colsum, key_lo=s.prompt, key_hi=S, k=s.k,
                        topk_idx=ti, topk_val=tv, workspace=wsc)
    torch.cuda.synchronize()
    assert np.array_equal(offsets.cpu().numpy(), roff)
    c_g = host(colsum)
    errs = dict(o=maxabs(host(o), o_o), lse=maxabs(host(lse), lse_o), colsum=maxabs(c_g, c_o))
    say("  " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k_, v_ in errs.items():
        assert v_ <= TOL["bf16"], f"{k_}: {v_}"
    # column sums total the number of selected queries times the heads
    assert np.allclose(c_g.sum(axis=1), s.Hq * nq, rtol=1e-5)
    ti_g = ti.cpu().numpy()
    check_topk(ti_g, c_o, s.prompt, S, s.k)
    tv_g = tv.cpu().numpy()
    assert np.all(np.diff(tv_g, axis=1) <= 0)
    for b in range(B):
        assert np.array_equal(tv_g[b], c_g[b, ti_g[b]].astype(np.float32))
        # the selection itself is exact on the kernel's own sums: the first k
        # window positions ordered by (-colsum, position)
        win = np.arange(s.prompt, S)
        order = win[np.lexsort((win, -c_g[b, win].astype(np.float64)))]
        assert np.array_equal(ti_g[b], order[: s.k]), f"sequence {b}: top-{s.k} differs from its own sums"
    # determinism: a second run is bit-identical
    c2 = torch.zeros_like(colsum)
    ti2 = torch.zeros_like(ti)
    dlm.dlm_attn_colsum(q, offsets, n, kc, lse, scale, c2, key_lo=s.prompt, key_hi=S, k=s.k,
                        topk_idx=ti2, workspace=wsc)
    torch.cuda.synchronize()
    assert torch.equal(c2, colsum) and torch.equal(ti2, ti)
    return ti_g, c_g


def test_colsum_workload_full_size(dlm):
    """The attention + column-sum workload at its full size, in the launch
    configuration the benchmark times (B = 4, S = 4096, 32 heads of 128, the
    3072 masked positions of every sequence as queries): O and LSE of 32 rows
    sampled over all sequences, and every column sum of every sequence (with
    the oracle's own LSE of all its queries), against the oracle; each
    sequence's top-64 by the band rule and exactly on the kernel's own sums;
    for every sequence the total sum_j c = Hq * n_q."""
    inp = W.colsum_inputs(W.COLSUM_TOP64)
    s = inp.shape
    B, S, nq = s.B, s.S, s.S - s.prompt
    scale = 1.0 / math.sqrt(s.hd)
    say(f"[colsum full size] B={B} S={S} prompt={s.prompt} Hq={s.Hq} Hkv={s.Hkv} k={s.k}")
    sc = inp.masked_scores()
    ridx, _, roff = O.compact(sc, 0, S, 0.5)
    n = int(roff[-1])
    q_np = inp.q.reshape(n, s.Hq, s.hd)
    q, kc, vc = dev(q_np, "bf16"), dev(inp.k_cache, "bf16"), dev(inp.v_cache, "bf16")
    offsets = i32(roff)
    o = torch.zeros_like(q)
    lse = torch.zeros(n, s.Hq, dtype=torch.float32, device="cuda")
    wsa = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, n, B, S, s.Hq, s.Hkv, s.hd))
    dlm.dlm_partial_attn(q, i32(ridx), offsets, n, kc, vc, scale, o, lse, workspace=wsa)
    colsum = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    ti = torch.zeros(B, s.k, dtype=torch.int32, device="cuda")
    tv = torch.zeros(B, s.k, dtype=torch.float32, device="cuda")
    wsc = workspace(dlm.dlm_attn_colsum_workspace_size(B, S, s.Hkv))
    dlm.dlm_attn_colsum(q, offsets, n, kc, lse, scale, colsum, key_lo=s.prompt, key_hi=S, k=s.k,
                        topk_idx=ti, topk_val=tv, workspace=wsc)
    torch.cuda.synchronize()
    # sampled rows over all sequences
    pick = np.unique(np.linspace(0, n - 1, 32).astype(np.int64))
    counts = np.array([np.sum((pick >= roff[b]) & (pick < roff[b + 1])) for b in range(B)])
    poff = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    o_o, lse_o = O.partial_attention(q_np[pick], ridx[pick], poff, inp.k_cache, inp.v_cache, s.Hq, s.Hkv, scale)
    eo, el = maxabs(host(o)[pick], o_o), maxabs(host(lse)[pick], lse_o)
    say(f"  rows {len(pick)}: o={eo:.2e} lse={el:.2e}")
    assert eo <= TOL["bf16"] and el <= TOL["bf16"]
    c_g = host(colsum)
    ti_g, tv_g = ti.cpu().numpy(), tv.cpu().numpy()
    off1 = np.array([0, nq], dtype=np.int64)
    for b in range(B):
        # every column of sequence b, with the oracle's own LSE of all its queries
        qb = q_np[b * nq:(b + 1) * nq]
        kb, vb = inp.k_cache[b:b + 1], inp.v_cache[b:b + 1]
        _, lse_b = O.partial_attention(qb, ridx[b * nq:(b + 1) * nq], off1, kb, vb, s.Hq, s.Hkv, scale)
        c_b = O.column_sums(qb, off1, kb, lse_b, s.Hq, s.Hkv, scale)
        ec = maxabs(c_g[b:b + 1], c_b)
        say(f"  sequence {b}: column sums {ec:.2e}")
        assert ec <= TOL["bf16"]
        check_topk(ti_g[b:b + 1], c_b, s.prompt, S, s.k)
        win = np.arange(s.prompt, S)
        order = win[np.lexsort((win, -c_g[b, win]))]
        assert np.array_equal(ti_g[b], order[: s.k]), f"sequence {b}: top-{s.k} differs from its own sums"
        assert np.array_equal(tv_g[b], c_g[b, ti_g[b]].astype(np.float32))
    assert np.allclose(c_g.sum(axis=1), s.Hq * nq, rtol=1e-4)


def test_colsum_window_bench_launch(dlm):
    """The block-wise column sums as the benchmark's key-window call runs them:
    so many partials that the separate reduce pass runs (here 16 KV heads over
    a 1280-key covering range), then the radix select (k = 64 over a window of
    1040 keys).  The window [1000, 2040) starts inside a 256-key block, so the
    reduce pass starts at an offset.  Inside the window the sums match the
    full call's and the oracle's; outside the covering blocks [768, 2048)
    nothing is written; the top-k is exact on the window call's own sums and
    within the band rule of the oracle's."""
    rng = np.random.default_rng(62)
    B, S, Hq, Hkv, hd = 2, 2048, 16, 16, 128
    scale = 1.0 / math.sqrt(hd)
    kc = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    vc = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    n_b = [300, 211]
    rows = [np.sort(rng.choice(S, m, replace=False)) for m in n_b]
    idx = np.concatenate(rows).astype(np.int32)
    offsets = np.array([0, n_b[0], sum(n_b)], np.int32)
    n = sum(n_b)
    q = W.round_bf16(rng.standard_normal((n, Hq, hd)))
    _, lse = O.partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, scale)
    c_o = O.column_sums(q, offsets, kc, lse, Hq, Hkv, scale)
    lo, hi, kk = 1000, 2040, 64
    say(f"[colsum window, reduce pass] B={B} S={S} Hkv={Hkv} window [{lo},{hi}) k={kk}")
    qd, kd, ld, od = dev(q, "bf16"), dev(kc, "bf16"), dev(lse, "f32"), i32(offsets)
    ws = workspace(dlm.dlm_attn_colsum_workspace_size(B, S, Hkv))
    full = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    dlm.dlm_attn_colsum(qd, od, n, kd, ld, scale, full, workspace=ws)
    win = torch.full((B, S), -1.0, dtype=torch.float32, device="cuda")
    ti = torch.zeros(B, kk, dtype=torch.int32, device="cuda")
    tv = torch.zeros(B, kk, dtype=torch.float32, device="cuda")
    dlm.dlm_attn_colsum(qd, od, n, kd, ld, scale, win, key_lo=lo, key_hi=hi, k=kk, topk_idx=ti, topk_val=tv,
                        workspace=ws, window_only=True)
    torch.cuda.synchronize()
    f, w = full.cpu().numpy(), win.cpu().numpy()
    assert np.allclose(w[:, lo:hi], f[:, lo:hi], rtol=1e-5, atol=1e-6)
    ec = maxabs(w[:, 768:], c_o[:, 768:])
    say(f"  window sums against the oracle {ec:.2e}")
    assert ec <= TOL["bf16"]
    assert np.all(w[:, :768] == -1.0), "written outside the covering blocks"
    check_topk(ti.cpu().numpy(), c_o, lo, hi, kk)
    for b in range(B):
        order = np.lexsort((np.arange(lo, hi), -w[b, lo:hi].astype(np.float64)))[:kk] + lo
        assert np.array_equal(ti[b].cpu().numpy(), order)
        assert np.array_equal(tv[b].cpu().numpy(), w[b, order])


def test_colsum_group_not_power_of_two(dlm):
    """Three query heads per KV head (the column-sum pass's generic query
    addressing) at head dim 64 and 128."""
    run_colsum(dlm, B=2, S=600, prompt=100, Hq=6, Hkv=2, hd=64, k=16)
    run_colsum(dlm, B=2, S=600, prompt=100, Hq=6, Hkv=2, hd=128, k=16)


def test_colsum_topk_reduced(dlm):
    run_colsum(dlm, B=2, S=1024, prompt=256, Hq=4, Hkv=4, k=16)


def test_colsum_topk_gqa_ragged(dlm):
    run_colsum(dlm, B=3, S=520, prompt=77, Hq=8, Hkv=2, k=24)


@pytest.mark.parametrize("B,S", [(5, 1000), (12, 3000), (70, 8192)])
def test_given_select_batch_paths(dlm, B, S):
    """Compaction of supplied scores over the window [3, S-5): B = 5 and
    B = 12 take the one-workgroup-per-row kernel (B = 12: earlier rows counted
    in two batches of eight, a 2,992-position window in two chunks), B = 70
    (B*B*window over the limit for recounting) the single-workgroup loop.  Index sets, counts and offsets
    are bit-exact against the oracle (the scores are exact float32 values and
    0.5 is exact, so both sides take the same decisions)."""
    lo, hi = 3, S - 5
    say(f"[given select] B={B} S={S} window=[{lo},{hi})")
    rng = np.random.default_rng(7000 + B)
    sc = rng.random((B, S), dtype=np.float32)
    sc[0, lo:hi] = 1.0  # an empty row
    ridx, rcnt, roff = O.compact(sc, lo, hi, 0.5)
    idx = torch.full((B * S,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    dlm.dlm_saliency_select(dlm.DLM_SCORE_GIVEN, dev(sc, "f32"), None, lo=lo, hi=hi, threshold=0.5,
                            idx=idx, counts=cnt, offsets=offsets)
    torch.cuda.synchronize()
    n = int(roff[-1])
    assert np.array_equal(offsets.cpu().numpy(), roff) and np.array_equal(cnt.cpu().numpy(), rcnt)
    got = idx.cpu().numpy()
    assert np.array_equal(got[:n], ridx)
    assert np.all(got[n:] == -7), "compaction wrote past the selected entries"


@pytest.mark.parametrize("k,S,prompt", [(1, 1536, 256), (64, 1536, 256), (100, 1536, 256), (16, 1024, 256)])
def test_colsum_topk_sizes(dlm, k, S, prompt):
    """k = 1 and k = 64 over a 1280-key window take the radix-select path,
    k = 100 and the 768-key window the sort of the whole window; all against
    the oracle's band rule and, exactly, against the order of the kernel's
    own sums."""
    run_colsum(dlm, B=2, S=S, prompt=prompt, Hq=4, Hkv=4, k=k)


@pytest.mark.parametrize("S,prompt,k", [(512, 128, 20), (2048, 512, 64)])
def test_colsum_uniform_ties_pick_lowest_positions(dlm, S, prompt, k):
    """Q = 0: every column sum is equal, so the top-k is the k lowest window
    positions; the 1536-key window resolves the ties in the radix select's
    position digits."""
    ti, c = run_colsum(dlm, zero_q=True, B=2, S=S, prompt=prompt, Hq=4, Hkv=4, k=k)
    assert ti.tolist() == [list(range(prompt, prompt + k))] * 2


# ---------------------------------------------------------------------------
# confidence + longest stable prefix
# ---------------------------------------------------------------------------
def lsp_shape(**kw):
    D = kw.get("D", 256)
    base = dict(B=3, S=160, prompt=32, D=D, V=2048, w_std=0.02 * math.sqrt(4096 / D), steps=8)
    base.update(kw)
    return W.LspShape(**{**W.LSP_COMMIT.__dict__, **base})


def stability_state(ring, amb_ring, mp, conf, band=BAND):
    """1 stable / 0 not / 2 ambiguous, per generated position of one batch row."""
    eq = np.all(ring == ring[:, :1], axis=1) & (ring[:, 0] != -1)
    amb_arg = np.any(amb_ring, axis=1)
    st = np.where(eq & (mp >= conf), 1, 0)
    amb = amb_arg | (np.abs(mp - conf) <= band)
    return np.where(amb, 2, st)


def test_confidence_and_stable_prefix_loop(dlm):
    sh = lsp_shape()
    inp = W.lsp_inputs(sh)
    B, S, S_gen = sh.B, sh.S, inp.S_gen
    say(f"[lsp] B={B} S={S} D={sh.D} V={sh.V} steps={sh.steps}")
    w = dev(inp.w_lm, "bf16")
    scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    argmax = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    ring = torch.full((B, S_gen, sh.W), -1, dtype=torch.int32, device="cuda")
    committed = torch.zeros(B, dtype=torch.int32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    n_act = inp.n_active()
    ws = workspace(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_CONFIDENCE, B, S, sh.V, B * n_act))
    ring_o = np.full((B, S_gen, sh.W), -1, np.int64)
    amb_o = np.zeros((B, S_gen, sh.W), bool)
    arg_o = np.full((B, S), -1, np.int64)
    mp_o = np.zeros((B, S))
    amb_now = np.zeros((B, S), bool)
    for t in range(sh.steps):
        rows = inp.active_rows(t)
        h = inp.hidden(t)
        ev_idx, ev_off = W.pack_rows(rows)
        dlm.dlm_saliency_select(dlm.DLM_SCORE_CONFIDENCE, dev(h, "bf16"), w, lo=sh.prompt, hi=S,
                                threshold=sh.conf, idx=idx, counts=counts, offsets=offsets,
                                scores=scores, argmax=argmax, eval_idx=i32(ev_idx),
                                eval_offsets=i32(ev_off), max_eval=len(ev_idx), workspace=ws)
        torch.cuda.synchronize()
        sc_g, am_g = scores.cpu().numpy(), argmax.cpu().numpy()
        worst = 0.0
        for b in range(B):
            mp, a, gap = O.confidence(h[b, rows[b]], inp.w_lm)
            arg_o[b, rows[b]] = a
            mp_o[b, rows[b]] = mp
            amb_now[b, rows[b]] = gap <= BAND
            clear = gap > BAND
            assert np.array_equal(am_g[b, rows[b]][clear], a[clear]), f"step {t} b {b}: argmax"
            worst = max(worst, maxabs(sc_g[b, rows[b]], mp))
        assert worst <= TOL["bf16"]
        check_selection(idx.cpu().numpy(), counts.cpu().numpy(), offsets.cpu().numpy(), mp_o,
                        sh.prompt, S, sh.conf) if t == 0 else None
        prev_L = committed.cpu().numpy().copy()
        dlm.dlm_stable_prefix(argmax, scores, sh.prompt, S, ring, t, sh.conf, committed)
        torch.cuda.synchronize()
        ring_o[:, :, t % sh.W] = arg_o[:, sh.prompt:]
        amb_o[:, :, t % sh.W] = amb_now[:, sh.prompt:]
        L_g = committed.cpu().numpy()
        for b in range(B):
            st = stability_state(ring_o[b], amb_o[b], mp_o[b, sh.prompt:], sh.conf)
            adm = O.admissible_frontiers({int(prev_L[b])}, st, S_gen, 0)
            assert int(L_g[b]) in adm, f"step {t} b {b}: frontier {L_g[b]} not in {sorted(adm)}"
        say(f"  step {t}: frontiers {L_g.tolist()} max-prob err {worst:.2e}")
    assert committed.cpu().numpy().max() > 0


def test_confidence_full_size_first_step(dlm):
    """The first step of the confidence + stable-prefix workload at full size
    (B = 16, S = 1024, D = 4096, V = 32768, 230 evaluated rows per sequence),
    in the launch configuration the benchmark times: max-prob and argmax of 16
    evaluated rows per sequence (256 in all) against the oracle (argmax where the top-2 logit gap
    is outside the band); the selected set is exactly the generated positions
    whose returned max-prob is below the threshold."""
    sh = W.LSP_COMMIT
    inp = W.lsp_inputs(sh)
    B, S = sh.B, sh.S
    say(f"[confidence full size] B={B} S={S} D={sh.D} V={sh.V}")
    rows = inp.active_rows(0)
    h = inp.hidden(0)
    ev_idx, ev_off = W.pack_rows(rows)
    scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    argmax = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    ws = workspace(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_CONFIDENCE, B, S, sh.V, len(ev_idx)))
    dlm.dlm_saliency_select(dlm.DLM_SCORE_CONFIDENCE, dev(h, "bf16"), dev(inp.w_lm, "bf16"), lo=sh.prompt,
                            hi=S, threshold=sh.conf, idx=idx, counts=counts, offsets=offsets, scores=scores,
                            argmax=argmax, eval_idx=i32(ev_idx), eval_offsets=i32(ev_off),
                            max_eval=len(ev_idx), workspace=ws)
    torch.cuda.synchronize()
    sc_g, am_g = scores.cpu().numpy(), argmax.cpu().numpy()
    worst, checked = 0.0, 0
    for b in range(B):
        pick = np.asarray(rows[b])[np.linspace(0, len(rows[b]) - 1, 16).astype(np.int64)]
        mp, a, gap = O.confidence(h[b, pick], inp.w_lm)
        clear = gap > BAND
        assert np.array_equal(am_g[b, pick][clear], a[clear]), f"b {b}: argmax"
        worst = max(worst, maxabs(sc_g[b, pick], mp))
        checked += len(pick)
    say(f"  {checked} sampled rows: max-prob err {worst:.2e}")
    assert worst <= TOL["bf16"]
    # compaction of the returned scores over the generated region
    offs, ix = offsets.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        want = sh.prompt + np.nonzero(sc_g[b, sh.prompt:] < sh.conf)[0]
        assert np.array_equal(ix[offs[b]:offs[b + 1]], want), f"b {b}: selected set"


@pytest.mark.parametrize("Wd,S,gen_lo", [(3, 700, 60), (1, 700, 60), (2, 700, 60), (4, 1500, 100), (6, 700, 60)])
def test_stable_prefix_bit_exact_on_given_inputs(dlm, Wd, S, gen_lo):
    """Prefix step alone, fed identical float32 max-probs: the frontiers and the
    ring must match the oracle bit for bit (decisions in the same precision).
    Ring depths 1-4 take the kernel's unrolled paths (1,400 generated positions:
    two batches of loads per thread), depth 6 its general loop."""
    rng = np.random.default_rng(21)
    B = 5
    S_gen = S - gen_lo
    ring_o = np.full((B, S_gen, Wd), -1, np.int64)
    com_o = np.zeros(B, np.int64)
    ring = torch.full((B, S_gen, Wd), -1, dtype=torch.int32, device="cuda")
    com = torch.zeros(B, dtype=torch.int32, device="cuda")
    say(f"[prefix] B={B} S={S} gen_lo={gen_lo} W={Wd}")
    for t in range(12):
        am = rng.integers(0, 2, size=(B, S)).astype(np.int64)
        am[:, : gen_lo + 40 * t] = 1                                    # a growing stable head
        mp = rng.choice(np.array([0.5, 0.9, 0.95, 0.8999999], np.float32), size=(B, S), p=[0.05, 0.3, 0.6, 0.05])
        min_commit = t % 2
        ring_o, com_new = O.stable_prefix_step(am, mp, ring_o, t, gen_lo, S, 0.9, min_commit, com_o)
        dlm.dlm_stable_prefix(i32(am), torch.from_numpy(mp).cuda(), gen_lo, S, ring, t, 0.9, com,
                              min_commit=min_commit)
        torch.cuda.synchronize()
        assert np.array_equal(com.cpu().numpy(), com_new), f"step {t}"
        assert np.array_equal(ring.cpu().numpy(), ring_o)
        com_o = com_new
    assert com_o.max() > 0


# ---------------------------------------------------------------------------
# measurement aid: the MFMA ceiling probe
# ---------------------------------------------------------------------------
def test_mfma_probe_matches_closed_form(dlm):
    """The MFMA ceiling probe does the work it is timed for: each thread's
    sink value equals 8 chains x iters x the sum of its 16 result registers of
    A.B, built on the host from the probe's operand values and the 32x32x16
    fragment layout (A: row lane%32, k = 8*(lane/32)+e; B: column lane%32, same
    k; C register r: row 8(r/4) + 4*(lane/32) + r%4, column lane%32)."""
    iters, grid = 3, 2
    say(f"[mfma probe] iters={iters} grid={grid}")
    sink = torch.zeros(grid * 256, dtype=torch.float32, device="cuda")
    dlm.dlm_probe_mfma_bf16(iters, grid, sink)
    torch.cuda.synchronize()
    f32 = np.float32
    bf = lambda v: float(W.round_bf16(np.array([v], dtype=np.float32))[0])
    A = np.zeros((32, 16))
    Bm = np.zeros((16, 32))
    for m in range(32):
        for k in range(16):
            la, e = m + 32 * (k // 8), k % 8
            A[m, k] = bf(f32(1) + f32(1e-3) * f32(la)) if e % 2 == 0 else bf(f32(1) - f32(1e-3) * f32(e // 2))
    for k in range(16):
        for n in range(32):
            lb, e = n + 32 * (k // 8), k % 8
            Bm[k, n] = bf(f32(1e-3) * f32(e // 2)) if e % 2 == 0 else bf(f32(1e-3) * f32(lb))
    C = A @ Bm
    exp = np.array([sum(C[8 * (r // 4) + 4 * (l // 32) + r % 4, l % 32] for r in range(16)) for l in range(64)])
    exp = 8 * iters * exp
    got = host(sink).reshape(grid * 4, 64)
    err = float(np.max(np.abs(got - exp[None, :]) / np.abs(exp[None, :])))
    say(f"  max relative error {err:.2e}")
    assert err <= 1e-4


# ---------------------------------------------------------------------------
# non-salient value-change update, and the row copies that keep its caches
# ---------------------------------------------------------------------------
def run_dv_update(dlm, B, S, Hq, Hkv, hd, n_per_b, dtype="bf16", seed=31, loose_bound=None, sal=None):
    """Previous step: each position's query and LSE over the old K (its last
    computation) and a cached output.  This step: the salient rows get new V.
    On the device the old K/V rows are gathered from the caches before the new
    values are scattered in (both bit-exact), then the update runs; every row
    is compared with the oracle, and salient rows must be left untouched."""
    rng = np.random.default_rng(seed)
    rnd = W.round_bf16 if dtype == "bf16" else (lambda a: np.asarray(a, np.float32).astype(np.float64))
    scale = 1.0 / math.sqrt(hd)
    G = Hq // Hkv
    k_old_c = rnd(rng.standard_normal((B, S, Hkv, hd)))
    v_old_c = rnd(rng.standard_normal((B, S, Hkv, hd)))
    q = rnd(rng.standard_normal((B, S, Hq, hd)))
    lse = np.zeros((B, S, Hq))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, :, h] @ k_old_c[b, :, h // G].T)
            m = s.max(axis=1, keepdims=True)
            lse[b, :, h] = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    lse = lse.astype(np.float32).astype(np.float64)
    o = rnd(0.5 * rng.standard_normal((B, S, Hq, hd)))
    if sal is None:
        sal = [np.sort(rng.choice(S, n, replace=False)).astype(np.int32) for n in n_per_b]
    else:
        sal = [np.asarray(x, np.int32) for x in sal]
        n_per_b = [len(x) for x in sal]
    idx = np.concatenate(sal).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(n_per_b)]).astype(np.int32)
    v_new_c = v_old_c.copy()
    for b in range(B):
        v_new_c[b, sal[b]] = rnd(rng.standard_normal((len(sal[b]), Hkv, hd)))
    n = int(offsets[-1])
    bound = n if loose_bound is None else loose_bound   # host-side row bound (>= the device count)
    say(f"[dv update] {dtype} B={B} S={S} Hq={Hq} Hkv={Hkv} hd={hd} salient per row {list(n_per_b)} bound {bound}")
    kd, vd = dev(k_old_c, dtype), dev(v_old_c, dtype)
    k_rows = torch.zeros(max(bound, 1), Hkv, hd, dtype=kd.dtype, device="cuda")
    v_rows = torch.zeros_like(k_rows)
    it, ot = i32(idx), i32(offsets)
    dlm.dlm_gather_rows(kd, it, ot, bound, k_rows)
    dlm.dlm_gather_rows(vd, it, ot, bound, v_rows)
    new_rows = torch.zeros_like(k_rows)
    new_rows[:n] = dev(O.gather_rows(v_new_c, idx, offsets), dtype)
    dlm.dlm_scatter_rows(new_rows, it, ot, bound, vd)
    od = dev(o, dtype)
    dlm.dlm_nonsalient_dv_update(dev(q, dtype), dev(lse, "f32"), it, ot, bound, k_rows, v_rows, vd, scale, od)
    torch.cuda.synchronize()
    k_old, v_old = O.gather_rows(k_old_c, idx, offsets), O.gather_rows(v_old_c, idx, offsets)
    assert np.array_equal(host(k_rows)[:n], k_old) and np.array_equal(host(v_rows)[:n], v_old)
    assert np.array_equal(host(vd), v_new_c)
    ref = O.nonsalient_dv_update(q, lse, idx, offsets, k_old, v_old, v_new_c, o, Hq, Hkv, scale)
    got = host(od)
    for b in range(B):
        assert np.array_equal(got[b, sal[b]], o[b, sal[b]])
    err, moved = maxabs(got, ref), maxabs(ref, o)
    say(f"  max |o - oracle| = {err:.2e}; largest update {moved:.2e}")
    assert err <= TOL[dtype]
    assert moved > 0.05


def test_dv_update_mha_ragged_with_empty_row(dlm):
    """MHA, d = 128; 300 positions (ragged last position tile); salient sets of
    70 (a full and a ragged 64-row tile), none, and 13."""
    run_dv_update(dlm, B=3, S=300, Hq=4, Hkv=4, hd=128, n_per_b=[70, 0, 13])


@pytest.mark.parametrize("Hq,Hkv", [(8, 4), (8, 2)])
def test_dv_update_gqa(dlm, Hq, Hkv):
    """GQA 2:1 and 4:1 (two or four query heads per KV head in a position
    tile); one salient set of exactly two tiles, one ragged."""
    run_dv_update(dlm, B=2, S=257, Hq=Hq, Hkv=Hkv, hd=128, n_per_b=[128, 65], seed=32)


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(32, 16), (32, 8)])
def test_dv_update_many_position_tiles(dlm, hd, Hq, Hkv):
    """Enough position tiles (B = 2, S = 2048) for two 256-vector workgroups
    per CU: GQA 2:1 runs them, GQA 4:1 the 128-vector workgroups; salient sets
    of 300 and 777 rows (ragged last tiles)."""
    run_dv_update(dlm, B=2, S=2048, Hq=Hq, Hkv=Hkv, hd=hd, n_per_b=[300, 777], seed=37)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4)])
def test_dv_update_clustered_and_dense_salient_sets(dlm, Hq, Hkv):
    """Salient sets that a wave's stable positions must be found around: a run
    of 300 consecutive salient positions among scattered ones (a wave whose
    ranks straddle the run reads several 64-row windows of the salient list),
    95 % salient, all but three salient, and every position salient (nothing
    to update in that sequence)."""
    S = 700
    rng = np.random.default_rng(39)
    scattered = rng.choice(np.setdiff1d(np.arange(S), np.arange(100, 400)), 20, replace=False)
    sal = [np.sort(np.concatenate([np.arange(100, 400), scattered])),
           np.sort(rng.choice(S, 665, replace=False)),
           np.setdiff1d(np.arange(S), [0, 350, 699]),
           np.arange(S)]
    run_dv_update(dlm, B=4, S=S, Hq=Hq, Hkv=Hkv, hd=128, n_per_b=None, seed=40, sal=sal)


def test_dv_update_loose_row_bound(dlm):
    """A host-side row bound far above the device count (as a caller without the
    selection count passes it): every call, the row copies included, stops at
    the device's offsets."""
    run_dv_update(dlm, B=2, S=300, Hq=8, Hkv=2, hd=128, n_per_b=[45, 70], seed=38, loose_bound=600)


def test_dv_update_head_dim_64(dlm):
    run_dv_update(dlm, B=1, S=200, Hq=4, Hkv=2, hd=64, n_per_b=[37], seed=33)


def test_dv_update_one_layer_full_size(dlm):
    """One bf16 layer of 1024 positions, 32 heads x 128, 102 salient rows: all
    922 stable rows of every head against the oracle."""
    run_dv_update(dlm, B=1, S=1024, Hq=32, Hkv=32, hd=128, n_per_b=[102], seed=34)


def test_dv_update_fp32_tiny_layer(dlm):
    """The tiny fp32 layer: 128 positions, 4 heads x 64, 16 salient rows."""
    run_dv_update(dlm, B=1, S=128, Hq=4, Hkv=4, hd=64, n_per_b=[16], dtype="f32", seed=35)


def test_row_copies_four_byte_rows(dlm):
    """Rows of 12 bytes (an LSE row of 3 heads): the 4-byte copy path; gather
    and scatter bit-exact, other rows untouched."""
    rng = np.random.default_rng(36)
    B, S, H = 2, 50, 3
    cache = rng.standard_normal((B, S, H)).astype(np.float32)
    idx = np.array([3, 49, 0, 7, 8], np.int32)
    offsets = np.array([0, 2, 5], np.int32)
    cd = torch.from_numpy(cache).cuda()
    rows = torch.zeros(5, H, dtype=torch.float32, device="cuda")
    dlm.dlm_gather_rows(cd, i32(idx), i32(offsets), 5, rows)
    new = rng.standard_normal((5, H)).astype(np.float32)
    dlm.dlm_scatter_rows(torch.from_numpy(new).cuda(), i32(idx), i32(offsets), 5, cd)
    torch.cuda.synchronize()
    assert np.array_equal(rows.cpu().numpy(), O.gather_rows(cache, idx, offsets))
    assert np.array_equal(cd.cpu().numpy(), O.scatter_rows(new, idx, offsets, cache))


def test_row_copies_more_rows_than_workgroups(dlm):
    """22,793 selected rows of 16-byte units (more rows than the copy's
    16,384 workgroups, so most workgroups copy a second row; a ragged split
    over 13 batch rows, one of them empty) with a loose bound: gather and
    scatter bit-exact against the oracle, unselected rows untouched."""
    rng = np.random.default_rng(37)
    B, S, H = 13, 2500, 24  # 96-byte rows: six 16-byte units
    keep = [rng.random(S) < f for f in np.linspace(0.5, 1.0, B)]
    keep[4][:] = False
    idx = np.concatenate([np.nonzero(k)[0] for k in keep]).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum([k.sum() for k in keep])]).astype(np.int32)
    n = int(offsets[-1])
    say(f"[row copies] B={B} S={S} rows={n} bound={n + 100}")
    assert n > 16384 + 4096
    cache = rng.standard_normal((B, S, H)).astype(np.float32)
    cd = torch.from_numpy(cache).cuda()
    rows = torch.full((n + 100, H), -3.0, dtype=torch.float32, device="cuda")
    dlm.dlm_gather_rows(cd, i32(idx), i32(offsets), n + 100, rows)
    new = rng.standard_normal((n, H)).astype(np.float32)
    dlm.dlm_scatter_rows(torch.from_numpy(new).cuda(), i32(idx), i32(offsets), n, cd)
    torch.cuda.synchronize()
    got = rows.cpu().numpy()
    assert np.array_equal(got[:n], O.gather_rows(cache, idx, offsets))
    assert np.all(got[n:] == -3.0), "rows past the selection were written"
    assert np.array_equal(cd.cpu().numpy(), O.scatter_rows(new, idx, offsets, cache))


# ---------------------------------------------------------------------------
# FFN of the salient rows (SwiGLU; gate and up interleaved by row)
# ---------------------------------------------------------------------------
def run_salient_ffn(dlm, B, S, D, F, n_per_b, seed=41, loose_bound=None):
    rng = np.random.default_rng(seed)
    x = W.round_bf16(rng.standard_normal((B, S, D)))
    w_gu = W.round_bf16(rng.standard_normal((2 * F, D)) / math.sqrt(D))
    w_down = W.round_bf16(rng.standard_normal((D, F)) / math.sqrt(F))
    cache = W.round_bf16(rng.standard_normal((B, S, D)))
    sal = [np.sort(rng.choice(S, n, replace=False)).astype(np.int32) for n in n_per_b]
    idx = np.concatenate(sal).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(n_per_b)]).astype(np.int32)
    n = int(offsets[-1])
    max_rows = n if loose_bound is None else loose_bound
    say(f"[salient ffn] B={B} S={S} D={D} F={F} rows {list(n_per_b)} bound {max_rows}")
    out = dev(cache, "bf16")
    ws = workspace(dlm.dlm_salient_ffn_workspace_size(dlm.DLM_BF16, max_rows, D, F))
    dlm.dlm_salient_ffn(dev(x, "bf16"), i32(idx), i32(offsets), max_rows, dev(w_gu, "bf16"), dev(w_down, "bf16"),
                        out, workspace=ws)
    torch.cuda.synchronize()
    h_ref, ref = O.salient_ffn(x, idx, offsets, w_gu, w_down, cache)
    got = host(out)
    mask = rows_mask(B, S, idx, offsets)
    assert np.array_equal(got[~mask], cache[~mask])
    err = maxabs(got[mask], ref[mask])
    # h, the bf16 intermediate in the workspace (not an output), reaches |h| ~ 16
    # at 4 sigma: checked relative to its size (half a bf16 ulp is 2^-9 of it)
    h = host(ws[:n * F * 2].view(torch.bfloat16).reshape(n, F))
    eh = float(np.max(np.abs(h - h_ref) - 2.0 ** -7 * np.abs(h_ref)))
    say(f"  max |y - oracle| = {err:.2e}; max of |h - oracle| - 2^-7 |h| = {eh:.2e}")
    assert err <= TOL["bf16"] and eh <= TOL["bf16"]


def test_salient_ffn_short_selection(dlm):
    """100 rows: the weight-streaming tilings (two batch rows, one empty)."""
    run_salient_ffn(dlm, B=2, S=512, D=1024, F=1024, n_per_b=[100, 0])


def test_salient_ffn_short_selection_loose_bound(dlm):
    """40 rows under a bound of 128 (the device plans the down projection's
    K split from the real count): 32 output tiles split 4 ways."""
    run_salient_ffn(dlm, B=2, S=512, D=2048, F=2048, n_per_b=[30, 10], seed=46, loose_bound=128)


def test_salient_ffn_no_rows(dlm):
    """An empty selection under a bound of 64: nothing is written."""
    B, S, D, F = 2, 256, 1024, 2048
    rng = np.random.default_rng(47)
    x = dev(W.round_bf16(rng.standard_normal((B, S, D))), "bf16")
    w_gu = dev(W.round_bf16(rng.standard_normal((2 * F, D)) / 32), "bf16")
    w_down = dev(W.round_bf16(rng.standard_normal((D, F)) / 45), "bf16")
    cache = W.round_bf16(rng.standard_normal((B, S, D)))
    out = dev(cache, "bf16")
    ws = workspace(dlm.dlm_salient_ffn_workspace_size(dlm.DLM_BF16, 64, D, F))
    dlm.dlm_salient_ffn(x, i32(np.zeros(64, np.int32)), i32(np.zeros(B + 1, np.int32)), 64, w_gu, w_down, out,
                        workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), cache)


def test_salient_ffn_long_selection_split_k(dlm):
    """1300 rows: the resident 256x256 tiling with split-K partials (workspace)."""
    run_salient_ffn(dlm, B=2, S=1024, D=512, F=1536, n_per_b=[700, 600], seed=42)


def test_salient_ffn_short_k_and_loose_bound(dlm):
    """K / 64 not a multiple of 4 (D = 320, F = 640) with a loose row bound."""
    run_salient_ffn(dlm, B=1, S=1024, D=320, F=640, n_per_b=[300], seed=43, loose_bound=1024)


def test_salient_ffn_many_rows_unsplit_tiles(dlm):
    """2048 rows (two batch rows of 1024) with 256 gate/up output tiles: the
    resident 256 x 256 tiling with the SwiGLU epilogue inside the GEMM kernel
    (no split-K), as the benchmark's 2048-row case runs it; the down
    projection has 8 tiles and splits K."""
    run_salient_ffn(dlm, B=2, S=1024, D=256, F=4096, n_per_b=[1024, 1024], seed=45)


def test_salient_ffn_one_layer_full_size(dlm):
    """One layer of 1024 positions, D = 4096, F = 12288, 102 salient rows."""
    run_salient_ffn(dlm, B=1, S=1024, D=4096, F=12288, n_per_b=[102], seed=44)


# ---------------------------------------------------------------------------
# LSP: logit margin scores and the adaptive-threshold commit
# ---------------------------------------------------------------------------
def margin_select(dlm, h, w_lm, rows, lo, S):
    """Margin scores (and argmax) of the listed rows through the select call."""
    B = h.shape[0]
    ev_idx, ev_off = W.pack_rows(rows)
    scores = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    argmax = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    idx = torch.zeros(B * S, dtype=torch.int32, device="cuda")
    counts = torch.zeros(B, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(B + 1, dtype=torch.int32, device="cuda")
    ws = workspace(dlm.dlm_select_workspace_size(dlm.DLM_SCORE_MARGIN, B, S, w_lm.shape[0], len(ev_idx)))
    dlm.dlm_saliency_select(dlm.DLM_SCORE_MARGIN, dev(h, "bf16"), dev(w_lm, "bf16"), lo=lo, hi=S, threshold=0.5,
                            idx=idx, counts=counts, offsets=offsets, scores=scores, argmax=argmax,
                            eval_idx=i32(ev_idx), eval_offsets=i32(ev_off), max_eval=len(ev_idx), workspace=ws)
    torch.cuda.synchronize()
    return scores, argmax


def check_margins(h, w_lm, rows, scores, argmax, sample=None):
    sc, am = scores.cpu().numpy(), argmax.cpu().numpy()
    worst, n = 0.0, 0
    for b, r in enumerate(rows):
        pick = np.asarray(r) if sample is None else np.asarray(r)[np.linspace(0, len(r) - 1, sample).astype(int)]
        m, a = O.logit_margin(h[b, pick], w_lm)
        clear = m > BAND
        assert np.array_equal(am[b, pick][clear], a[clear]), f"b {b}: argmax"
        worst = max(worst, maxabs(sc[b, pick], m))
        n += len(pick)
    say(f"  {n} rows: margin err {worst:.2e}")
    assert worst <= TOL["bf16"]


def test_margin_scores_small(dlm):
    """A few evaluated rows (split-K LM-head tiles and their reduce pass):
    margins and argmax against the oracle; rows not evaluated keep -1."""
    rng = np.random.default_rng(51)
    B, S, D, V = 2, 96, 512, 2048
    h = W.round_bf16(rng.standard_normal((B, S, D)))
    w = W.round_bf16(rng.standard_normal((V, D)) * 0.05)
    rows = [np.arange(40, 70), np.arange(10, 19)]
    say(f"[margin small] B={B} S={S} D={D} V={V}")
    scores, argmax = margin_select(dlm, h, w, rows, 0, S)
    check_margins(h, w, rows, scores, argmax)
    assert argmax[0, 0].item() == -1 and argmax[1, 95].item() == -1


def test_margin_scores_lsp_workload_full_size(dlm):
    """The LSP workload's first step at full size (B = 16, S = 1024, D = 4096,
    V = 32768, the active rows): 48 sampled rows against the oracle."""
    sh = W.LSP_COMMIT
    inp = W.lsp_inputs(sh)
    rows = inp.active_rows(0)
    h = inp.hidden(0)
    say(f"[margin full size] B={sh.B} S={sh.S} D={sh.D} V={sh.V}")
    scores, argmax = margin_select(dlm, h, inp.w_lm, rows, sh.prompt, sh.S)
    check_margins(h, inp.w_lm, rows, scores, argmax, sample=3)


def test_lsp_adaptive_commit_bit_exact(dlm):
    """On given float32 margins (ties on purpose, every frontier including the
    done and one-left cases, three fraction ranges, no floor and three margin
    floors, the last above every margin so only the fallback commits):
    committed and tau identical to the oracle."""
    rng = np.random.default_rng(52)
    B, S, gen_lo = 16, 700, 100
    G = S - gen_lo
    for fl, fh, floor in [(0.25, 0.5, -math.inf), (0.1, 0.3, -math.inf), (0.5, 0.5, -math.inf),
                          (0.25, 0.5, 0.5), (0.25, 0.5, 1.5), (0.1, 0.3, 100.0)]:
        m = np.round(rng.standard_normal((B, S)) * 2, 1).astype(np.float32)
        com = rng.integers(0, G + 1, B).astype(np.int32)
        com[0], com[1], com[2] = G, G - 1, 0
        ct = i32(com)
        tau = torch.zeros(B, dtype=torch.float32, device="cuda")
        dlm.dlm_lsp_adaptive_commit(torch.from_numpy(m).cuda(), gen_lo, S, ct, fl, fh, tau=tau, margin_floor=floor)
        torch.cuda.synchronize()
        want, wt = O.lsp_adaptive_commit(m, gen_lo, S, com, float(np.float32(fl)), float(np.float32(fh)),
                                         margin_floor=floor)
        assert np.array_equal(ct.cpu().numpy(), want)
        got_t = tau.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got_t), np.isnan(wt))
        assert np.array_equal(got_t[~np.isnan(wt)], wt[~np.isnan(wt)])


def test_lsp_margin_commit_loop(dlm):
    """A decoding loop on the library alone: margins of the active rows, then the
    adaptive commit, until every generated position is committed; each commit
    equals the oracle's on the same margins, and each step commits between
    the fraction bounds."""
    rng = np.random.default_rng(53)
    B, S, D, V, gen_lo = 3, 192, 256, 1024, 64
    G = S - gen_lo
    w = W.round_bf16(rng.standard_normal((V, D)) * 0.05)
    com = torch.zeros(B, dtype=torch.int32, device="cuda")
    steps = 0
    say(f"[margin loop] B={B} S={S} D={D} V={V}")
    while int(com.min().item()) < G:
        h = W.round_bf16(rng.standard_normal((B, S, D)))
        c = com.cpu().numpy()
        rows = [np.arange(gen_lo + int(c[b]), S) if c[b] < G else np.arange(gen_lo, gen_lo + 1) for b in range(B)]
        scores, _ = margin_select(dlm, h, w, rows, gen_lo, S)
        dlm.dlm_lsp_adaptive_commit(scores, gen_lo, S, com)
        torch.cuda.synchronize()
        want, _ = O.lsp_adaptive_commit(scores.cpu().numpy(), gen_lo, S, c)
        got = com.cpu().numpy()
        assert np.array_equal(got, want)
        for b in range(B):
            A = G - int(c[b])
            if A > 0:
                assert max(1, math.ceil(0.25 * A)) <= got[b] - c[b] <= max(1, math.ceil(0.25 * A), math.floor(0.5 * A))
        steps += 1
        assert steps < 40
    say(f"  done in {steps} steps")


def test_colsum_key_window_only(dlm):
    """Attn-Sampler's block-wise column sums: the window call computes the key
    blocks covering [key_lo, key_hi) only. Inside the window its sums match the
    full call's and the oracle's; outside the covering blocks nothing is
    written; its top-k is exact on its own sums."""
    rng = np.random.default_rng(61)
    B, S, Hq, Hkv, hd = 2, 1500, 8, 4, 128
    scale = 1.0 / math.sqrt(hd)
    kc = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    vc = W.round_bf16(rng.standard_normal((B, S, Hkv, hd)))
    rows = [np.sort(rng.choice(S, 64, replace=False)), np.sort(rng.choice(S, 40, replace=False))]
    idx = np.concatenate(rows).astype(np.int32)
    offsets = np.array([0, 64, 104], np.int32)
    q = W.round_bf16(rng.standard_normal((104, Hq, hd)))
    _, lse = O.partial_attention(q, idx, offsets, kc, vc, Hq, Hkv, scale)
    c_o = O.column_sums(q, offsets, kc, lse, Hq, Hkv, scale)
    lo, hi, kk = 600, 1100, 16
    say(f"[colsum window] B={B} S={S} window [{lo},{hi}) k={kk}")
    qd, kd, ld, od = dev(q, "bf16"), dev(kc, "bf16"), dev(lse, "f32"), i32(offsets)
    ws = workspace(dlm.dlm_attn_colsum_workspace_size(B, S, Hkv))
    full = torch.zeros(B, S, dtype=torch.float32, device="cuda")
    dlm.dlm_attn_colsum(qd, od, 104, kd, ld, scale, full, workspace=ws)
    win = torch.full((B, S), -1.0, dtype=torch.float32, device="cuda")
    ti = torch.zeros(B, kk, dtype=torch.int32, device="cuda")
    tv = torch.zeros(B, kk, dtype=torch.float32, device="cuda")
    dlm.dlm_attn_colsum(qd, od, 104, kd, ld, scale, win, key_lo=lo, key_hi=hi, k=kk, topk_idx=ti, topk_val=tv,
                        workspace=ws, window_only=True)
    torch.cuda.synchronize()
    f, w = full.cpu().numpy(), win.cpu().numpy()
    assert np.allclose(w[:, lo:hi], f[:, lo:hi], rtol=1e-5, atol=1e-6)
    assert maxabs(w[:, lo:hi], c_o[:, lo:hi]) <= TOL["bf16"]
    assert np.all(w[:, :512] == -1.0) and np.all(w[:, 1280:] == -1.0)   # blocks [512, 1280) cover the window
    for b in range(B):
        order = np.lexsort((np.arange(lo, hi), -w[b, lo:hi].astype(np.float64)))[:kk] + lo
        assert np.array_equal(ti[b].cpu().numpy(), order)
        assert np.array_equal(tv[b].cpu().numpy(), w[b, order])
