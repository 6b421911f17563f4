"""SureLock's lock criterion on the GPU (dlm_kl_lock) against the oracle:
the local KL divergence between consecutive posteriors, this step's max
probability and argmax of every evaluated position; the lock decision (KL
below eps, optionally gated by the nearest-rank percentile of the
uncertainty) taken on the library's own float32 values must equal the
oracle's rule applied to those same values, bit for bit."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import dlm_oracle as O
from sparse_query_attention_dlm_amd import workloads as W
from helpers import BAND, TOL, dev, i32, maxabs, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dlm():
    from sparse_query_attention_dlm_amd import binding
    return binding


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_kl_lock(dlm, h_cur, h_prev, w_lm, rows, eps, gate_q, sample=None, locked0=None):
    B, S, D = h_cur.shape
    V = w_lm.shape[0]
    ev_idx, ev_off = W.pack_rows(rows)
    n = len(ev_idx)
    kl = torch.full((B, S), -5.0, dtype=torch.float32, device="cuda")
    mp = torch.full((B, S), -5.0, dtype=torch.float32, device="cuda")
    am = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    lk0 = np.zeros((B, S), np.float32) if locked0 is None else locked0
    lk = torch.from_numpy(lk0.copy()).cuda()
    ws = workspace(dlm.dlm_kl_lock_workspace_size(B, S, V, n))
    dlm.dlm_kl_lock(dev(h_cur, "bf16"), dev(h_prev, "bf16"), dev(w_lm, "bf16"), i32(ev_idx), i32(ev_off), n,
                    eps, kl, mp, am, lk, gate_q=gate_q, workspace=ws)
    torch.cuda.synchronize()
    kl_g, mp_g, am_g, lk_g = kl.cpu().numpy(), mp.cpu().numpy(), am.cpu().numpy(), lk.cpu().numpy()
    # values against the oracle (all evaluated rows, or a sample per sequence)
    worst_kl = worst_mp = 0.0
    checked = 0
    for b in range(B):
        r = np.asarray(rows[b])
        if r.size == 0:
            continue
        pick = r if sample is None else r[np.linspace(0, r.size - 1, sample).astype(np.int64)]
        k_o, m_o, a_o, gap = O.kl_divergence(h_cur[b, pick], h_prev[b, pick], w_lm)
        clear = gap > BAND
        assert np.array_equal(am_g[b, pick][clear], a_o[clear]), f"sequence {b}: argmax"
        worst_kl = max(worst_kl, maxabs(kl_g[b, pick], k_o))
        worst_mp = max(worst_mp, maxabs(mp_g[b, pick], m_o))
        checked += pick.size
    say(f"  {checked} rows: kl err {worst_kl:.2e}, max-prob err {worst_mp:.2e}")
    assert worst_kl <= TOL["bf16"] and worst_mp <= TOL["bf16"]
    # the decision: exact on the library's own float32 values
    want = O.surelock_lock(kl_g, mp_g, ev_idx, ev_off, lk0, np.float32(eps), gate_q)
    assert np.array_equal(lk_g, want.astype(np.float32)), "lock decision differs from the rule"
    # nothing written outside the evaluated positions
    mask = np.zeros((B, S), bool)
    for b in range(B):
        mask[b, np.asarray(rows[b], np.int64)] = True
    assert np.all(kl_g[~mask] == -5.0) and np.all(am_g[~mask] == -1)
    return kl_g, lk_g, want


@pytest.mark.parametrize("gate_q", [0.0, 0.5])
def test_kl_lock_small_split_k(dlm, gate_q):
    """A few evaluated rows per sequence (the LM head splits K over spare
    workgroups: the epilogue runs in the reduce pass); half the positions
    barely move between the steps (small KL), the others are redrawn; one
    sequence evaluates nothing."""
    rng = np.random.default_rng(71)
    B, S, D, V = 3, 160, 256, 2048
    h_prev = W.round_bf16(rng.standard_normal((B, S, D)) * 2.0)
    h_cur = h_prev + 0.02 * rng.standard_normal((B, S, D))
    moved = rng.random((B, S)) < 0.5
    h_cur[moved] = 2.0 * rng.standard_normal((int(moved.sum()), D))
    h_cur = W.round_bf16(h_cur)
    w = W.round_bf16(rng.standard_normal((V, D)) * 0.1)
    rows = [np.sort(rng.choice(S, 45, replace=False)), np.array([], np.int64), np.sort(rng.choice(S, 30, replace=False))]
    say(f"[kl lock small] B={B} S={S} D={D} V={V} gate_q={gate_q}")
    lk0 = np.zeros((B, S), np.float32)
    lk0[0, rows[0][:3]] = 1.0   # already locked stay locked
    kl, lk, _ = run_kl_lock(dlm, h_cur, h_prev, w, rows, 0.05, gate_q, locked0=lk0)
    assert 0 < int(lk.sum()) - 3 < 75


def test_kl_lock_lsp_workload_full_size(dlm):
    """The confidence workload's second step at full size (B = 16, S = 1024,
    D = 4096, V = 32768, 230 evaluated positions per sequence), against its
    first step: planted positions keep their token (small KL), flip rows
    change it.  KL, max-prob and argmax of 16 positions per sequence against
    the oracle; the lock decision with the gate at the 50th percentile exact
    on the library's own values for all 3680 positions."""
    sh = W.LSP_COMMIT
    inp = W.lsp_inputs(sh)
    rows = inp.active_rows(1)
    say(f"[kl lock full size] B={sh.B} S={sh.S} D={sh.D} V={sh.V}")
    kl, lk, _ = run_kl_lock(dlm, inp.hidden(1), inp.hidden(0), inp.w_lm, rows, 0.05, 0.5, sample=16)
    n_lock = int(lk.sum())
    say(f"  locked {n_lock} of {sum(len(r) for r in rows)}")
    assert n_lock > 0
