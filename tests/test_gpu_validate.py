"""DLM_VALIDATE=1: the calls that scatter rows check the selection's index
arrays on the device first and reject a malformed selection with
DLM_ERR_INVALID_ARG before any other launch, so the caches stay
byte-identical.  Only in-bounds malformed sets (and bounds the check itself
catches before anything else runs) are used; without the variable the same
in-bounds set is trusted as documented."""
import math
import sys

import numpy as np
import pytest
import torch

from sparse_query_attention_dlm_amd import workloads as W
from helpers import dev, i32, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dlm():
    from sparse_query_attention_dlm_amd import binding
    return binding


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


B, S, D, Hq, Hkv, hd = 2, 96, 256, 4, 2, 64


def state(seed=5):
    rng = np.random.default_rng(seed)
    x = dev(W.round_bf16(rng.standard_normal((B, S, D))), "bf16")
    w = dev(W.round_bf16(rng.standard_normal(((Hq + 2 * Hkv) * hd, D)) / 16), "bf16")
    kc = dev(W.round_bf16(rng.standard_normal((B, S, Hkv, hd))), "bf16")
    vc = dev(W.round_bf16(rng.standard_normal((B, S, Hkv, hd))), "bf16")
    out = dev(W.round_bf16(rng.standard_normal((B, S, Hq * hd))), "bf16")
    return x, w, kc, vc, out


def calls(dlm, idx, offsets, max_rows, x, w, kc, vc, out):
    """The scattering calls of one step on the given selection; each returns
    the DlmError it raised (or None)."""
    q = torch.zeros(max_rows, Hq, hd, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    errs = []
    for f in (lambda: dlm.dlm_gather_qkv_scatter_kv(x, idx, offsets, max_rows, w, Hq, Hkv, hd, q, kc, vc),
              lambda: dlm.dlm_partial_attn(q, idx, offsets, max_rows, kc, vc, 1.0 / math.sqrt(hd), o,
                                           out_cache=out),
              lambda: dlm.dlm_scatter_rows(q.view(max_rows, Hq * hd), idx, offsets, max_rows, out)):
        try:
            f()
            errs.append(None)
        except dlm.DlmError as e:
            errs.append(e)
    torch.cuda.synchronize()
    return errs


MALFORMED = {
    "unordered": ([5, 3, 9, 1, 2], [0, 3, 5], 5),          # in bounds, row 0 out of order
    "repeated": ([5, 5, 9, 1, 2], [0, 3, 5], 5),           # a position twice in a row
    "past_sequence": ([5, 7, 96, 1, 2], [0, 3, 5], 5),     # position S
    "negative": ([5, 7, 9, -1, 2], [0, 3, 5], 5),
    "offsets_decrease": ([5, 7, 9, 1, 2], [0, 3, 2], 5),
    "offsets_start": ([5, 7, 9, 1, 2], [1, 3, 5], 5),
    "offsets_past_bound": ([5, 7, 9, 1, 2], [0, 3, 5], 4),
}


@pytest.mark.parametrize("case", sorted(MALFORMED))
def test_validate_rejects_before_any_scatter(dlm, monkeypatch, case):
    monkeypatch.setenv("DLM_VALIDATE", "1")
    idx, offsets, max_rows = MALFORMED[case]
    say(f"[validate] {case}: idx={idx} offsets={offsets} max_rows={max_rows}")
    x, w, kc, vc, out = state()
    before = [t.clone() for t in (kc, vc, out)]
    errs = calls(dlm, i32(idx), i32(offsets), max_rows, x, w, kc, vc, out)
    for e in errs:
        assert e is not None and e.status == dlm.DLM_ERR_INVALID_ARG, f"{case}: {e}"
        assert "DLM_VALIDATE" in str(e)
    for t, t0 in zip((kc, vc, out), before):
        assert torch.equal(t, t0), f"{case}: a cache changed"


def test_validate_accepts_valid_selection(dlm, monkeypatch):
    monkeypatch.setenv("DLM_VALIDATE", "1")
    x, w, kc, vc, out = state()
    before = kc.clone()
    errs = calls(dlm, i32([1, 5, 95, 0, 2]), i32([0, 3, 5]), 8, x, w, kc, vc, out)
    assert errs == [None, None, None]
    assert not torch.equal(kc, before)


def test_validate_column_sums_checks_offsets(dlm, monkeypatch):
    monkeypatch.setenv("DLM_VALIDATE", "1")
    q = torch.zeros(5, Hq, hd, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, S, Hkv, hd, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(5, Hq, dtype=torch.float32, device="cuda")
    cs = torch.full((B, S), -1.0, dtype=torch.float32, device="cuda")
    ws = workspace(dlm.dlm_attn_colsum_workspace_size(B, S, Hkv))
    with pytest.raises(dlm.DlmError) as ei:
        dlm.dlm_attn_colsum(q, i32([0, 4, 3]), 5, kc, lse, 0.1, cs, workspace=ws)
    assert ei.value.status == dlm.DLM_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(cs == -1.0)


def test_without_validate_in_bounds_selection_is_trusted(dlm, monkeypatch):
    """Off by default: an unordered but in-bounds selection is not checked and
    the calls run (they stay inside the caches)."""
    monkeypatch.delenv("DLM_VALIDATE", raising=False)
    x, w, kc, vc, out = state()
    errs = calls(dlm, i32([5, 3, 9, 1, 2]), i32([0, 3, 5]), 5, x, w, kc, vc, out)
    assert errs == [None, None, None]
