"""Shared helpers of the GPU tests: device transfer, workspaces and the
comparison rules (float tolerances, index sets modulo the 1e-4 threshold band)."""
import numpy as np
import torch

BAND = 1e-4          # scores within this distance of a threshold may go either way
TOL = {"f32": 1e-4, "bf16": 2e-2}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(a, dtype="f32"):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(TORCH_DT[dtype]) if isinstance(dtype, str) else t.to(dtype)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def workspace(nbytes, fill=0x5A):
    """Device scratch of the requested size, filled with junk: the library must
    not depend on workspace contents."""
    return torch.full((max(int(nbytes), 16),), fill, dtype=torch.uint8, device="cuda")


def maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rows_mask(B, S, idx, offsets):
    m = np.zeros((B, S), dtype=bool)
    for b in range(B):
        m[b, np.asarray(idx[offsets[b]:offsets[b + 1]], dtype=np.int64)] = True
    return m


def check_selection(idx_g, counts_g, offsets_g, scores_o, lo, hi, tau, band=BAND):
    """GPU index set vs the oracle's: identical outside the threshold band,
    ascending and unique inside every batch row, offsets consistent."""
    B = scores_o.shape[0]
    counts_g = np.asarray(counts_g)
    offsets_g = np.asarray(offsets_g)
    assert offsets_g[0] == 0 and np.array_equal(np.diff(offsets_g), counts_g)
    for b in range(B):
        got = np.asarray(idx_g[offsets_g[b]:offsets_g[b + 1]], dtype=np.int64)
        assert np.all(np.diff(got) > 0), "indices not strictly ascending"
        assert np.all((got >= lo) & (got < hi))
        s = scores_o[b]
        amb = {i for i in range(lo, hi) if abs(s[i] - tau) <= band}
        want = {i for i in range(lo, hi) if s[i] < tau}
        assert set(got.tolist()) - amb == want - amb, f"batch row {b}: selection differs"


def check_topk(ti_g, c_o, key_lo, key_hi, k, band=BAND):
    """Top-k set rule: every key whose oracle sum beats the k-th largest by more
    than the band is in, every key below it by more than the band is out."""
    B = c_o.shape[0]
    for b in range(B):
        vals = c_o[b, key_lo:key_hi]
        ck = np.sort(vals)[::-1][k - 1]
        got = set(np.asarray(ti_g[b]).tolist())
        assert len(got) == k
        must = {key_lo + j for j in np.nonzero(vals > ck + band)[0]}
        must_not = {key_lo + j for j in np.nonzero(vals < ck - band)[0]}
        assert must <= got, f"batch row {b}: missing {sorted(must - got)[:5]}"
        assert not (got & must_not), f"batch row {b}: wrongly included {sorted(got & must_not)[:5]}"
