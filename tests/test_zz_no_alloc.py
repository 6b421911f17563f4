"""The allocation-free partial attention (dlm_partial_attn_noalloc) against
the entry point it varies (dlm_partial_attn with a caller workspace), through
the C ABI: two calls in a row on one GPU, the second with a smaller input and
a different split of the keys, so that it runs on the scratch the first call
left behind.  Same kernels and work plan: outputs, LSE and scattered output
rows must be bit-identical."""
import math
import sys

import numpy as np
import pytest
import torch

from sparse_query_attention_dlm_amd import workloads as W
from helpers import dev, i32, workspace

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_call(dlm, B, S, Hq, Hkv, hd, rows_per_b, seed, bound=None):
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(hd)
    kc = dev(W.round_bf16(rng.standard_normal((B, S, Hkv, hd))), "bf16")
    vc = dev(W.round_bf16(rng.standard_normal((B, S, Hkv, hd))), "bf16")
    rows = [np.sort(rng.choice(S, m, replace=False)) for m in rows_per_b]
    idx = i32(np.concatenate(rows))
    offsets = i32(np.concatenate([[0], np.cumsum(rows_per_b)]))
    n = int(sum(rows_per_b))
    max_rows = n if bound is None else bound
    q = dev(W.round_bf16(rng.standard_normal((max_rows, Hq, hd))), "bf16")
    out0 = dev(W.round_bf16(rng.standard_normal((B, S, Hq * hd))), "bf16")
    say(f"[no-alloc attention] B={B} S={S} Hq={Hq} Hkv={Hkv} hd={hd} rows {list(rows_per_b)} bound {max_rows}")
    res = []
    for noalloc in (False, True):
        o = torch.full((max_rows, Hq, hd), 7.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((max_rows, Hq), 7.0, dtype=torch.float32, device="cuda")
        out = out0.clone()
        if noalloc:
            dlm.dlm_partial_attn_noalloc(q, idx, offsets, max_rows, kc, vc, scale, o, lse, out_cache=out)
        else:
            ws = workspace(dlm.dlm_partial_attn_workspace_size(dlm.DLM_BF16, max_rows, B, S, Hq, Hkv, hd))
            dlm.dlm_partial_attn(q, idx, offsets, max_rows, kc, vc, scale, o, lse, out_cache=out, workspace=ws)
        torch.cuda.synchronize()
        res.append((o[:n].clone(), lse[:n].clone(), out))
    (o1, l1, u1), (o2, l2, u2) = res
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(u1, u2)
    assert not torch.equal(u2, out0), "no output row was written"


def test_noalloc_partial_attention_two_calls(dlm_binding):
    dlm = dlm_binding
    assert dlm.dlm_partial_attn_noalloc_scratch_bytes() == 2 * 512 * 128 * 129 * 4
    # first call: keys split four ways (few query tiles over 1024 keys)
    one_call(dlm, B=2, S=1024, Hq=8, Hkv=4, hd=128, rows_per_b=[40, 17], seed=91)
    # second call, smaller: two splits over 600 keys at head dim 64, a loose bound
    one_call(dlm, B=1, S=600, Hq=4, Hkv=2, hd=64, rows_per_b=[23], seed=92, bound=50)


@pytest.fixture(scope="module")
def dlm_binding():
    from sparse_query_attention_dlm_amd import binding
    return binding
