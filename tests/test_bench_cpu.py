"""CPU checks of the benchmark's contract and of the lock loop's work figures
(no GPU needed)."""
import os
import subprocess
import sys

from sparse_query_attention_dlm_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    """--gpus N > 1 stops before anything touches a GPU, with exit status 2 and
    a message that this build measures one GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def test_lock_loop_row_schedule():
    """The 64-step loop's unlocked counts: floor(0.95 t / 63 * 2048) locked
    positions per sequence, so M runs 2048 -> 103 and the loop recomputes
    550,752 rows over 8 sequences."""
    s = W.GQA_LOCK_LOOP
    m = [W.unlocked_count(s.S, t, s.steps, s.lock_max) for t in range(s.steps)]
    assert (s.B, s.S, s.steps) == (8, 2048, 64)
    assert m[0] == 2048 and m[-1] == 103
    assert all(a >= b for a, b in zip(m, m[1:]))
    assert s.B * sum(m) == 550_752


def test_lock_loop_work_figures():
    """Algorithmic work of the loop as the benchmark counts it: Q/K/V
    2 D (Hq + 2 Hkv) d flop per recomputed row (50.33 MFLOP), attention
    4 S d Hq flop per row (33.55 MFLOP); 27.72 and 18.48 TFLOP over the loop."""
    s = W.GQA_LOCK_LOOP
    rows = s.B * sum(W.unlocked_count(s.S, t, s.steps, s.lock_max) for t in range(s.steps))
    qkv_row = 2.0 * s.D * (s.Hq + 2 * s.Hkv) * s.hd
    attn_row = 4.0 * s.S * s.hd * s.Hq
    assert round(qkv_row / 1e6, 2) == 50.33
    assert round(attn_row / 1e6, 2) == 33.55
    assert round(rows * qkv_row / 1e12, 2) == 27.72
    assert round(rows * attn_row / 1e12, 2) == 18.48
