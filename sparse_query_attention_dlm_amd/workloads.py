"""Seeded synthetic inputs for the sparse-query denoising step.

This module only *constructs inputs*: random draws, the planted structure that
makes a workload meaningful, and the one-time rounding of inputs to their
storage precision.  It contains none of the step's arithmetic (no cosine, no
projection, no softmax, no selection), so both the fp64 oracle and the HIP path
can be fed from it without sharing any of the method.

Shapes, value distributions and structure follow the five workloads that the
method pages describe (stand-ins for the benchmarks they evaluate on; no dataset
or trained weight is available here):

* ``tiny_fp32``      - one fp32 layer, S=128, hidden 256, 4 heads x 64, cosine
                        select with 16 resampled rows (DyLLM, Methodologie 1).
* ``bf16_s1024``     - one bf16 layer, S=1024, hidden 4096, 32 heads x 128, ~10 %
                        of rows redrawn (DyLLM, Methodologie 1 and 2).
* ``gqa_lock_loop``  - 64-step loop, GQA 32/8 heads, S=2048, B=8, locked fraction
                        rising 0 -> 95 % (SureLock, Methodik "Kernprinzipien").
* ``colsum_top64``   - B=4, S=4096, attention column sums over the masked region
                        and top-64 (Attention-Based Sampler, Methodologie 2).
* ``lsp_commit``     - B=16, S=1024, LM head 4096 x 32768, confidence + longest
                        stable prefix (Longest Stable Prefixes, Methodologie 2;
                        SlowFast Sampling, Metodologia principles 1-2).
* ``dyllm_loop``     - the bf16 S=1024 layer over 8 steps with a 512-token prompt
                        and a 512-token response (DyLLM, Methodologie 3:
                        response-only input on most steps).

Every generator takes explicit sizes so tests can run reduced versions that
still span several kernel tiles and a ragged tail.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np


# --------------------------------------------------------------------------
# storage rounding (input construction only)
# --------------------------------------------------------------------------
def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bf16.  Inputs
    are assumed finite (all generators here draw finite normals)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x_exact) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x_exact, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits: input is not bf16-exact")
    return (u >> np.uint32(16)).astype(np.uint16)


def to_storage(x, dtype: str) -> np.ndarray:
    """float32 array holding the values as stored on the device ('f32' or 'bf16')."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# workload shapes (full sizes of the five workloads)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class CosineStepShape:
    name: str
    dtype: str
    B: int
    S: int
    D: int
    Hq: int
    Hkv: int
    hd: int
    n_redrawn: int          # rows of `prev` redrawn fresh (per batch row)
    noise_std: float        # std of the perturbation prev - cur on stable rows
    w_std: float            # std of the projection weights
    tau: float              # cosine threshold (selected iff cos < tau)
    with_wo: bool           # project the context through W_o before the scatter
    seed: int


TINY_FP32 = CosineStepShape(
    name="tiny_fp32_s128_h256", dtype="f32", B=1, S=128, D=256, Hq=4, Hkv=4, hd=64,
    n_redrawn=16, noise_std=0.01, w_std=1.0 / 16.0, tau=0.9, with_wo=True, seed=1)

BF16_S1024 = CosineStepShape(
    name="bf16_b1_s1024_d4096_h32x128", dtype="bf16", B=1, S=1024, D=4096, Hq=32, Hkv=32,
    hd=128, n_redrawn=round(0.1 * 1024), noise_std=1e-3, w_std=1.0 / 64.0, tau=0.95,
    with_wo=False, seed=2)


@dataclass(frozen=True)
class LockLoopShape:
    name: str
    B: int
    S: int
    D: int
    Hq: int
    Hkv: int
    hd: int
    steps: int
    lock_max: float
    w_std: float
    seed: int


GQA_LOCK_LOOP = LockLoopShape(
    name="bf16_gqa_b8_s2048_h32kv8_64steps", B=8, S=2048, D=4096, Hq=32, Hkv=8, hd=128,
    steps=64, lock_max=0.95, w_std=1.0 / 64.0, seed=3)


@dataclass(frozen=True)
class ColsumShape:
    name: str
    B: int
    S: int
    prompt: int
    Hq: int
    Hkv: int
    hd: int
    k: int
    seed: int


COLSUM_TOP64 = ColsumShape(
    name="bf16_colsum_b4_s4096_h32x128_top64", B=4, S=4096, prompt=1024, Hq=32, Hkv=32,
    hd=128, k=64, seed=4)


@dataclass(frozen=True)
class LspShape:
    name: str
    B: int
    S: int
    prompt: int
    D: int
    V: int
    active_frac: float
    steps: int
    conf: float
    W: int
    w_std: float
    beta: float
    seed: int


LSP_COMMIT = LspShape(
    name="bf16_lsp_b16_s1024_d4096_v32768", B=16, S=1024, prompt=256, D=4096, V=32768,
    active_frac=0.3, steps=8, conf=0.9, W=3, w_std=0.02, beta=16.0, seed=5)


# --------------------------------------------------------------------------
# cosine-selected single step (tiny_fp32, bf16_s1024)
# --------------------------------------------------------------------------
@dataclass
class CosineStepInputs:
    shape: CosineStepShape
    cur: np.ndarray        # [B,S,D]   storage values (float32 holding f32 or bf16-exact)
    prev: np.ndarray       # [B,S,D]
    w_qkv: np.ndarray      # [(Hq+2Hkv)*hd, D] out-major (row = output feature)
    w_o: np.ndarray | None  # [D_out, Hq*hd] out-major, or None
    redrawn: list          # per batch row: sorted positions whose prev was redrawn


def cosine_step_inputs(shape: CosineStepShape, **override) -> CosineStepInputs:
    """Hidden states of the current and previous denoising step plus weights.

    prev = cur + N(0, noise_std) except ``n_redrawn`` positions per batch row,
    which are redrawn N(0,1) (the salient tokens).  Weights ~ N(0, w_std)."""
    if override:
        shape = CosineStepShape(**{**shape.__dict__, **override})
    s = shape
    rng = np.random.default_rng(s.seed)
    cur = rng.standard_normal((s.B, s.S, s.D), dtype=np.float32)
    prev = cur + np.float32(s.noise_std) * rng.standard_normal((s.B, s.S, s.D), dtype=np.float32)
    redrawn = []
    for b in range(s.B):
        pos = np.sort(rng.choice(s.S, size=s.n_redrawn, replace=False))
        prev[b, pos] = rng.standard_normal((s.n_redrawn, s.D), dtype=np.float32)
        redrawn.append(pos.astype(np.int64))
    n_qkv = (s.Hq + 2 * s.Hkv) * s.hd
    w_qkv = np.float32(s.w_std) * rng.standard_normal((n_qkv, s.D), dtype=np.float32)
    w_o = None
    if s.with_wo:
        w_o = np.float32(s.w_std) * rng.standard_normal((s.D, s.Hq * s.hd), dtype=np.float32)
    st = lambda a: None if a is None else to_storage(a, s.dtype)
    return CosineStepInputs(s, st(cur), st(prev), st(w_qkv), st(w_o), redrawn)


# --------------------------------------------------------------------------
# lock loop (gqa_lock_loop)
# --------------------------------------------------------------------------
def unlocked_count(S: int, t: int, steps: int, lock_max: float) -> int:
    """Active (unlocked) positions per sequence at step t: the locked count rises
    linearly from 0 to lock_max*S over the loop, floor-rounded."""
    locked = math.floor(lock_max * t / (steps - 1) * S) if steps > 1 else 0
    return S - locked


@dataclass
class LockLoopInputs:
    shape: LockLoopShape
    w_qkv: np.ndarray        # [(Hq+2Hkv)*hd, D] bf16-exact float32
    perms: np.ndarray        # [B,S] one permutation per sequence; unlocked = first M_t entries

    def unlocked_scores(self, t: int) -> np.ndarray:
        """Given-score input for step t: 0 for unlocked positions, 1 for locked."""
        s = self.shape
        m = unlocked_count(s.S, t, s.steps, s.lock_max)
        sc = np.ones((s.B, s.S), dtype=np.float32)
        for b in range(s.B):
            sc[b, self.perms[b, :m]] = 0.0
        return sc

    def hidden(self, t: int) -> np.ndarray:
        """x_t [B,S,D], redrawn N(0,1) every step so a skipped scatter cannot pass."""
        s = self.shape
        rng = np.random.default_rng(s.seed * 1000 + t)
        return round_bf16(rng.standard_normal((s.B, s.S, s.D), dtype=np.float32))


def lock_loop_inputs(shape: LockLoopShape = GQA_LOCK_LOOP, **override) -> LockLoopInputs:
    if override:
        shape = LockLoopShape(**{**shape.__dict__, **override})
    s = shape
    rng = np.random.default_rng(s.seed)
    n_qkv = (s.Hq + 2 * s.Hkv) * s.hd
    w = round_bf16(np.float32(s.w_std) * rng.standard_normal((n_qkv, s.D), dtype=np.float32))
    perms = np.stack([rng.permutation(s.S) for _ in range(s.B)]).astype(np.int64)
    return LockLoopInputs(s, w, perms)


# --------------------------------------------------------------------------
# attention column sums (colsum_top64)
# --------------------------------------------------------------------------
@dataclass
class ColsumInputs:
    shape: ColsumShape
    q: np.ndarray          # [B, S-prompt, Hq, hd] queries of the masked region, bf16-exact
    k_cache: np.ndarray    # [B, S, Hkv, hd]
    v_cache: np.ndarray    # [B, S, Hkv, hd]

    def masked_scores(self) -> np.ndarray:
        """Given-score input: prompt positions 1, masked positions 0 (select < 0.5)."""
        s = self.shape
        sc = np.zeros((s.B, s.S), dtype=np.float32)
        sc[:, : s.prompt] = 1.0
        return sc


def colsum_inputs(shape: ColsumShape = COLSUM_TOP64, zero_q: bool = False, **override) -> ColsumInputs:
    if override:
        shape = ColsumShape(**{**shape.__dict__, **override})
    s = shape
    rng = np.random.default_rng(s.seed)
    nq = s.S - s.prompt
    q = rng.standard_normal((s.B, nq, s.Hq, s.hd), dtype=np.float32)
    k = rng.standard_normal((s.B, s.S, s.Hkv, s.hd), dtype=np.float32)
    v = rng.standard_normal((s.B, s.S, s.Hkv, s.hd), dtype=np.float32)
    if zero_q:
        q[:] = 0.0
    return ColsumInputs(s, round_bf16(q), round_bf16(k), round_bf16(v))


# --------------------------------------------------------------------------
# confidence + longest stable prefix (lsp_commit)
# --------------------------------------------------------------------------
@dataclass
class LspInputs:
    shape: LspShape
    w_lm: np.ndarray        # [V, D] out-major, bf16-exact
    frontier: np.ndarray    # [B] P_b: generated positions < P_b are planted (will stabilise)
    targets: np.ndarray     # [B, S_gen] planted token per generated position
    flip: np.ndarray        # [B, S_gen] bool: rows past P_b whose target is redrawn each step
    base_noise: np.ndarray  # [B, S, D] N(0,1) noise shared by all steps
    _unit: np.ndarray = field(repr=False, default=None)

    @property
    def S_gen(self) -> int:
        return self.shape.S - self.shape.prompt

    def n_active(self) -> int:
        return int(math.floor(self.shape.active_frac * self.S_gen))

    def active_rows(self, t: int) -> list:
        """Per batch row, the sorted absolute positions evaluated at step t: a uniform
        draw without replacement of n_active positions of the generated region."""
        s = self.shape
        rng = np.random.default_rng(s.seed * 1000 + t)
        rows = []
        for b in range(s.B):
            r = np.sort(rng.choice(self.S_gen, size=self.n_active(), replace=False)) + s.prompt
            rows.append(r.astype(np.int64))
        return rows

    def hidden(self, t: int) -> np.ndarray:
        """Hidden states at step t.  Generated rows before P_b point strongly at a
        fixed token (beta * unit(w_v) + noise); row P_b is diffuse; rows after it are
        diffuse or 'flip' rows whose planted token is redrawn every step."""
        s = self.shape
        h = self.base_noise.copy()
        rng = np.random.default_rng(s.seed * 1000 + 500 + t)
        for b in range(s.B):
            P = int(self.frontier[b])
            tok = self.targets[b].copy()
            nflip = int(self.flip[b].sum())
            tok[self.flip[b]] = rng.integers(0, s.V, size=nflip)
            planted = np.zeros(self.S_gen, dtype=bool)
            planted[:P] = True
            planted |= self.flip[b]
            rows = np.nonzero(planted)[0]
            h[b, s.prompt + rows] += np.float32(s.beta) * self._unit[tok[rows]]
        return round_bf16(h)


def lsp_inputs(shape: LspShape = LSP_COMMIT, **override) -> LspInputs:
    if override:
        shape = LspShape(**{**shape.__dict__, **override})
    s = shape
    rng = np.random.default_rng(s.seed)
    w = round_bf16(np.float32(s.w_std) * rng.standard_normal((s.V, s.D), dtype=np.float32))
    S_gen = s.S - s.prompt
    frontier = rng.integers(0, S_gen, size=s.B)
    targets = rng.integers(0, s.V, size=(s.B, S_gen))
    flip = np.zeros((s.B, S_gen), dtype=bool)
    for b in range(s.B):
        tail = np.arange(frontier[b] + 1, S_gen)
        flip[b, tail] = rng.random(tail.size) < 0.5
    base = rng.standard_normal((s.B, s.S, s.D), dtype=np.float32)
    wd = w.astype(np.float64)
    unit = (wd / np.linalg.norm(wd, axis=1, keepdims=True)).astype(np.float32)
    return LspInputs(s, w, frontier.astype(np.int64), targets.astype(np.int64), flip, base, unit)


# --------------------------------------------------------------------------
# DyLLM's adaptive input: a multi-step loop with a prompt and a response
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class DyllmLoopShape:
    name: str
    B: int
    S: int
    prompt: int             # positions [0, prompt) are the prompt, the rest the response
    D: int
    Hq: int
    Hkv: int
    hd: int
    steps: int
    refresh: int            # the whole sequence is scored every `refresh` steps
    response_redrawn: int   # response rows redrawn fresh per step (per batch row)
    prompt_redrawn: int     # prompt rows redrawn fresh per step (per batch row)
    noise_std: float        # per-step drift of every other row
    w_std: float
    tau: float
    seed: int


DYLLM_LOOP = DyllmLoopShape(
    name="bf16_dyllm_b1_s1024_p512_8steps", B=1, S=1024, prompt=512, D=4096, Hq=32, Hkv=32, hd=128,
    steps=8, refresh=4, response_redrawn=51, prompt_redrawn=4, noise_std=1e-3, w_std=1.0 / 64.0, tau=0.95,
    seed=6)


@dataclass
class DyllmLoopInputs:
    shape: DyllmLoopShape
    w_qkv: np.ndarray                       # [(Hq+2Hkv)*hd, D] bf16-exact
    _states: list = field(repr=False, default=None)
    _redrawn: list = field(repr=False, default=None)

    def hidden(self, t: int) -> np.ndarray:
        """Hidden states h_t [B,S,D] (bf16-exact) for t = -1 .. steps-1: h_{-1}
        ~ N(0,1); each later step adds N(0, noise_std) drift to every row and
        redraws `response_redrawn` response rows and `prompt_redrawn` prompt
        rows fresh (the salient tokens of that step)."""
        return self._states[t + 1]

    def redrawn(self, t: int) -> list:
        """Per batch row, the sorted positions redrawn at step t (t >= 0)."""
        return self._redrawn[t]


def dyllm_loop_inputs(shape: DyllmLoopShape = DYLLM_LOOP, **override) -> DyllmLoopInputs:
    if override:
        shape = DyllmLoopShape(**{**shape.__dict__, **override})
    s = shape
    rng = np.random.default_rng(s.seed)
    n_qkv = (s.Hq + 2 * s.Hkv) * s.hd
    w = round_bf16(np.float32(s.w_std) * rng.standard_normal((n_qkv, s.D), dtype=np.float32))
    h = rng.standard_normal((s.B, s.S, s.D), dtype=np.float32)
    states, redrawn = [round_bf16(h)], []
    for _ in range(s.steps):
        h = h + np.float32(s.noise_std) * rng.standard_normal((s.B, s.S, s.D), dtype=np.float32)
        per_b = []
        for b in range(s.B):
            pos = np.concatenate([rng.choice(s.prompt, s.prompt_redrawn, replace=False),
                                  s.prompt + rng.choice(s.S - s.prompt, s.response_redrawn, replace=False)])
            pos = np.sort(pos)
            h[b, pos] = rng.standard_normal((pos.size, s.D), dtype=np.float32)
            per_b.append(pos.astype(np.int64))
        states.append(round_bf16(h))
        redrawn.append(per_b)
    return DyllmLoopInputs(s, w, states, redrawn)


def pack_rows(rows_per_batch) -> tuple:
    """(idx int32 [n], offsets int32 [B+1]) from per-batch sorted position lists."""
    counts = [len(r) for r in rows_per_batch]
    offsets = np.zeros(len(counts) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    idx = np.concatenate([np.asarray(r, dtype=np.int32) for r in rows_per_batch]) if counts else np.zeros(0, np.int32)
    return idx.astype(np.int32), offsets
