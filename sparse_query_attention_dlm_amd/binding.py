"""Thin ctypes binding of libdlm (include/dlm.h).

Argument marshalling only: tensors become device pointers, shapes become ints,
the current torch stream becomes the hipStream_t.  Every computation runs in
the library's HIP kernels; there is no fallback path.  Importing this module
fails loudly if libdlm.so has not been built.

Function names match the C entry points."""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

DLM_OK, DLM_ERR_INVALID_ARG, DLM_ERR_UNSUPPORTED, DLM_ERR_WORKSPACE, DLM_ERR_HIP = range(5)
DLM_F32, DLM_BF16 = 0, 1
DLM_SCORE_COSINE, DLM_SCORE_CONFIDENCE, DLM_SCORE_GIVEN, DLM_SCORE_MARGIN = 0, 1, 2, 3


class DlmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    return ctypes.CDLL(LIB_PATH)


lib = _load()

_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
lib.dlm_status_string.restype = ctypes.c_char_p
lib.dlm_status_string.argtypes = [_I]
lib.dlm_last_error.restype = ctypes.c_char_p
lib.dlm_version.restype = ctypes.c_char_p
lib.dlm_select_workspace_size.restype = _Z
lib.dlm_select_workspace_size.argtypes = [_I, _I, _I, _I, _I]
lib.dlm_saliency_select.restype = _I
lib.dlm_saliency_select.argtypes = [_I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _F,
                                    _P, _P, _P, _P, _P, _P, _Z, _P]
lib.dlm_gather_qkv_workspace_size.restype = _Z
lib.dlm_gather_qkv_workspace_size.argtypes = [_I] * 6
lib.dlm_gather_qkv_scatter_kv.restype = _I
lib.dlm_gather_qkv_scatter_kv.argtypes = [_I, _P, _I, _I, _I, _P, _P, _I, _P, _I, _I, _I,
                                          _P, _P, _P, _P, _Z, _P]
lib.dlm_partial_attn_workspace_size.restype = _Z
lib.dlm_partial_attn_workspace_size.argtypes = [_I] * 8
lib.dlm_partial_attn.restype = _I
lib.dlm_partial_attn.argtypes = [_I, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P,
                                 _P, _I, _P, _P, _Z, _P]
lib.dlm_partial_attn_noalloc.restype = _I
lib.dlm_partial_attn_noalloc.argtypes = [_I, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P,
                                         _P, _I, _P, _P]
lib.dlm_partial_attn_noalloc_scratch_bytes.restype = _Z
lib.dlm_partial_attn_noalloc_scratch_bytes.argtypes = []
lib.dlm_attn_colsum_workspace_size.restype = _Z
lib.dlm_attn_colsum_workspace_size.argtypes = [_I, _I, _I]
lib.dlm_attn_colsum.restype = _I
lib.dlm_attn_colsum.argtypes = [_I, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _I, _I,
                                _P, _P, _P, _Z, _P]
lib.dlm_attn_colsum_window.restype = _I
lib.dlm_attn_colsum_window.argtypes = lib.dlm_attn_colsum.argtypes
lib.dlm_stable_prefix.restype = _I
lib.dlm_stable_prefix.argtypes = [_P, _P, _I, _I, _I, _I, _P, _I, _I, _F, _I, _P, _P]
lib.dlm_probe_mfma_bf16.restype = _I
lib.dlm_probe_mfma_bf16.argtypes = [_I, _I, _P, _P]
lib.dlm_nonsalient_dv_update.restype = _I
lib.dlm_nonsalient_dv_update.argtypes = [_I, _P, _P, _P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P,
                                         _P]
lib.dlm_salient_ffn_workspace_size.restype = _Z
lib.dlm_salient_ffn_workspace_size.argtypes = [_I] * 4
lib.dlm_salient_ffn.restype = _I
lib.dlm_salient_ffn.argtypes = [_I, _P, _I, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _Z, _P]
lib.dlm_lsp_adaptive_commit.restype = _I
lib.dlm_lsp_adaptive_commit.argtypes = [_P, _I, _I, _I, _I, _F, _F, _F, _P, _P, _P]
lib.dlm_kl_lock_workspace_size.restype = _Z
lib.dlm_kl_lock_workspace_size.argtypes = [_I] * 4
lib.dlm_kl_lock.restype = _I
lib.dlm_kl_lock.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _F, _F, _P, _P, _P, _P, _P, _Z, _P]
lib.dlm_gather_rows.restype = _I
lib.dlm_gather_rows.argtypes = [_P, _I, _I, _I, _P, _P, _I, _P, _P]
lib.dlm_scatter_rows.restype = _I
lib.dlm_scatter_rows.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P]


def version() -> str:
    return lib.dlm_version().decode()


def _check(rc: int) -> None:
    if rc != DLM_OK:
        raise DlmError(rc, f"{lib.dlm_status_string(rc).decode()}: {lib.dlm_last_error().decode()}")


def _ptr(t, name, dtype=None, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _dt(t) -> int:
    if t.dtype == torch.bfloat16:
        return DLM_BF16
    if t.dtype == torch.float32:
        return DLM_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, "workspace"), ws.numel() * ws.element_size()


def dlm_select_workspace_size(mode, B, S, V=0, max_eval=0) -> int:
    return int(lib.dlm_select_workspace_size(mode, B, S, V, max_eval))


def dlm_partial_attn_workspace_size(dtype, max_rows, B, S, Hq, Hkv, hd, D_out_wo=0) -> int:
    return int(lib.dlm_partial_attn_workspace_size(dtype, max_rows, B, S, Hq, Hkv, hd, D_out_wo))


def dlm_gather_qkv_workspace_size(dtype, max_rows, D, Hq, Hkv, hd) -> int:
    return int(lib.dlm_gather_qkv_workspace_size(dtype, max_rows, D, Hq, Hkv, hd))


def dlm_attn_colsum_workspace_size(B, S, Hkv) -> int:
    return int(lib.dlm_attn_colsum_workspace_size(B, S, Hkv))


def dlm_saliency_select(mode, a, b, *, lo, hi, threshold, idx, counts, offsets, workspace=None,
                        scores=None, argmax=None, eval_idx=None, eval_offsets=None, max_eval=0,
                        stream=None):
    """a, b: COSINE cur/prev [B,S,D]; CONFIDENCE and MARGIN hidden [B,S,D] /
    W_lm [V,D]; GIVEN scores f32 [B,S] (b None)."""
    if mode == DLM_SCORE_GIVEN:
        B, S = a.shape
        D = V = 0
        dtype = DLM_F32
        _ptr(a, "scores", torch.float32)
    else:
        B, S, D = a.shape
        dtype = _dt(a)
        V = b.shape[0] if mode in (DLM_SCORE_CONFIDENCE, DLM_SCORE_MARGIN) else 0
    wp, wn = _ws(workspace)
    rc = lib.dlm_saliency_select(
        mode, dtype, _ptr(a, "a"), _ptr(b, "b", required=False), B, S, D, V,
        _ptr(eval_idx, "eval_idx", torch.int32, False), _ptr(eval_offsets, "eval_offsets", torch.int32, False),
        int(max_eval), int(lo), int(hi), float(threshold),
        _ptr(scores, "scores", torch.float32, False), _ptr(argmax, "argmax", torch.int32, False),
        _ptr(idx, "idx", torch.int32), _ptr(counts, "counts", torch.int32),
        _ptr(offsets, "offsets", torch.int32), wp, wn, _stream(stream))
    _check(rc)


def dlm_gather_qkv_scatter_kv(x, idx, offsets, max_rows, w_qkv, Hq, Hkv, hd, q_out, k_cache,
                              v_cache, workspace=None, stream=None):
    B, S, D = x.shape
    wp, wn = _ws(workspace)
    rc = lib.dlm_gather_qkv_scatter_kv(
        _dt(x), _ptr(x, "x"), B, S, D, _ptr(idx, "idx", torch.int32, False),
        _ptr(offsets, "offsets", torch.int32, False), int(max_rows), _ptr(w_qkv, "w_qkv", x.dtype),
        Hq, Hkv, hd, _ptr(q_out, "q_out", x.dtype, False), _ptr(k_cache, "k_cache", x.dtype),
        _ptr(v_cache, "v_cache", x.dtype), wp, wn, _stream(stream))
    _check(rc)


def dlm_partial_attn(q_sel, idx, offsets, max_rows, k_cache, v_cache, scale, o_sel, lse=None,
                     w_o=None, out_cache=None, workspace=None, stream=None):
    B, S, Hkv, hd = k_cache.shape
    Hq = q_sel.shape[1]
    D_out = out_cache.shape[-1] if out_cache is not None else 0
    wp, wn = _ws(workspace)
    rc = lib.dlm_partial_attn(
        _dt(q_sel), _ptr(q_sel, "q_sel"), _ptr(idx, "idx", torch.int32),
        _ptr(offsets, "offsets", torch.int32), int(max_rows), _ptr(k_cache, "k_cache", q_sel.dtype),
        _ptr(v_cache, "v_cache", q_sel.dtype), B, S, Hq, Hkv, hd, float(scale),
        _ptr(o_sel, "o_sel", q_sel.dtype), _ptr(lse, "lse", torch.float32, False),
        _ptr(w_o, "w_o", q_sel.dtype, False), D_out, _ptr(out_cache, "out_cache", q_sel.dtype, False),
        wp, wn, _stream(stream))
    _check(rc)


def dlm_partial_attn_noalloc(q_sel, idx, offsets, max_rows, k_cache, v_cache, scale, o_sel, lse=None,
                             w_o=None, out_cache=None, stream=None):
    """dlm_partial_attn without a workspace: split-KV partials in the library's
    fixed per-GPU scratch (calls overlapping on one GPU race)."""
    B, S, Hkv, hd = k_cache.shape
    Hq = q_sel.shape[1]
    D_out = out_cache.shape[-1] if out_cache is not None else 0
    rc = lib.dlm_partial_attn_noalloc(
        _dt(q_sel), _ptr(q_sel, "q_sel"), _ptr(idx, "idx", torch.int32),
        _ptr(offsets, "offsets", torch.int32), int(max_rows), _ptr(k_cache, "k_cache", q_sel.dtype),
        _ptr(v_cache, "v_cache", q_sel.dtype), B, S, Hq, Hkv, hd, float(scale),
        _ptr(o_sel, "o_sel", q_sel.dtype), _ptr(lse, "lse", torch.float32, False),
        _ptr(w_o, "w_o", q_sel.dtype, False), D_out, _ptr(out_cache, "out_cache", q_sel.dtype, False),
        _stream(stream))
    _check(rc)


def dlm_partial_attn_noalloc_scratch_bytes() -> int:
    return int(lib.dlm_partial_attn_noalloc_scratch_bytes())


def dlm_attn_colsum(q_sel, offsets, max_rows, k_cache, lse, scale, colsum, key_lo=0, key_hi=None,
                    k=0, topk_idx=None, topk_val=None, workspace=None, stream=None, window_only=False):
    """window_only: dlm_attn_colsum_window (sums of the window's key blocks only)."""
    B, S, Hkv, hd = k_cache.shape
    Hq = q_sel.shape[1]
    key_hi = S if key_hi is None else key_hi
    wp, wn = _ws(workspace)
    fn = lib.dlm_attn_colsum_window if window_only else lib.dlm_attn_colsum
    rc = fn(
        _dt(q_sel), _ptr(q_sel, "q_sel"), _ptr(offsets, "offsets", torch.int32), int(max_rows),
        _ptr(k_cache, "k_cache", q_sel.dtype), _ptr(lse, "lse", torch.float32), B, S, Hq, Hkv, hd,
        float(scale), _ptr(colsum, "colsum", torch.float32), int(key_lo), int(key_hi), int(k),
        _ptr(topk_idx, "topk_idx", torch.int32, False), _ptr(topk_val, "topk_val", torch.float32, False),
        wp, wn, _stream(stream))
    _check(rc)


def dlm_stable_prefix(argmax, maxprob, gen_lo, gen_hi, ring, step, conf_threshold, committed,
                      min_commit=0, stream=None):
    B, S = argmax.shape
    W = ring.shape[-1]
    rc = lib.dlm_stable_prefix(
        _ptr(argmax, "argmax", torch.int32), _ptr(maxprob, "maxprob", torch.float32), B, S,
        int(gen_lo), int(gen_hi), _ptr(ring, "ring", torch.int32), W, int(step),
        float(conf_threshold), int(min_commit), _ptr(committed, "committed", torch.int32),
        _stream(stream))
    _check(rc)


def dlm_nonsalient_dv_update(q_cache, lse_cache, idx, offsets, max_rows, k_old, v_old, v_cache, scale,
                             o_cache, stream=None):
    B, S, Hq, hd = q_cache.shape
    Hkv = v_cache.shape[2]
    dt = q_cache.dtype
    rc = lib.dlm_nonsalient_dv_update(
        _dt(q_cache), _ptr(q_cache, "q_cache"), _ptr(lse_cache, "lse_cache", torch.float32),
        _ptr(idx, "idx", torch.int32, False), _ptr(offsets, "offsets", torch.int32, False), int(max_rows),
        _ptr(k_old, "k_old", dt, False), _ptr(v_old, "v_old", dt, False), _ptr(v_cache, "v_cache", dt),
        B, S, Hq, Hkv, hd, float(scale), _ptr(o_cache, "o_cache", dt), _stream(stream))
    _check(rc)


def dlm_salient_ffn_workspace_size(dtype, max_rows, D, F) -> int:
    return int(lib.dlm_salient_ffn_workspace_size(int(dtype), int(max_rows), int(D), int(F)))


def dlm_salient_ffn(x, idx, offsets, max_rows, w_gu, w_down, out_cache, workspace=None, stream=None):
    B, S, D = x.shape
    F = w_down.shape[1]
    wp, wn = _ws(workspace)
    rc = lib.dlm_salient_ffn(
        _dt(x), _ptr(x, "x"), B, S, D, _ptr(idx, "idx", torch.int32, False),
        _ptr(offsets, "offsets", torch.int32, False), int(max_rows), _ptr(w_gu, "w_gu", x.dtype), F,
        _ptr(w_down, "w_down", x.dtype), _ptr(out_cache, "out_cache", x.dtype), wp, wn, _stream(stream))
    _check(rc)


def dlm_lsp_adaptive_commit(margin, gen_lo, gen_hi, committed, frac_lo=0.25, frac_hi=0.5, tau=None,
                            margin_floor=float("-inf"), stream=None):
    B, S = margin.shape
    rc = lib.dlm_lsp_adaptive_commit(
        _ptr(margin, "margin", torch.float32), B, S, int(gen_lo), int(gen_hi), float(frac_lo), float(frac_hi),
        float(margin_floor), _ptr(committed, "committed", torch.int32), _ptr(tau, "tau", torch.float32, False),
        _stream(stream))
    _check(rc)


def dlm_kl_lock_workspace_size(B, S, V, max_eval) -> int:
    return int(lib.dlm_kl_lock_workspace_size(int(B), int(S), int(V), int(max_eval)))


def dlm_kl_lock(h_cur, h_prev, w_lm, eval_idx, eval_offsets, max_eval, eps, kl, maxprob, argmax, locked,
                gate_q=0.0, workspace=None, stream=None):
    """h_cur, h_prev [B,S,D] bf16; w_lm [V,D] bf16; kl, maxprob, locked f32 [B,S]; argmax i32 [B,S]."""
    B, S, D = h_cur.shape
    V = w_lm.shape[0]
    wp, wn = _ws(workspace)
    rc = lib.dlm_kl_lock(
        _ptr(h_cur, "h_cur", torch.bfloat16), _ptr(h_prev, "h_prev", torch.bfloat16), _ptr(w_lm, "w_lm", torch.bfloat16),
        B, S, D, V, _ptr(eval_idx, "eval_idx", torch.int32, False), _ptr(eval_offsets, "eval_offsets", torch.int32, False),
        int(max_eval), float(eps), float(gate_q), _ptr(kl, "kl", torch.float32), _ptr(maxprob, "maxprob", torch.float32),
        _ptr(argmax, "argmax", torch.int32), _ptr(locked, "locked", torch.float32), wp, wn, _stream(stream))
    _check(rc)


def dlm_gather_rows(cache, idx, offsets, max_rows, rows, stream=None):
    """rows[r] = cache[b, idx[r]] for cache [B, S, ...] and rows [max_rows, ...]."""
    B, S = cache.shape[0], cache.shape[1]
    row_bytes = cache[0, 0].numel() * cache.element_size()
    rc = lib.dlm_gather_rows(_ptr(cache, "cache"), B, S, row_bytes, _ptr(idx, "idx", torch.int32, False),
                             _ptr(offsets, "offsets", torch.int32, False), int(max_rows),
                             _ptr(rows, "rows", cache.dtype, False), _stream(stream))
    _check(rc)


def dlm_scatter_rows(rows, idx, offsets, max_rows, cache, stream=None):
    """cache[b, idx[r]] = rows[r] for cache [B, S, ...] and rows [max_rows, ...]."""
    B, S = cache.shape[0], cache.shape[1]
    row_bytes = cache[0, 0].numel() * cache.element_size()
    rc = lib.dlm_scatter_rows(_ptr(rows, "rows", cache.dtype, False), _ptr(idx, "idx", torch.int32, False),
                              _ptr(offsets, "offsets", torch.int32, False), int(max_rows), B, S, row_bytes,
                              _ptr(cache, "cache"), _stream(stream))
    _check(rc)


def dlm_probe_mfma_bf16(iters, grid, sink, stream=None):
    """Measurement aid: grid*4 waves each run iters x 8 bf16 32x32x16 MFMAs
    on registers (grid*4*iters*8*32768 flop); sink f32 [grid*256]."""
    assert sink.numel() >= grid * 256, "sink needs grid*256 floats"
    _check(lib.dlm_probe_mfma_bf16(int(iters), int(grid), _ptr(sink, "sink", torch.float32), _stream(stream)))
