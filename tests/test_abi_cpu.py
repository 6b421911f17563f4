"""CPU-side checks of the C-ABI library: it loads without a GPU, exports every
entry point declared in include/dlm.h, and rejects invalid requests on the host
(before any launch) with the documented status codes.  No compute call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlm.h")
LIB = os.path.join(ROOT, "sparse_query_attention_dlm_amd", "libdlm.so")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
COSINE, CONFIDENCE, GIVEN = 0, 1, 2
FAKE = 0x10000          # a 16-byte aligned non-null pointer value; never dereferenced here
MISALIGNED = 0x10008

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdlm.so not built")


@pytest.fixture(scope="module")
def lib():
    L = ctypes.CDLL(LIB)
    L.dlm_last_error.restype = ctypes.c_char_p
    L.dlm_status_string.restype = ctypes.c_char_p
    L.dlm_select_workspace_size.restype = ctypes.c_size_t
    L.dlm_partial_attn_workspace_size.restype = ctypes.c_size_t
    L.dlm_attn_colsum_workspace_size.restype = ctypes.c_size_t
    return L


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dlm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for fn in ["dlm_saliency_select", "dlm_gather_qkv_scatter_kv", "dlm_partial_attn",
               "dlm_attn_colsum", "dlm_stable_prefix"]:
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.dlm_status_string(OK) == b"DLM_OK"
    assert lib.dlm_status_string(INVALID) == b"DLM_ERR_INVALID_ARG"
    assert lib.dlm_status_string(WORKSPACE) == b"DLM_ERR_WORKSPACE"
    assert lib.dlm_status_string(99) == b"DLM_ERR_UNKNOWN"


def p(v):
    return ctypes.c_void_p(v)


def f(v):
    return ctypes.c_float(v)


def select(lib, mode=COSINE, dtype=BF16, a=FAKE, b=FAKE, B=1, S=16, D=64, V=0, ev=0, evo=0,
           max_eval=0, lo=0, hi=16, scores=0, argmax=0, idx=FAKE, counts=FAKE, offsets=FAKE,
           ws=FAKE, ws_bytes=1 << 20):
    return lib.dlm_saliency_select(mode, dtype, p(a), p(b), B, S, D, V, p(ev), p(evo), max_eval, lo, hi,
                                   f(0.5), p(scores), p(argmax), p(idx), p(counts), p(offsets), p(ws),
                                   ctypes.c_size_t(ws_bytes), p(0))


def test_select_rejections(lib):
    assert select(lib, mode=7) == INVALID
    assert select(lib, dtype=5) == INVALID
    assert select(lib, B=0) == INVALID
    assert select(lib, lo=5, hi=4) == INVALID
    assert select(lib, hi=17) == INVALID
    assert select(lib, idx=0) == INVALID
    assert b"idx" in lib.dlm_last_error()
    assert select(lib, a=0) == INVALID
    assert select(lib, b=0) == INVALID
    assert select(lib, a=MISALIGNED) == INVALID
    assert select(lib, D=12) == INVALID                      # bf16 rows must be 16-byte chunks
    assert select(lib, ws=0) == WORKSPACE
    assert select(lib, ws_bytes=8) == WORKSPACE
    assert select(lib, mode=CONFIDENCE, dtype=F32, V=256, ev=FAKE, evo=FAKE, scores=FAKE, argmax=FAKE) == INVALID
    assert select(lib, mode=CONFIDENCE, V=128, ev=FAKE, evo=FAKE, scores=FAKE, argmax=FAKE, max_eval=4) == INVALID
    assert select(lib, mode=CONFIDENCE, V=256, ev=FAKE, evo=FAKE, scores=0, argmax=FAKE) == INVALID
    assert select(lib, mode=CONFIDENCE, V=256, ev=0, evo=FAKE, scores=FAKE, argmax=FAKE) == INVALID


def test_select_workspace_size_covers_partials(lib):
    small = lib.dlm_select_workspace_size(COSINE, 2, 100, 0, 0)
    assert small >= 2 * 100 * 4
    big = lib.dlm_select_workspace_size(CONFIDENCE, 2, 100, 32768, 50)
    assert big >= small + 50 * (32768 // 256) * 16
    # the LM head's split-K partials are sized by the bound: 50 rows x 32768
    # = 128 output tiles may split 8 ways (1024 tiles); 20 rows of a 2048-word
    # vocabulary = 8 tiles, at most 64 partial tiles
    assert big >= 1024 * 256 * 256 * 4
    tiny = lib.dlm_select_workspace_size(CONFIDENCE, 2, 100, 2048, 20)
    assert 64 * 256 * 256 * 4 <= tiny < 65 * 256 * 256 * 4


def gqkv(lib, dtype=BF16, x=FAKE, B=1, S=8, D=64, idx=FAKE, off=FAKE, max_rows=8, w=FAKE, Hq=2, Hkv=1,
         hd=64, q=FAKE, k=FAKE, v=FAKE):
    return lib.dlm_gather_qkv_scatter_kv(dtype, p(x), B, S, D, p(idx), p(off), max_rows, p(w), Hq, Hkv,
                                         hd, p(q), p(k), p(v), p(FAKE), ctypes.c_size_t(1 << 30), p(0))


def test_gather_qkv_rejections(lib):
    assert gqkv(lib, x=0) == INVALID
    assert gqkv(lib, w=0) == INVALID
    assert gqkv(lib, Hq=3, Hkv=2) == INVALID                 # Hq % Hkv != 0
    assert gqkv(lib, hd=96) == INVALID                       # unsupported head dim
    assert gqkv(lib, D=96) == INVALID                        # bf16 needs D % 64 == 0
    assert gqkv(lib, max_rows=9) == INVALID                  # more rows than B*S
    assert gqkv(lib, max_rows=-1) == INVALID
    assert gqkv(lib, k=MISALIGNED) == INVALID
    lib.dlm_gather_qkv_workspace_size.restype = ctypes.c_size_t
    # 256 features, bounds up to 1024 rows: no tiling splits K, no scratch
    assert lib.dlm_gather_qkv_workspace_size(BF16, 1024, 64, 2, 1, 64) == 0
    assert lib.dlm_gather_qkv_workspace_size(BF16, 1024, 4096, 32, 32, 128) == 0
    # K = 64 is too short for the 4-deep ring of the large tiling: the
    # 128 x 128 tiling runs, unsplit, at any bound
    assert lib.dlm_gather_qkv_workspace_size(BF16, 2048, 64, 2, 1, 64) == 0
    # a looser bound may split the large tiling on the device: room for up to
    # 8 fp32 256 x 256 partial tiles per output tile of the bound (2048 rows x
    # 256 features = 8 tiles), never more than 1024 tiles
    need = lib.dlm_gather_qkv_workspace_size(BF16, 2048, 256, 2, 1, 64)
    assert need == 8 * 8 * 256 * 256 * 4
    assert lib.dlm_gather_qkv_workspace_size(BF16, 16384, 4096, 32, 8, 128) == 1024 * 256 * 256 * 4
    assert lib.dlm_gather_qkv_scatter_kv(BF16, p(FAKE), 1, 2048, 256, p(FAKE), p(FAKE), 2048, p(FAKE), 2,
                                         1, 64, p(FAKE), p(FAKE), p(FAKE), p(FAKE),
                                         ctypes.c_size_t(need - 1), p(0)) == WORKSPACE
    assert lib.dlm_gather_qkv_scatter_kv(BF16, p(FAKE), 1, 2048, 256, p(FAKE), p(FAKE), 2048, p(FAKE), 2,
                                         1, 64, p(FAKE), p(FAKE), p(FAKE), p(0), ctypes.c_size_t(0),
                                         p(0)) == WORKSPACE


def attn(lib, dtype=BF16, q=FAKE, idx=FAKE, off=FAKE, max_rows=4, k=FAKE, v=FAKE, B=1, S=64, Hq=2,
         Hkv=1, hd=128, scale=0.1, o=FAKE, lse=0, wo=0, D_out=0, out=0, ws=0, ws_bytes=0):
    return lib.dlm_partial_attn(dtype, p(q), p(idx), p(off), max_rows, p(k), p(v), B, S, Hq, Hkv, hd,
                                f(scale), p(o), p(lse), p(wo), D_out, p(out), p(ws),
                                ctypes.c_size_t(ws_bytes), p(0))


def test_partial_attn_rejections(lib):
    assert attn(lib, q=0) == INVALID
    assert attn(lib, o=0) == INVALID
    assert attn(lib, hd=32) == INVALID
    assert attn(lib, Hq=3, Hkv=2) == INVALID
    assert attn(lib, scale=0.0) == INVALID
    assert attn(lib, wo=FAKE, out=0, D_out=64) == INVALID    # W_o without an output cache
    assert attn(lib, out=FAKE, D_out=100) == INVALID         # no W_o: D_out must be Hq*hd
    assert attn(lib, wo=FAKE, out=FAKE, D_out=100) == INVALID  # bf16 W_o: D_out % 64
    # bf16 addresses one sequence's K/V slice with 32-bit offsets: under 2 GiB
    assert attn(lib, S=(1 << 20) - 64, Hq=8, Hkv=8) == INVALID
    # a short selection needs split-KV scratch: refused without it
    need = lib.dlm_partial_attn_workspace_size(BF16, 4, 1, 4096, 2, 1, 128, 0)
    assert need > 0
    assert attn(lib, S=4096) == WORKSPACE
    assert attn(lib, S=4096, ws=FAKE, ws_bytes=need - 1) == WORKSPACE


def colsum(lib, dtype=BF16, q=FAKE, off=FAKE, max_rows=4, k=FAKE, lse=FAKE, B=1, S=64, Hq=2, Hkv=1,
           hd=128, cs=FAKE, lo=0, hi=64, kk=4, ti=FAKE, tv=0, ws=FAKE, ws_bytes=1 << 20, window=False):
    fn = lib.dlm_attn_colsum_window if window else lib.dlm_attn_colsum
    return fn(dtype, p(q), p(off), max_rows, p(k), p(lse), B, S, Hq, Hkv, hd, f(0.1),
              p(cs), lo, hi, kk, p(ti), p(tv), p(ws), ctypes.c_size_t(ws_bytes), p(0))


@pytest.mark.parametrize("window", [False, True])
def test_colsum_rejections(lib, window):
    assert colsum(lib, dtype=F32, window=window) == UNSUPPORTED
    assert colsum(lib, lse=0, window=window) == INVALID
    assert colsum(lib, lo=10, hi=5, window=window) == INVALID
    assert colsum(lib, kk=65, window=window) == INVALID                     # k larger than the key window
    assert colsum(lib, S=10000, hi=10000, window=window) == INVALID         # top-k window over 8192 keys
    assert colsum(lib, ti=0, tv=0, window=window) == INVALID                # k > 0 but nowhere to write
    assert colsum(lib, ws_bytes=4, window=window) == WORKSPACE
    assert colsum(lib, ws=0, window=window) == WORKSPACE
    # per-key float partials for up to 4 query splits of each KV head
    assert lib.dlm_attn_colsum_workspace_size(4, 4096, 32) == 4 * 32 * 4 * 4096 * 4


def test_colsum_window_empty_enqueues_nothing(lib):
    """An empty key window with k = 0 returns DLM_OK at once: no launch is made
    (without a GPU any launch would fail with DLM_ERR_HIP)."""
    for at in (0, 37, 256):
        assert colsum(lib, S=512, lo=at, hi=at, kk=0, window=True) == OK, lib.dlm_last_error()


def test_partial_attn_noalloc_rejections(lib):
    """The allocation-free attention validates like dlm_partial_attn and
    refuses, before any launch, a bf16 W_o projection whose loose row bound
    (above 1024) would need split-K partials it has no scratch for."""
    L = lib
    L.dlm_partial_attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    assert L.dlm_partial_attn_noalloc_scratch_bytes() == 2 * 512 * 128 * 129 * 4

    def call(dtype=BF16, q=FAKE, max_rows=4, B=1, S=64, Hq=2, Hkv=1, hd=128, o=FAKE, wo=0, D_out=0, out=0):
        return L.dlm_partial_attn_noalloc(dtype, p(q), p(FAKE), p(FAKE), max_rows, p(FAKE), p(FAKE), B, S, Hq,
                                          Hkv, hd, f(0.1), p(o), p(0), p(wo), D_out, p(out), p(0))
    assert call(hd=96) == INVALID
    assert call(q=0) == INVALID
    assert call(q=MISALIGNED) == INVALID
    assert call(Hq=3, Hkv=2) == INVALID
    assert call(max_rows=0) == OK                       # nothing to do, nothing launched
    assert call(max_rows=2048, B=1, S=4096, wo=FAKE, D_out=256, out=FAKE) == WORKSPACE
    assert b"1024" in L.dlm_last_error()


def test_probe_rejections(lib):
    assert lib.dlm_probe_mfma_bf16(0, 1, p(FAKE), p(0)) == INVALID
    assert lib.dlm_probe_mfma_bf16(1, 0, p(FAKE), p(0)) == INVALID
    assert lib.dlm_probe_mfma_bf16(1, 1, p(0), p(0)) == INVALID


def test_stable_prefix_rejections(lib):
    def sp(argmax=FAKE, mp=FAKE, B=2, S=32, lo=8, hi=32, ring=FAKE, W=3, step=0, com=FAKE):
        return lib.dlm_stable_prefix(p(argmax), p(mp), B, S, lo, hi, p(ring), W, step, f(0.9), 0, p(com), p(0))
    assert sp(argmax=0) == INVALID
    assert sp(ring=0) == INVALID
    assert sp(lo=8, hi=8) == INVALID
    assert sp(hi=33) == INVALID
    assert sp(W=0) == INVALID
    assert sp(step=-1) == INVALID


def test_dv_update_rejections(lib):
    def dv(dtype=BF16, q=FAKE, lse=FAKE, idx=FAKE, off=FAKE, max_rows=4, ko=FAKE, vo=FAKE, v=FAKE, B=1,
           S=64, Hq=4, Hkv=2, hd=128, scale=0.1, o=FAKE):
        return lib.dlm_nonsalient_dv_update(dtype, p(q), p(lse), p(idx), p(off), max_rows, p(ko), p(vo), p(v),
                                            B, S, Hq, Hkv, hd, f(scale), p(o), p(0))
    assert dv(dtype=7) == INVALID
    assert dv(q=0) == INVALID
    assert dv(lse=0) == INVALID
    assert dv(ko=0) == INVALID
    assert dv(o=MISALIGNED) == INVALID
    assert dv(hd=96) == INVALID
    assert dv(Hq=6, Hkv=4) == INVALID                        # Hq not a multiple of Hkv
    assert dv(Hq=3, Hkv=1) == INVALID                        # G = 3 must divide 128
    assert dv(max_rows=65) == INVALID                        # more rows than B*S
    assert dv(scale=0.0) == INVALID
    # no salient rows: nothing to do, and the row arrays may be NULL
    assert dv(max_rows=0, idx=0, off=0, ko=0, vo=0) == OK


def test_row_copy_rejections(lib):
    def g(cache=FAKE, B=2, S=8, rb=64, idx=FAKE, off=FAKE, max_rows=3, rows=FAKE):
        return lib.dlm_gather_rows(p(cache), B, S, rb, p(idx), p(off), max_rows, p(rows), p(0))

    def s(rows=FAKE, idx=FAKE, off=FAKE, max_rows=3, B=2, S=8, rb=64, cache=FAKE):
        return lib.dlm_scatter_rows(p(rows), p(idx), p(off), max_rows, B, S, rb, p(cache), p(0))
    for fn in (g, s):
        assert fn(rb=6) == INVALID                           # not a multiple of 4 bytes
        assert fn(rb=0) == INVALID
        assert fn(idx=0) == INVALID
        assert fn(max_rows=17) == INVALID                    # more rows than B*S
        assert fn(max_rows=0, idx=0, off=0) == OK
    assert g(rows=MISALIGNED) == INVALID                     # 16-byte rows need 16-byte alignment


def test_salient_ffn_rejections(lib):
    lib.dlm_salient_ffn_workspace_size.restype = ctypes.c_size_t

    def ffn(dtype=BF16, x=FAKE, B=1, S=64, D=128, idx=FAKE, off=FAKE, max_rows=8, wgu=FAKE, F=256, wd=FAKE,
            out=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return lib.dlm_salient_ffn(dtype, p(x), B, S, D, p(idx), p(off), max_rows, p(wgu), F, p(wd), p(out), p(ws),
                                   ctypes.c_size_t(ws_bytes), p(0))
    assert ffn(dtype=F32) == UNSUPPORTED
    assert ffn(x=0) == INVALID
    assert ffn(wgu=0) == INVALID
    assert ffn(out=MISALIGNED) == INVALID
    assert ffn(D=100) == INVALID                             # D and F multiples of 64
    assert ffn(F=100) == INVALID
    assert ffn(max_rows=65) == INVALID
    assert ffn(ws_bytes=16) == WORKSPACE
    assert ffn(ws=0) == WORKSPACE
    assert ffn(max_rows=0, idx=0, off=0, ws=0) == OK
    # h [max_rows, F] bf16 first, 256-byte aligned
    assert lib.dlm_salient_ffn_workspace_size(BF16, 8, 128, 256) == 8 * 256 * 2
    assert lib.dlm_salient_ffn_workspace_size(F32, 8, 128, 256) == 0
    # a short selection (<= 128 rows) splits the down projection's K when it has
    # fewer than 128 output tiles of 64 features: D = 4096 -> 64 tiles, F = 12288
    # -> 192 k-steps of 64 in rings of 4; splits double (2, 4) while the items
    # (tiles x splits) stay below 256, each split a 64 x 128 fp32 tile
    ws = lib.dlm_salient_ffn_workspace_size
    assert ws(BF16, 102, 4096, 12288) == 102 * 12288 * 2 + 64 * 4 * 64 * 128 * 4
    # D = 1024: 16 tiles; F = 1024 has 16 k-steps, so a split of 4 would leave
    # one ring per split (two are needed): 2 splits
    assert ws(BF16, 100, 1024, 1024) == 100 * 1024 * 2 + 16 * 2 * 64 * 128 * 4
    # no split: more than 128 rows, 128 tiles or more, or K too short to split
    assert ws(BF16, 129, 4096, 12288) == 129 * 12288 * 2
    assert ws(BF16, 64, 8192, 4096) == 64 * 4096 * 2
    assert ws(BF16, 8, 128, 256) == 8 * 256 * 2


def test_margin_mode_and_adaptive_commit_rejections(lib):
    MARGIN = 3
    assert select(lib, mode=MARGIN, dtype=F32, V=256, ev=FAKE, evo=FAKE, scores=FAKE, argmax=FAKE) == INVALID
    assert select(lib, mode=MARGIN, V=128, ev=FAKE, evo=FAKE, scores=FAKE, argmax=FAKE, max_eval=4) == INVALID
    assert select(lib, mode=MARGIN, V=256, ev=FAKE, evo=FAKE, scores=0, argmax=FAKE) == INVALID
    # the margin mode needs the same LM-head partials as the confidence mode
    assert lib.dlm_select_workspace_size(MARGIN, 2, 64, 32768, 16) == lib.dlm_select_workspace_size(CONFIDENCE, 2, 64, 32768, 16)

    def lsp(m=FAKE, B=2, S=32, lo=8, hi=32, fl=0.25, fh=0.5, com=FAKE, tau=0, floor=float("-inf")):
        return lib.dlm_lsp_adaptive_commit(p(m), B, S, lo, hi, f(fl), f(fh), f(floor), p(com), p(tau), p(0))
    assert lsp(floor=float("nan")) == INVALID
    assert lsp(m=0) == INVALID
    assert lsp(com=0) == INVALID
    assert lsp(lo=8, hi=8) == INVALID
    assert lsp(hi=33) == INVALID
    assert lsp(fl=0.0) == INVALID
    assert lsp(fl=0.6, fh=0.5) == INVALID
    assert lsp(fh=1.5) == INVALID
