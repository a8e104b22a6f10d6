"""CPU checks of the C ABI: libdsa.so loads, exports every function include/dsa.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed: no call below
reaches a kernel launch, the device pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from sparse_attention_sum_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.lib_path()):
        from sparse_attention_sum_amd import build
        build.build()
    return dsa.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"^(?:dsa_status|size_t|const char\*)\s+(dsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla", "dsa_forward"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(dsa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dsa_version().startswith(b"libdsa")
    assert lib.dsa_status_string(0) == b"ok"


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _batch(T=4, B=1, max_len=100, max_q=4):
    return dsa._Batch(T, B, FAKE, FAKE, FAKE, max_len, max_q)


def _cache(dim=128, dtype=dsa.DSA_FP8_E4M3, rows=1000, stride=100, pt=None, pt_stride=0, page=64):
    return dsa._Cache(FAKE, None, dtype, dim, rows, stride, pt, pt_stride, page)


def _idx(lib, head_dim=128, batch=None, cache=None, ld=128, q=FAKE, heads=64, dtype=dsa.DSA_FP8_E4M3):
    b = batch or _batch()
    c = cache or _cache()
    return lib.dsa_indexer_scores(q, dtype, None, FAKE, heads, head_dim, ctypes.byref(c), ctypes.byref(b), 1.0,
                                  FAKE, ld, None)


def test_indexer_validation(lib):
    assert _idx(lib, head_dim=64) == dsa.DSA_ERR_UNSUPPORTED
    assert b"head_dim" in lib.dsa_last_error()
    assert _idx(lib, heads=0) == dsa.DSA_ERR_UNSUPPORTED
    assert _idx(lib, heads=129) == dsa.DSA_ERR_UNSUPPORTED
    assert _idx(lib, q=None) == dsa.DSA_ERR_INVALID_ARG
    assert _idx(lib, ld=99) == dsa.DSA_ERR_INVALID_ARG
    assert _idx(lib, dtype=7) == dsa.DSA_ERR_INVALID_ARG
    assert _idx(lib, dtype=dsa.DSA_BF16) == dsa.DSA_ERR_UNSUPPORTED            # q / cache dtypes differ
    assert _idx(lib, cache=_cache(dim=576)) == dsa.DSA_ERR_UNSUPPORTED
    assert _idx(lib, cache=_cache(stride=50)) == dsa.DSA_ERR_INVALID_ARG         # seq_stride < max_len
    assert _idx(lib, cache=_cache(rows=50)) == dsa.DSA_ERR_INVALID_ARG           # B * stride > rows
    assert _idx(lib, cache=_cache(pt=FAKE, pt_stride=1)) == dsa.DSA_ERR_INVALID_ARG   # 100 tokens need 2 pages
    assert _idx(lib, cache=_cache(pt=FAKE, pt_stride=2, page=0)) == dsa.DSA_ERR_INVALID_ARG
    assert _idx(lib, batch=_batch(max_q=0)) == dsa.DSA_ERR_INVALID_ARG
    assert _idx(lib, batch=_batch(B=0)) == dsa.DSA_ERR_INVALID_ARG
    # launch-grid limits, rejected by the batch check itself (the message names the field)
    big = _cache(rows=65536 * 100)
    assert _idx(lib, batch=_batch(B=65536), cache=big) == dsa.DSA_ERR_INVALID_ARG
    assert b"num_seqs 65536 > 65535" in lib.dsa_last_error()
    assert _idx(lib, batch=_batch(B=65535), cache=big, q=None) == dsa.DSA_ERR_INVALID_ARG   # the limit itself passes
    assert b"q or weights" in lib.dsa_last_error()
    assert _idx(lib, batch=_batch(max_len=65535 * 256 + 1)) == dsa.DSA_ERR_INVALID_ARG
    assert b"max_len 16776961 > 16776960" in lib.dsa_last_error()
    bad = dsa._Batch(4, 1, None, FAKE, FAKE, 100, 4)
    assert _idx(lib, batch=bad) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_indexer_scores(FAKE, 2, None, FAKE, 64, 128, None, ctypes.byref(_batch()), 1.0, FAKE, 128,
                                  None) == dsa.DSA_ERR_INVALID_ARG


def test_topk_validation(lib):
    b = _batch()
    assert lib.dsa_topk(FAKE, 128, ctypes.byref(b), 0, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, 128, ctypes.byref(b), 70000, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, 99, ctypes.byref(b), 16, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, 128, ctypes.byref(b), 16, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk(FAKE, 128, None, 16, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG


def _mla(lib, heads=128, dqk=576, dv=512, cache=None, k=2048, ws=None, ws_bytes=0, batch=None):
    c = cache or _cache(dim=576, dtype=dsa.DSA_BF16)
    b = batch or _batch(T=4)
    return lib.dsa_sparse_mla(FAKE, heads, dqk, dv, ctypes.byref(c), ctypes.byref(b), FAKE, k, 0.04, FAKE, None,
                              ws, ws_bytes, None)


def test_sparse_mla_validation(lib):
    assert _mla(lib, dqk=512) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(lib, dv=256) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(lib, heads=0) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(lib, heads=256) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(lib, k=0) == dsa.DSA_ERR_INVALID_ARG
    assert _mla(lib, cache=_cache(dim=576, dtype=dsa.DSA_FP8_E4M3)) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(lib, cache=_cache(dim=128, dtype=dsa.DSA_BF16)) == dsa.DSA_ERR_UNSUPPORTED
    # 4 queries x 2048 slots need split partials in the workspace
    assert _mla(lib) == dsa.DSA_ERR_WORKSPACE
    assert b"workspace" in lib.dsa_last_error()
    assert _mla(lib, ws=FAKE, ws_bytes=16) == dsa.DSA_ERR_WORKSPACE


def test_forward_validation(lib):
    b = _batch(T=4, max_len=100)
    kc = _cache()
    lc = _cache(dim=576, dtype=dsa.DSA_BF16)
    # k >= max_len: no scores needed, so a bad indexer head_dim is not even looked at, but the
    # workspace is still required for the selection and the split partials
    st = lib.dsa_forward(FAKE, dsa.DSA_FP8_E4M3, None, FAKE, 64, ctypes.byref(kc), 1.0, 16, FAKE, 128,
                         ctypes.byref(lc), 0.04, ctypes.byref(b), None, FAKE, None, None, 0, None)
    assert st == dsa.DSA_ERR_WORKSPACE
    st = lib.dsa_forward(FAKE, dsa.DSA_BF16, None, FAKE, 64, ctypes.byref(kc), 1.0, 16, FAKE, 128,
                         ctypes.byref(lc), 0.04, ctypes.byref(b), None, FAKE, None, None, 0, None)
    assert st == dsa.DSA_ERR_UNSUPPORTED                     # indexer q / cache dtype mismatch


def _itk(lib, k=2048, indices=FAKE, head_dim=128, batch=None, cache=None, ws=None, ws_bytes=0):
    b = batch or _batch()
    c = cache or _cache()
    return lib.dsa_indexer_topk(FAKE, dsa.DSA_FP8_E4M3, None, FAKE, 64, head_dim, ctypes.byref(c), ctypes.byref(b),
                                1.0, k, indices, ws, ws_bytes, None)


def test_indexer_topk_validation(lib):
    assert _itk(lib, k=0) == dsa.DSA_ERR_INVALID_ARG
    assert _itk(lib, k=70000) == dsa.DSA_ERR_INVALID_ARG
    assert _itk(lib, indices=None) == dsa.DSA_ERR_INVALID_ARG
    assert _itk(lib, head_dim=64) == dsa.DSA_ERR_UNSUPPORTED
    assert _itk(lib, batch=_batch(T=0)) == dsa.DSA_OK                       # empty batch: nothing launched
    # long fp8 decode rows take the fused route, which keeps the slices' candidates in the workspace
    long_b = _batch(T=64, B=64, max_len=131072, max_q=1)
    long_c = _cache(rows=64 * 131072, stride=131072)
    need = lib.dsa_workspace_size(dsa.DSA_OP_INDEXER_TOPK, ctypes.byref(long_b), 2048, 64, 512)
    assert need > 0
    assert _itk(lib, batch=long_b, cache=long_c) == dsa.DSA_ERR_WORKSPACE
    assert b"workspace" in lib.dsa_last_error()
    assert _itk(lib, batch=long_b, cache=long_c, ws=FAKE, ws_bytes=16) == dsa.DSA_ERR_WORKSPACE
    # rows longer than k on the unfused route need the score rows in the workspace
    mid_b = _batch(T=4, B=1, max_len=5000, max_q=4)
    mid_c = _cache(rows=5000, stride=5000)
    assert _itk(lib, batch=mid_b, cache=mid_c) == dsa.DSA_ERR_WORKSPACE


def test_workspace_sizes(lib):
    # decode: 64 queries, k = 2048 -> 4 splits of 512 slots
    b = _batch(T=64, B=64, max_len=8192, max_q=1)
    mla = lib.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, ctypes.byref(b), 2048, 128, 512)
    assert mla >= 64 * 4 * 128 * (512 * 2 + 4)
    fwd = lib.dsa_workspace_size(dsa.DSA_OP_FORWARD, ctypes.byref(b), 2048, 128, 512)
    assert fwd >= mla + 64 * 8192 * 4 + 64 * 2048 * 4
    # prefill with many queries: one split, no partials
    b = _batch(T=16384, B=1, max_len=16384, max_q=16384)
    assert lib.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, ctypes.byref(b), 2048, 128, 512) == 0
    assert lib.dsa_workspace_size(dsa.DSA_OP_TOPK, ctypes.byref(b), 2048, 128, 512) == 0
    assert lib.dsa_workspace_size(dsa.DSA_OP_FORWARD, None, 2048, 128, 512) == 0
    # rows longer than 32768 keys: the top-k runs in two passes and needs room for the slices'
    # candidates, 4 slices of 32768 keys x k (key, position) pairs per row at 131072
    b = _batch(T=64, B=64, max_len=131072, max_q=1)
    tk = lib.dsa_workspace_size(dsa.DSA_OP_TOPK, ctypes.byref(b), 2048, 128, 512)
    assert tk >= 64 * 4 * 2048 * 8
    mla = lib.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, ctypes.byref(b), 2048, 128, 512)
    fwd = lib.dsa_workspace_size(dsa.DSA_OP_FORWARD, ctypes.byref(b), 2048, 128, 512)
    assert fwd >= max(tk, mla) + 64 * 131072 * 4 + 64 * 2048 * 4
    b = _batch(T=64, B=64, max_len=32768, max_q=1)
    assert lib.dsa_workspace_size(dsa.DSA_OP_TOPK, ctypes.byref(b), 2048, 128, 512) == 0
    b = _batch(T=64, B=64, max_len=65536, max_q=1)                 # two slices of 32768
    assert lib.dsa_workspace_size(dsa.DSA_OP_TOPK, ctypes.byref(b), 2048, 128, 512) >= 64 * 2 * 2048 * 8


def _append(lib, k_new=FAKE, k_dtype=dsa.DSA_F32, lat=FAKE, lat_dtype=dsa.DSA_BF16, T=4, B=2, kc=None, lc=None,
            kr=None, lr=None, seq=FAKE, pos=FAKE):
    kc = kc or dsa._Cache(FAKE, FAKE, dsa.DSA_FP8_E4M3, 128, 1000, 100, None, 0, 64)
    lc = lc or dsa._Cache(FAKE, None, dsa.DSA_BF16, 576, 1000, 100, None, 0, 64)
    return lib.dsa_cache_append(k_new, k_dtype, lat, lat_dtype, seq, pos, T, B,
                                None if kr is None else ctypes.byref(kr), None if lr is None else ctypes.byref(lr),
                                ctypes.byref(kc), ctypes.byref(lc), None)


def test_cache_append_validation(lib):
    assert _append(lib, T=-1) == dsa.DSA_ERR_INVALID_ARG
    assert _append(lib, seq=None) == dsa.DSA_ERR_INVALID_ARG
    assert _append(lib, k_dtype=dsa.DSA_FP8_E4M3) == dsa.DSA_ERR_UNSUPPORTED          # sources are f32 / bf16
    assert _append(lib, lat_dtype=7) == dsa.DSA_ERR_UNSUPPORTED
    # fp8 key cache without a scale array
    assert _append(lib, kc=dsa._Cache(FAKE, None, dsa.DSA_FP8_E4M3, 128, 1000, 100, None, 0, 64)) == dsa.DSA_ERR_INVALID_ARG
    assert _append(lib, kc=dsa._Cache(FAKE, FAKE, dsa.DSA_FP8_E4M3, 576, 1000, 100, None, 0, 64)) == dsa.DSA_ERR_UNSUPPORTED
    assert _append(lib, lc=dsa._Cache(FAKE, None, dsa.DSA_F32, 576, 1000, 100, None, 0, 64)) == dsa.DSA_ERR_UNSUPPORTED
    assert _append(lib, lc=dsa._Cache(FAKE, None, dsa.DSA_BF16, 576, 1000, 100, FAKE, 0, 64)) == dsa.DSA_ERR_INVALID_ARG
    assert _append(lib, lc=dsa._Cache(None, None, dsa.DSA_BF16, 576, 1000, 100, None, 0, 64)) == dsa.DSA_ERR_INVALID_ARG
    assert _append(lib, kr=dsa._Rope(0, 63, 1, 10000.0)) == dsa.DSA_ERR_INVALID_ARG   # odd width
    assert _append(lib, kr=dsa._Rope(100, 64, 1, 10000.0)) == dsa.DSA_ERR_INVALID_ARG  # past the row
    assert _append(lib, lr=dsa._Rope(512, 64, 1, 0.0)) == dsa.DSA_ERR_INVALID_ARG     # base <= 0
    assert _append(lib, lr=dsa._Rope(512, 64, 1, float("inf"))) == dsa.DSA_ERR_INVALID_ARG
    assert b"latent_rope" in lib.dsa_last_error()
    # nothing to write: returns before any launch
    assert _append(lib, k_new=None, lat=None, kc=dsa._Cache(), lc=dsa._Cache()) == dsa.DSA_OK


def _ropeq(lib, qi=FAKE, qi_dtype=dsa.DSA_BF16, hi=64, qo=FAKE, qo_dtype=dsa.DSA_FP8_E4M3, qs=FAKE, ri=None,
           qm=FAKE, hm=128, rm=None, pos=FAKE, T=4):
    return lib.dsa_rope_queries(qi, qi_dtype, hi, qo, qo_dtype, qs, None if ri is None else ctypes.byref(ri), qm, hm,
                                None if rm is None else ctypes.byref(rm), pos, T, None)


def test_rope_queries_validation(lib):
    assert _ropeq(lib, T=-1) == dsa.DSA_ERR_INVALID_ARG
    assert _ropeq(lib, pos=None) == dsa.DSA_ERR_INVALID_ARG
    assert _ropeq(lib, qi_dtype=dsa.DSA_FP8_E4M3) == dsa.DSA_ERR_UNSUPPORTED
    assert _ropeq(lib, qo_dtype=9) == dsa.DSA_ERR_INVALID_ARG
    assert _ropeq(lib, qs=None) == dsa.DSA_ERR_INVALID_ARG                          # fp8 needs the scales
    assert _ropeq(lib, qo=None) == dsa.DSA_ERR_INVALID_ARG
    assert _ropeq(lib, hi=0) == dsa.DSA_ERR_UNSUPPORTED
    assert _ropeq(lib, hm=129) == dsa.DSA_ERR_UNSUPPORTED
    assert _ropeq(lib, rm=dsa._Rope(520, 64, 0, 10000.0)) == dsa.DSA_ERR_INVALID_ARG  # past the 576-wide row
    assert _ropeq(lib, ri=dsa._Rope(-2, 64, 1, 10000.0)) == dsa.DSA_ERR_INVALID_ARG
    # nothing to do: no indexer queries and an MLA rotation of width 0
    assert _ropeq(lib, qi=None, rm=dsa._Rope(0, 0, 1, 10000.0)) == dsa.DSA_OK


def test_value_restore_validation(lib):
    assert lib.dsa_value_restore(FAKE, FAKE, -1, 128, 128, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_value_restore(FAKE, FAKE, 4, 0, 128, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_value_restore(FAKE, FAKE, 4, 129, 128, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_value_restore(FAKE, FAKE, 4, 128, 64, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED     # d_h % 128
    assert lib.dsa_value_restore(FAKE, FAKE, 4, 128, 640, FAKE, None) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_value_restore(None, FAKE, 4, 128, 128, FAKE, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_value_restore(FAKE + 2, FAKE, 4, 128, 128, FAKE, None) == dsa.DSA_ERR_INVALID_ARG   # alignment
    assert b"aligned" in lib.dsa_last_error()
    assert lib.dsa_value_restore(None, None, 0, 128, 128, None, None) == dsa.DSA_OK                   # nothing to do


def test_topk_select_validation(lib):
    b = _batch()
    assert lib.dsa_topk_select(FAKE, 128, ctypes.byref(b), 0, None, 0, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_select(FAKE, 128, ctypes.byref(b), 16, None, -1, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_select(FAKE, 128, ctypes.byref(b), 65000, None, 1000, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_select(FAKE, 99, ctypes.byref(b), 16, None, 0, FAKE, None, 0, None) == dsa.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_select(FAKE, 128, ctypes.byref(b), 16, None, 0, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARG


def test_forward_noalloc_rejects_a_batch_past_its_scratch(lib):
    """dsa_forward_noalloc checks the batch's workspace against its 96 MiB static scratch on the host,
    before any device call: 320 queries at 70000 positions need more (their scores alone are 85 MiB)."""
    T, L = 320, 70000
    b = dsa._Batch(T, 8, FAKE, FAKE, FAKE, L, 40)
    kc = _cache(dim=128, rows=8 * L, stride=L)
    lc = dsa._Cache(FAKE, None, dsa.DSA_BF16, 576, 8 * L, L, None, 0, 64)
    assert lib.dsa_workspace_size(dsa.DSA_OP_FORWARD, ctypes.byref(b), 2048, 128, 512) > 96 << 20
    st = lib.dsa_forward_noalloc(FAKE, dsa.DSA_FP8_E4M3, None, FAKE, 64, ctypes.byref(kc), 1.0, 2048, FAKE, 128,
                                 ctypes.byref(lc), 1 / 24, ctypes.byref(b), None, FAKE, None, None)
    assert st == dsa.DSA_ERR_WORKSPACE
    assert b"scratch" in lib.dsa_last_error()
    # argument errors come first, as in dsa_forward
    assert lib.dsa_forward_noalloc(FAKE, dsa.DSA_FP8_E4M3, None, FAKE, 64, ctypes.byref(kc), 1.0, 0, FAKE, 128,
                                   ctypes.byref(lc), 1 / 24, ctypes.byref(b), None, FAKE, None,
                                   None) == dsa.DSA_ERR_INVALID_ARG


def test_mla_prologue_wait_check_counts_the_loads():
    """build.py's check of the sparse-MLA prologue: the explicit vmcnt(18) after the index DMA is
    sound only with at least 18 vector-memory instructions issued between them."""
    from sparse_attention_sum_amd import build
    head = "<_ZN3dsa12_GLOBAL__N_117sparse_mla_kernelEv>:\n\tglobal_load_lds_dword v[2:3], off\n"
    ok = head + "\tglobal_load_dwordx4 v[4:7], v[8:9], off\n" * 18 + "\ts_waitcnt vmcnt(18)\n"
    assert build.mla_prologue_loads(ok) == 18
    short = head + "\tglobal_load_dwordx4 v[4:7], v[8:9], off\n" * 9 + "\ts_waitcnt vmcnt(18)\n"
    with pytest.raises(RuntimeError):
        build.mla_prologue_loads(short)
    co = os.path.join(ROOT, "_build", "sparse_mla.hip.co")
    if os.path.exists(co):
        assert build.check_mla_prologue_wait(co) >= 18
