"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sia.h, and host-side validation rejects bad arguments
before anything is launched."""
import ctypes
import os
import re

import pytest

from sparse_index_attention_amd import sia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sia.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sia_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sia.library_path()):
        pytest.skip("libsia.so not built")
    return sia.lib()


@pytest.fixture(scope="module")
def Lcpu(L):
    # These tests hand fake device addresses to calls that must fail host-side
    # validation.  Keep them off GPU machines, where a validation gap would
    # launch a kernel on a fake address.
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run on CPU-only machines")
    return L


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for f in ("sia_index_scores", "sia_topk", "sia_index_topk", "sia_sparse_mla_decode", "sia_sparse_mla_prefill",
              "sia_index_select_attend", "sia_workspace_size", "sia_status_string"):
        assert f in fns


def test_library_exports_every_declared_symbol(L):
    for f in declared_functions():
        assert hasattr(L, f), f


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4):
        assert L.sia_status_string(code)
    assert L.sia_status_string(123) == b"unknown status"


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced on failure paths


def good_seq(**kw):
    d = dict(q_seq=FAKE, q_pos=FAKE, block_table=FAKE, num_tokens=4, batch=1, max_pages=4, page_size=64,
             num_pages=4, max_visible=256)
    d.update(kw)
    return sia.SeqMapC(**d)


def good_indexer(**kw):
    d = dict(q=FAKE, q_scale=FAKE, w=FAKE, k_pool=FAKE, k_scale=FAKE, dtype=sia.SIA_FP8_E4M3,
             q_scale_per_head=0, heads=64, dim=128, q_bf16=0)
    d.update(kw)
    return sia.IndexerC(**d)


def call_scores(L, ix, seq, scores=FAKE, ld=256):
    return L.sia_index_scores(ctypes.byref(ix), ctypes.byref(seq), ctypes.c_void_p(scores), ld, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=32), -2),
    (dict(batch=0), -1),
    (dict(max_visible=257), -1),          # beyond max_pages * page_size
    (dict(q_pos=0), -1),
    (dict(num_tokens=-1), -1),
])
def test_seqmap_validation(Lcpu, kw, code):
    L = Lcpu
    assert call_scores(L, good_indexer(), good_seq(**kw)) == code


@pytest.mark.parametrize("kw,code", [
    (dict(heads=48), -2),
    (dict(dim=64), -2),
    (dict(q_scale=0), -1),
    (dict(dtype=7), -2),
    (dict(q=FAKE + 4), -1),               # misaligned fp8 operand
    (dict(dtype=sia.SIA_F32, heads=65, dim=4), -2),
    (dict(dtype=sia.SIA_MXFP8_E4M3, q_scale=FAKE + 2), -1),   # E8M0 scales need 4-byte alignment
    (dict(dtype=sia.SIA_MXFP8_E4M3, k_scale=FAKE + 1), -1),
    (dict(dtype=sia.SIA_MXFP8_E4M3, heads=16), -2),
])
def test_indexer_validation(Lcpu, kw, code):
    L = Lcpu
    assert call_scores(L, good_indexer(**kw), good_seq()) == code


def test_bf16_query_validation(Lcpu):
    L = Lcpu
    # the score entry point takes quantized queries only
    assert call_scores(L, good_indexer(q_bf16=1), good_seq()) == -2
    assert call_scores(L, good_indexer(q_bf16=2), good_seq()) == -1
    assert call_scores(L, good_indexer(q_bf16=1, dtype=sia.SIA_F32, heads=4, dim=32), good_seq()) == -2
    qz = lambda ix, codes=FAKE, scales=FAKE, T=4: L.sia_quantize_indexer_q(
        ctypes.byref(ix), T, ctypes.c_void_p(codes) if codes else None, ctypes.c_void_p(scales) if scales else None,
        None)
    assert qz(good_indexer(q_bf16=0)) == -1
    assert qz(good_indexer(q_bf16=1), codes=0) == -1
    assert qz(good_indexer(q_bf16=1), codes=FAKE + 8) == -1
    assert qz(good_indexer(q_bf16=1), T=-1) == -1
    assert qz(good_indexer(q_bf16=1, heads=48)) == -2
    assert qz(good_indexer(q_bf16=1, dtype=sia.SIA_MXFP8_E4M3), scales=FAKE + 1) == -1


def test_scores_buffer_validation(Lcpu):
    L = Lcpu
    assert call_scores(L, good_indexer(), good_seq(), scores=0) == -1
    assert call_scores(L, good_indexer(), good_seq(), scores=FAKE + 4) == -1
    assert call_scores(L, good_indexer(), good_seq(), ld=255) == -1
    assert call_scores(L, good_indexer(), good_seq(), ld=252) == -1   # < max_visible


def test_topk_validation(Lcpu):
    L = Lcpu
    seq = good_seq()
    f = lambda K, order=0, idx=FAKE: L.sia_topk(ctypes.c_void_p(FAKE), 256, ctypes.byref(seq), K, order,
                                               ctypes.c_void_p(idx), None, None)
    assert f(0) == -1
    assert f(2049) == -2
    assert f(16, order=2) == -1
    assert f(16, idx=0) == -1


def test_index_topk_validation(Lcpu):
    L = Lcpu
    seq = good_seq()
    need = L.sia_workspace_size(sia.OP_INDEX_TOPK, ctypes.byref(seq), 16, 1, 1)
    assert need > 0

    def f(K=16, order=0, idx=FAKE, ws=FAKE, ws_bytes=need, ix=None, method=0):
        return L.sia_index_topk(ctypes.byref(ix or good_indexer()), ctypes.byref(seq), K, order, method,
                                ctypes.c_void_p(idx), None, ctypes.c_void_p(ws) if ws else None, ws_bytes, None)
    assert f(K=0) == -1
    assert f(K=2049) == -2
    assert f(order=2) == -1                                        # pages: K must be a multiple of 64
    assert f(order=3) == -1
    assert f(idx=0) == -1
    assert f(ws=0) == -3
    assert f(ws_bytes=need - 1) == -3
    assert f(ws=FAKE + 16) == -3                                   # not 256-byte aligned
    assert f(ix=good_indexer(heads=48)) == -2
    assert f(method=3) == -1
    assert f(method=-1) == -1
    assert f(method=sia.INDEX_TOPK_ONCHIP, ix=good_indexer(dtype=sia.SIA_F32, heads=4, dim=32)) == -2
    need64 = L.sia_workspace_size(sia.OP_INDEX_TOPK, ctypes.byref(seq), 64, 1, 1)
    # the block-aligned selection goes through the score matrix only
    assert f(K=64, order=sia.SELECT_PAGES, method=sia.INDEX_TOPK_ONCHIP, ws_bytes=need64) == -2


def test_topk_pages_validation(Lcpu):
    L = Lcpu
    seq = good_seq()
    need = L.sia_workspace_size(sia.OP_TOPK_PAGES, ctypes.byref(seq), 128, 1, 1)
    # page scores [4, 4] + last pages [4] + kept pages and their scores [4, 2]
    assert need >= 4 * 4 * 4 + 4 * 4 + 2 * 4 * 2 * 4

    def f(K=128, idx=FAKE, ws=FAKE, ws_bytes=need, scores=FAKE, ld=256):
        return L.sia_topk_pages(ctypes.c_void_p(scores), ld, ctypes.byref(seq), K, ctypes.c_void_p(idx), None,
                                ctypes.c_void_p(ws) if ws else None, ws_bytes, None)
    assert f(K=0) == -1
    assert f(K=100) == -1                                          # not whole pages
    assert f(K=32) == -1
    assert f(K=2112) == -2
    assert f(idx=0) == -1
    assert f(scores=FAKE + 4) == -1
    assert f(ld=252) == -1
    assert f(ws=0) == -3
    assert f(ws_bytes=need - 1) == -3
    assert f(ws=FAKE + 64) == -3


def test_index_topk_method_choice(Lcpu):
    L = Lcpu
    m = lambda ix, seq: L.sia_index_topk_method(ctypes.byref(ix), ctypes.byref(seq))
    f32 = good_indexer(dtype=sia.SIA_F32, heads=4, dim=32)
    # one query per sequence and enough (query, range) pairs: on chip
    decode = good_seq(num_tokens=4096, batch=4096, max_pages=512, num_pages=4096, max_visible=32768)
    assert m(good_indexer(), decode) == sia.INDEX_TOPK_ONCHIP
    assert m(f32, decode) == sia.INDEX_TOPK_SCORES
    # many queries per sequence (prefill), or too few pairs to fill the GPU: score matrix
    assert m(good_indexer(), good_seq(num_tokens=65536, batch=1, max_pages=1024, num_pages=1024,
                                      max_visible=65536)) == sia.INDEX_TOPK_SCORES
    assert m(good_indexer(), good_seq(num_tokens=2, batch=2)) == sia.INDEX_TOPK_SCORES
    assert m(good_indexer(), good_seq(page_size=32)) == -2


def mla_call(L, fn, kv, heads=128, K=64, scale=0.04, ws=None, ws_bytes=0, q_dtype=sia.SIA_BF16, seq=None):
    seq = seq or good_seq()
    return fn(ctypes.c_void_p(FAKE), q_dtype, heads, ctypes.byref(kv), ctypes.byref(seq), ctypes.c_void_p(FAKE),
              K, scale, ctypes.c_void_p(FAKE), None, ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_mla_validation(Lcpu):
    L = Lcpu
    kv = sia.KvC(FAKE, 0, sia.SIA_BF16, 64, 512, 512, 64)
    P = L.sia_sparse_mla_prefill
    assert mla_call(L, P, kv, heads=96) == -2
    assert mla_call(L, P, kv, K=0) == -1
    assert mla_call(L, P, kv, scale=0.0) == -1
    assert mla_call(L, P, kv, q_dtype=sia.SIA_F32) == -2
    assert mla_call(L, P, sia.KvC(FAKE, 0, sia.SIA_BF16, 64, 512, 256, 64)) == -2
    assert mla_call(L, P, sia.KvC(FAKE, 0, sia.SIA_FP8_E4M3, 64, 512, 512, 64)) == -1     # no scales
    assert mla_call(L, P, sia.KvC(FAKE, FAKE, sia.SIA_FP8_E4M3, 32, 512, 512, 64)) == -2  # tile
    # decode needs workspace when it splits rows
    assert mla_call(L, L.sia_sparse_mla_decode, kv, K=2048) == -3


def test_workspace_size(L):
    seq = good_seq()
    n = L.sia_workspace_size(sia.OP_INDEX_SELECT_ATTEND, ctypes.byref(seq), 64, 128, 512)
    assert n >= 4 * 256 * 4 + 4 * 64 * 4
    assert L.sia_workspace_size(sia.OP_TOPK, ctypes.byref(seq), 64, 128, 512) == 0
    assert L.sia_workspace_size(sia.OP_TOPK_PAGES, ctypes.byref(seq), 64, 128, 512) > 0
    assert L.sia_workspace_size(9, ctypes.byref(seq), 64, 128, 512) == ctypes.c_size_t(-1).value
    bad = good_seq(page_size=16)
    assert L.sia_workspace_size(0, ctypes.byref(bad), 64, 128, 512) == ctypes.c_size_t(-1).value


def test_zero_tokens_is_a_noop(Lcpu):
    L = Lcpu
    seq = good_seq(num_tokens=0)
    assert call_scores(L, good_indexer(), seq) == 0


def test_noalloc_rejects_workspaces_beyond_its_array(Lcpu):
    """sia_index_select_attend_noalloc validates like sia_index_select_attend
    and returns SIA_ERR_WORKSPACE, before touching the device, for a call
    whose workspace would exceed the library's array (a long prefill's score
    matrix); invalid arguments keep their own status."""
    L = Lcpu
    kv = sia.KvC(FAKE, 0, sia.SIA_BF16, 64, 512, 512, 64)
    ix = good_indexer()

    def f(seq, K=2048, heads=128, order=0, kvs=kv):
        return L.sia_index_select_attend_noalloc(ctypes.byref(ix), ctypes.c_void_p(FAKE), sia.SIA_BF16, heads,
                                                 ctypes.byref(kvs), ctypes.byref(seq), K, order, 0.04,
                                                 ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, None)
    prefill = good_seq(num_tokens=65536, batch=1, max_pages=1024, num_pages=1024, max_visible=65536)
    n = L.sia_workspace_size(sia.OP_INDEX_SELECT_ATTEND, ctypes.byref(prefill), 2048, 128, 512)
    assert n > sia.NOALLOC_WORKSPACE_BYTES
    assert f(prefill) == -3
    assert f(prefill, heads=96) == -2
    assert f(prefill, order=5) == -1
    assert f(good_seq(page_size=32)) == -2
    assert f(good_seq(num_tokens=0)) == 0
    decode = good_seq(num_tokens=64, batch=64, max_pages=512, num_pages=32768, max_visible=32768)
    assert L.sia_workspace_size(sia.OP_INDEX_SELECT_ATTEND, ctypes.byref(decode), 2048, 128, 512) \
        <= sia.NOALLOC_WORKSPACE_BYTES
