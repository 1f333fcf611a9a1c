"""ctypes binding for libsia (argument marshalling only).

Every step of the path runs in the HIP kernels of libsia.so; this module only
turns torch tensors into device pointers and sizes, passes the current HIP
stream, and raises on a negative status.  There is no fallback: if the library
is missing or the tensors are not on a GPU, calls fail loudly.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsia.so")
_lib = None

SIA_F32, SIA_BF16, SIA_FP8_E4M3, SIA_MXFP8_E4M3 = 0, 1, 2, 3
OP_TOPK, OP_MLA_DECODE, OP_MLA_PREFILL, OP_INDEX_SELECT_ATTEND, OP_INDEX_TOPK, OP_TOPK_PAGES = 0, 1, 2, 3, 4, 5
ORDER_SCORE, ORDER_POSITION, SELECT_PAGES = 0, 1, 2
INDEX_TOPK_AUTO, INDEX_TOPK_ONCHIP, INDEX_TOPK_SCORES = 0, 1, 2

c_i32, c_i64, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class SeqMapC(ctypes.Structure):
    _fields_ = [("q_seq", c_p), ("q_pos", c_p), ("block_table", c_p), ("num_tokens", c_i32),
                ("batch", c_i32), ("max_pages", c_i32), ("page_size", c_i32), ("num_pages", c_i32),
                ("max_visible", c_i32)]


class IndexerC(ctypes.Structure):
    _fields_ = [("q", c_p), ("q_scale", c_p), ("w", c_p), ("k_pool", c_p), ("k_scale", c_p),
                ("dtype", ctypes.c_int), ("q_scale_per_head", c_i32), ("heads", c_i32), ("dim", c_i32),
                ("q_bf16", c_i32)]


class KvC(ctypes.Structure):
    _fields_ = [("kv_pool", c_p), ("kv_scale", c_p), ("dtype", ctypes.c_int), ("scale_tokens", c_i32),
                ("scale_elems", c_i32), ("latent_dim", c_i32), ("rope_dim", c_i32)]


class SiaError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libsia.so (built in-tree by sparse_index_attention_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise SiaError(f"{_LIB_PATH} not found: build it with `python -m sparse_index_attention_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        L.sia_index_scores.argtypes = [P(IndexerC), P(SeqMapC), c_p, c_i64, c_p]
        L.sia_topk.argtypes = [c_p, c_i64, P(SeqMapC), c_i32, c_i32, c_p, c_p, c_p]
        L.sia_topk_pages.argtypes = [c_p, c_i64, P(SeqMapC), c_i32, c_p, c_p, c_p, ctypes.c_size_t, c_p]
        L.sia_index_topk_method.argtypes = [P(IndexerC), P(SeqMapC)]
        L.sia_quantize_indexer_q.argtypes = [P(IndexerC), c_i32, c_p, c_p, c_p]
        L.sia_index_topk.argtypes = [P(IndexerC), P(SeqMapC), c_i32, c_i32, c_i32, c_p, c_p, c_p, ctypes.c_size_t,
                                     c_p]
        mla = [c_p, ctypes.c_int, c_i32, P(KvC), P(SeqMapC), c_p, c_i32, ctypes.c_float, c_p, c_p, c_p,
               ctypes.c_size_t, c_p]
        L.sia_sparse_mla_decode.argtypes = mla
        L.sia_sparse_mla_prefill.argtypes = mla
        L.sia_index_select_attend.argtypes = [P(IndexerC), c_p, ctypes.c_int, c_i32, P(KvC), P(SeqMapC), c_i32,
                                              c_i32, ctypes.c_float, c_p, c_p, c_p, c_p, ctypes.c_size_t, c_p]
        L.sia_index_select_attend_noalloc.argtypes = [P(IndexerC), c_p, ctypes.c_int, c_i32, P(KvC), P(SeqMapC),
                                                      c_i32, c_i32, ctypes.c_float, c_p, c_p, c_p, c_p]
        L.sia_workspace_size.argtypes = [c_i32, P(SeqMapC), c_i32, c_i32, c_i32]
        L.sia_workspace_size.restype = ctypes.c_size_t
        L.sia_status_string.argtypes = [ctypes.c_int]
        L.sia_status_string.restype = ctypes.c_char_p
        L.sia_last_hip_error.restype = ctypes.c_char_p
        for f in ("sia_index_scores", "sia_topk", "sia_sparse_mla_decode", "sia_sparse_mla_prefill",
                  "sia_index_select_attend", "sia_index_select_attend_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        L = lib()
        msg = L.sia_status_string(rc).decode()
        if rc == -4:
            msg += ": " + L.sia_last_hip_error().decode()
        raise SiaError(f"libsia error {rc}: {msg}")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise SiaError("libsia takes device tensors (HIP memory)")
    if not t.is_contiguous():
        raise SiaError("libsia takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocation context for buffers a call creates (outputs, workspace): they
    are allocated on the launch stream, so the caching allocator hands a freed
    workspace only to later work on that same stream, never to another stream
    while the library's kernels may still use it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SIA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return SIA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return SIA_FP8_E4M3
    raise SiaError(f"unsupported dtype {t.dtype}")


@dataclass
class SeqMap:
    """Query -> sequence map on the device (see sia_seqmap in include/sia.h)."""
    q_seq: torch.Tensor        # [T] int32
    q_pos: torch.Tensor        # [T] int32
    block_table: torch.Tensor  # [B, max_pages] int32
    num_pages: int
    max_visible: int
    page_size: int = 64

    def c(self) -> SeqMapC:
        for t in (self.q_seq, self.q_pos, self.block_table):
            if t.dtype != torch.int32:
                raise SiaError("sequence map tensors must be int32")
        T = self.q_pos.shape[0]
        return SeqMapC(_ptr(self.q_seq), _ptr(self.q_pos), _ptr(self.block_table), T,
                       self.block_table.shape[0], self.block_table.shape[1], self.page_size,
                       self.num_pages, self.max_visible)

    @property
    def num_tokens(self):
        return int(self.q_pos.shape[0])


@dataclass
class Indexer:
    """q, k_pool: uint8 e4m3 codes or float32.  fp8: q_scale [T] or [T, Hi] and
    k_scale [P, 64] float32.  MXFP8: q_scale [T, Hi, Di/32] and k_scale
    [P, 64, Di/32] uint8 E8M0 group scales (uint8 scales select MXFP8).  A
    bfloat16 q with e4m3 keys is quantized on the fly (q_scale unused)."""
    q: torch.Tensor              # [T, Hi, Di]
    w: torch.Tensor              # [T, Hi] float32
    k_pool: torch.Tensor         # [P, 64, Di] same dtype as q
    q_scale: torch.Tensor = None
    k_scale: torch.Tensor = None

    def c(self) -> IndexerC:
        coded_keys = self.k_pool.dtype in (torch.uint8, torch.float8_e4m3fn)
        mx = coded_keys and self.k_scale is not None and self.k_scale.dtype == torch.uint8
        q_bf16 = int(coded_keys and self.q.dtype == torch.bfloat16)
        per_head = int(not mx and not q_bf16 and self.q_scale is not None and self.q_scale.dim() == 2)
        code = SIA_MXFP8_E4M3 if mx else (SIA_FP8_E4M3 if coded_keys else dtype_code(self.q))
        return IndexerC(_ptr(self.q), _ptr(self.q_scale), _ptr(self.w), _ptr(self.k_pool), _ptr(self.k_scale),
                        code, per_head, self.q.shape[1], self.q.shape[2], q_bf16)


@dataclass
class LatentKV:
    pool: torch.Tensor            # bf16 [P,64,Dc+Dr] | f32 | uint8 [P,64,Dc+2Dr] (fp8 + bf16 rope)
    latent_dim: int = 512
    rope_dim: int = 64
    scale: torch.Tensor = None    # fp8: [P, 64/scale_tokens, Dc/scale_elems] float32
    scale_tokens: int = 64
    scale_elems: int = 512

    def c(self) -> KvC:
        return KvC(_ptr(self.pool), _ptr(self.scale), dtype_code(self.pool), self.scale_tokens,
                   self.scale_elems, self.latent_dim, self.rope_dim)


def workspace_size(op: int, seq: SeqMap, K: int, heads: int, latent_dim: int) -> int:
    s = seq.c()
    n = lib().sia_workspace_size(op, ctypes.byref(s), K, heads, latent_dim)
    if n == ctypes.c_size_t(-1).value:
        raise SiaError("invalid arguments for sia_workspace_size")
    return int(n)


def _workspace(ws, nbytes, device):
    if nbytes == 0:
        return ws
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def index_scores(ix: Indexer, seq: SeqMap, scores: torch.Tensor = None, ld: int = None, stream=None):
    """Indexer scores into scores[T, ld] (float32); entries beyond q_pos are unspecified."""
    T = seq.num_tokens
    if scores is None:
        ld = ld or (seq.max_visible + 3) // 4 * 4
        with _on(stream):
            scores = torch.empty(T, ld, dtype=torch.float32, device=ix.q.device)
    ld = scores.shape[1] if ld is None else ld
    a, s = ix.c(), seq.c()
    _check(lib().sia_index_scores(ctypes.byref(a), ctypes.byref(s), _ptr(scores), ld, _stream(stream)))
    return scores


def topk(scores: torch.Tensor, seq: SeqMap, K: int, order: int = 0, idx=None, vals=None, with_vals=False,
         stream=None):
    T = seq.num_tokens
    with _on(stream):
        if idx is None:
            idx = torch.empty(T, K, dtype=torch.int32, device=scores.device)
        if with_vals and vals is None:
            vals = torch.empty(T, K, dtype=torch.float32, device=scores.device)
    s = seq.c()
    _check(lib().sia_topk(_ptr(scores), scores.shape[1], ctypes.byref(s), K, order, _ptr(idx), _ptr(vals),
                          _stream(stream)))
    return (idx, vals) if with_vals else idx


def topk_pages(scores: torch.Tensor, seq: SeqMap, K: int, idx=None, vals=None, with_vals=False, ws=None,
               stream=None):
    """Block-aligned selection (sia_topk_pages): whole 64-position pages ranked by
    their best visible score, positions in ascending order, -1 padding."""
    T = seq.num_tokens
    with _on(stream):
        if idx is None:
            idx = torch.empty(T, K, dtype=torch.int32, device=scores.device)
        if with_vals and vals is None:
            vals = torch.empty(T, K, dtype=torch.float32, device=scores.device)
        ws = _workspace(ws, workspace_size(OP_TOPK_PAGES, seq, K, 1, 1), scores.device)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    s = seq.c()
    _check(lib().sia_topk_pages(_ptr(scores), scores.shape[1], ctypes.byref(s), K, _ptr(idx), _ptr(vals), _ptr(ws),
                                nbytes, _stream(stream)))
    return (idx, vals) if with_vals else idx


def index_topk(ix: Indexer, seq: SeqMap, K: int, order: int = 0, method: int = 0, idx=None, vals=None,
               with_vals=False, ws=None, stream=None):
    """Indexer scores and Top-K in one call: same result as topk(index_scores(ix, seq), seq, K, order)
    (order SELECT_PAGES: as topk_pages).  method: INDEX_TOPK_AUTO, INDEX_TOPK_ONCHIP or INDEX_TOPK_SCORES."""
    T = seq.num_tokens
    dev = ix.q.device
    with _on(stream):
        if idx is None:
            idx = torch.empty(T, K, dtype=torch.int32, device=dev)
        if with_vals and vals is None:
            vals = torch.empty(T, K, dtype=torch.float32, device=dev)
        ws = _workspace(ws, workspace_size(OP_INDEX_TOPK, seq, K, 1, 1), dev)
    a, s = ix.c(), seq.c()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().sia_index_topk(ctypes.byref(a), ctypes.byref(s), K, order, method, _ptr(idx), _ptr(vals), _ptr(ws),
                                nbytes, _stream(stream)))
    return (idx, vals) if with_vals else idx


def quantize_indexer_q(ix: Indexer, stream=None):
    """bf16 queries of `ix` -> (e4m3 codes [T, Hi, Di], scales): float [T] for
    fp8 keys, uint8 E8M0 [T, Hi, Di/32] for MXFP8 keys."""
    a = ix.c()
    T, Hi, Di = ix.q.shape
    with _on(stream):
        codes = torch.empty(T, Hi, Di, dtype=torch.uint8, device=ix.q.device)
        if a.dtype == SIA_MXFP8_E4M3:
            scales = torch.empty(T, Hi, Di // 32, dtype=torch.uint8, device=ix.q.device)
        else:
            scales = torch.empty(T, dtype=torch.float32, device=ix.q.device)
    _check(lib().sia_quantize_indexer_q(ctypes.byref(a), T, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def index_topk_method(ix: Indexer, seq: SeqMap) -> str:
    """Name of the method index_topk's INDEX_TOPK_AUTO runs for these arguments."""
    a, s = ix.c(), seq.c()
    m = lib().sia_index_topk_method(ctypes.byref(a), ctypes.byref(s))
    _check(min(m, 0))
    return {INDEX_TOPK_ONCHIP: "onchip", INDEX_TOPK_SCORES: "scores"}[m]


def _mla(fn, op, q, kv: LatentKV, seq: SeqMap, idx, K, softmax_scale, out, lse, ws, stream):
    T, H = q.shape[0], q.shape[1]
    n = workspace_size(op, seq, K, H, kv.latent_dim) if kv.pool.dtype != torch.float32 else 0
    with _on(stream):
        if out is None:
            out = torch.empty(T, H, kv.latent_dim, dtype=q.dtype, device=q.device)
        ws = _workspace(ws, n, q.device)
    s, k = seq.c(), kv.c()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(fn(_ptr(q), dtype_code(q), H, ctypes.byref(k), ctypes.byref(s), _ptr(idx), K, float(softmax_scale),
              _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream)))
    return out


def sparse_mla_decode(q, kv: LatentKV, seq: SeqMap, idx, K, softmax_scale, out=None, lse=None, ws=None,
                      stream=None):
    return _mla(lib().sia_sparse_mla_decode, OP_MLA_DECODE, q, kv, seq, idx, K, softmax_scale, out, lse, ws,
                stream)


def sparse_mla_prefill(q, kv: LatentKV, seq: SeqMap, idx, K, softmax_scale, out=None, lse=None, ws=None,
                       stream=None):
    return _mla(lib().sia_sparse_mla_prefill, OP_MLA_PREFILL, q, kv, seq, idx, K, softmax_scale, out, lse, ws,
                stream)


def index_select_attend(ix: Indexer, q, kv: LatentKV, seq: SeqMap, K, softmax_scale, order=0, idx_out=None,
                        out=None, lse=None, ws=None, stream=None):
    T, H = q.shape[0], q.shape[1]
    n = workspace_size(OP_INDEX_SELECT_ATTEND, seq, K, H, kv.latent_dim)
    with _on(stream):
        if out is None:
            out = torch.empty(T, H, kv.latent_dim, dtype=q.dtype, device=q.device)
        ws = _workspace(ws, n, q.device)
    a, s, k = ix.c(), seq.c(), kv.c()
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().sia_index_select_attend(ctypes.byref(a), _ptr(q), dtype_code(q), H, ctypes.byref(k),
                                         ctypes.byref(s), K, order, float(softmax_scale), _ptr(idx_out),
                                         _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream)))
    return out


NOALLOC_WORKSPACE_BYTES = 64 << 20   # SIA_NOALLOC_WORKSPACE_BYTES


def index_select_attend_noalloc(ix: Indexer, q, kv: LatentKV, seq: SeqMap, K, softmax_scale, order=0, idx_out=None,
                                out=None, lse=None, stream=None):
    """index_select_attend without a workspace: the library uses its own
    per-GPU device array (SIA_NOALLOC_WORKSPACE_BYTES) and allocates nothing.
    Pass `out` (and `idx_out`, `lse`) to keep the whole call allocation-free;
    calls that may overlap on one GPU must be serialized by the caller."""
    T, H = q.shape[0], q.shape[1]
    if out is None:
        with _on(stream):
            out = torch.empty(T, H, kv.latent_dim, dtype=q.dtype, device=q.device)
    a, s, k = ix.c(), seq.c(), kv.c()
    _check(lib().sia_index_select_attend_noalloc(ctypes.byref(a), _ptr(q), dtype_code(q), H, ctypes.byref(k),
                                                 ctypes.byref(s), K, order, float(softmax_scale), _ptr(idx_out),
                                                 _ptr(out), _ptr(lse), _stream(stream)))
    return out
