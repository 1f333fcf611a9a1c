"""Sparse index attention on AMD MI355X (gfx950).

The hot path (indexer scores -> per-query Top-K -> sparse MLA attention over a
paged latent KV cache) runs in the HIP kernels of libsia.so, behind the C ABI
declared in include/sia.h.  `sia` is the thin ctypes binding; `workloads` draws
the seeded synthetic inputs.
"""
from . import sia  # noqa: F401
from .sia import (Indexer, LatentKV, SeqMap, SiaError, index_scores, index_select_attend,  # noqa: F401
                  sparse_mla_decode, sparse_mla_prefill, topk, workspace_size)
