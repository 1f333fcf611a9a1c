"""Plain CPU oracle for sparse index attention (indexer -> Top-K -> sparse MLA).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and never falls back to it.

Everything is computed in float64 with NumPy, directly from the definitions, one
query row at a time.  Library primitives (matmul, lexsort, exp) are used as
single steps; nothing is blocked, fused or reordered beyond the definitions.

Pages cited (Baidu AI Cloud articles):
  [P1] "Day 0 Inference Adaptation and Optimization for Hybrid Attention Models"
  [P2] "Efficient Inference Deployment and Optimization for Hybrid Attention LLMs"
  [P3] "Day-One Inference Adaptation for Very Large Hybrid-Attention Models:
        From Operators to Serving Systems"
  [P4] "Inference Acceleration for New LLM Architectures: Day-0 Adaptation and
        Sparse Attention Optimization"
  [P5] "Inference Adaptation and Performance Optimization for a Domestically
        Developed LLM's New Architecture"

The pages describe the method in prose only (no formulas).  Where they leave a
step open, the reading taken here is stated next to the function; the readings
are: ReLU per indexer head before the head weighting; one indexer key per token
shared by all indexer heads; causal visibility s <= q_pos (diagonal included);
Top-K order (score descending, position ascending) with -0 == +0; K larger than
the visible count emits every visible position then -1; the MLA key is the whole
latent+rope row and the value is its latent part, shared by all heads; softmax is
exact; fp8 is OCP e4m3fn; an MXFP8 group is 32 consecutive elements of a query
head's or a key's dim axis sharing one OCP E8M0 scale.

Every function below is pinned by CPU tests against closed forms, library
routines, brute force or invariants (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_e4m3", "decode_bf16", "decode_e8m0", "mx_values", "encode_e4m3", "quantize_q_fp8", "quantize_q_mx",
    "physical_slots", "key_rows", "kv_rows",
    "index_scores_row", "index_scores", "topk_row", "topk", "topk_pages_row", "topk_pages", "sparse_mla_row",
    "sparse_mla", "merge_partials", "index_select_attend",
]


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------
def decode_e4m3(codes) -> np.ndarray:
    """OCP FP8 E4M3 ("e4m3fn") byte -> float64, from the format definition.

    Byte layout s eeee mmm, exponent bias 7.  e == 0 is subnormal
    (m/8 * 2^-6); e == 15 with m == 7 is NaN (the format has no infinities);
    otherwise (1 + m/8) * 2^(e-7).  Largest finite magnitude is 448.
    [P1, "Hierarchical Quantization"] and [P2, section 4] name FP8 for the index
    and KV paths; the e4m3 flavour is a reading (the OCP variant).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    sub = (m / 8.0) * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    val = np.where(e == 0, sub, nor)
    val = np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)
    return sign * val


def decode_e8m0(codes) -> np.ndarray:
    """OCP E8M0 scale byte -> float64: 2^(e - 127); 0xFF is NaN.

    The indexer's MXFP8 groups share one power-of-two scale ("block
    floating-point ... shared exponent", [P2, section 4.1]; [P5, section 4
    table]); the 8-bit exponent-only encoding is the OCP MX one (a reading:
    the pages name MXFP8 but print no encoding).
    """
    e = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    val = np.ldexp(1.0, (e - 127).astype(np.int64))
    return np.where(e == 255, np.nan, val)


def mx_values(codes, scales, group=32) -> np.ndarray:
    """MXFP8 block -> float64: e4m3 code x the E8M0 scale of its group of 32
    consecutive elements along the last axis ([P1, "Hierarchical
    Quantization"]: group size 32; [P2, section 4.1])."""
    v = decode_e4m3(codes)
    sc = decode_e8m0(scales)
    return v * np.repeat(sc, group, axis=-1)


_E4M3_GRID = None


def encode_e4m3(v) -> np.ndarray:
    """float -> e4m3 code: the nearest value of the format's grid (ties to the
    even code), saturating to +-448, sign kept (so -0 -> 0x80).  The grid is
    the decoded value of every finite code 0x00..0x7e."""
    global _E4M3_GRID
    if _E4M3_GRID is None:
        _E4M3_GRID = decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    x = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_GRID, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_GRID[lo], _E4M3_GRID[hi] - a
    code = np.where((dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0)), hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def quantize_q_fp8(q_bits):
    """Dynamic per-token fp8 quantization of bf16 queries [T, Hi, Di] -> (e4m3
    codes, float32 scale [T]).

    The indexer prolog quantizes Q on the fly ([P2, section 3.2 "Q
    quantization"]; [P3, section 2, three-stream prolog]).  Reading: one scale
    per token from its absolute maximum, scale = amax / 448 and codes =
    e4m3(x * (448 / amax)), both divisions and the product in float32 (a token
    of zeros gets scale 1 and zero codes)."""
    x = decode_bf16(q_bits).astype(np.float32)
    T = x.shape[0]
    amax = np.max(np.abs(x.reshape(T, -1)), axis=1).astype(np.float32)
    nz = amax > 0
    r = np.where(nz, np.float32(448.0) / np.where(nz, amax, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
    scale = np.where(nz, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    v = (x * r.reshape((T,) + (1,) * (x.ndim - 1))).astype(np.float32)
    return encode_e4m3(v), scale


def quantize_q_mx(q_bits, group=32):
    """Dynamic MXFP8 quantization of bf16 queries [T, Hi, Di] -> (e4m3 codes,
    E8M0 bytes [T, Hi, Di/group]).

    MXFP8 groups of 32 with a shared power-of-two scale ([P2, section 4.1];
    [P5, section 4 table]).  Reading: the scale is the smallest 2^e with
    amax <= 448 * 2^e (no element saturates; with amax = m * 2^E, m in
    [0.5, 1): e = E - 9 if m <= 0.875 else E - 8), byte e + 127, and an
    all-zero group gets byte 0; codes = e4m3(x * 2^-e)."""
    x = decode_bf16(q_bits)
    g = x.reshape(*x.shape[:-1], x.shape[-1] // group, group)
    amax = np.max(np.abs(g), axis=-1)
    m, E = np.frexp(amax)
    e = np.where(m <= 0.875, E - 9, E - 8)
    e = np.clip(np.where(amax > 0, e, -127), -127, 127).astype(np.int64)
    codes = encode_e4m3(g * np.ldexp(1.0, -e)[..., None]).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def decode_bf16(bits) -> np.ndarray:
    """bfloat16 bit pattern (uint16) -> float64: the upper half of an IEEE float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Paging
# ---------------------------------------------------------------------------
def physical_slots(block_table_row, positions, page_size) -> np.ndarray:
    """Logical token positions of one sequence -> physical slot numbers.

    Slot = block_table[b][pos // page] * page + pos % page.  The pages have the
    indexer read the paged key cache directly and the sparse kernel read the
    paged KV cache ([P1, "Sparse Attention Pipeline Optimization"],
    [P4, section 2]); the same block table serves both pools (a reading).
    """
    pos = np.asarray(positions, dtype=np.int64)
    table = np.asarray(block_table_row, dtype=np.int64)
    return table[pos // page_size] * page_size + pos % page_size


def key_rows(k_pool, k_scale, slots, k_mx=None):
    """Indexer keys at the given slots: (decoded key values [n, Di], key scales [n]).

    MXFP8 keys (k_mx given, [pages, page, Di/32] E8M0 bytes) fold their group
    scales into the values and have unit key scales."""
    D = k_pool.shape[-1]
    flat = k_pool.reshape(-1, D)[slots]
    if k_mx is not None:
        vals = mx_values(flat, np.asarray(k_mx).reshape(-1, D // 32)[slots])
        sc = np.ones(len(slots), dtype=np.float64)
    elif k_pool.dtype == np.uint8:
        vals = decode_e4m3(flat)
        sc = np.asarray(k_scale, dtype=np.float64).reshape(-1)[slots]
    elif k_pool.dtype == np.uint16:                 # bfloat16 bit patterns
        vals = decode_bf16(flat)
        sc = np.ones(len(slots), dtype=np.float64)
    else:
        vals = flat.astype(np.float64)
        sc = np.ones(len(slots), dtype=np.float64)
    return vals, sc


def kv_rows(kv, slots) -> np.ndarray:
    """Latent+rope KV rows at the given slots, decoded to float64 [n, Dc+Dr].

    kv is a dict with keys: pool, dtype ('f32' | 'bf16' | 'fp8'), Dc, Dr, page_size
    and, for fp8, scale and scale_tokens / scale_elems.

    fp8 rows hold Dc e4m3 codes followed by Dr bfloat16 values (rope kept in 16
    bits).  Latent element d of slot j is code * scale[tile], where the tile
    groups scale_tokens consecutive tokens of a page and scale_elems consecutive
    latent elements.  [P5, section 4 table] and [P2, section 4.2] give FP8 with
    a scale per token and per 128-element tile; a scale shared by a whole page of
    64 tokens over the 512 latent values is the other granularity supported.
    """
    pool, dt, Dc, Dr = kv["pool"], kv["dtype"], kv["Dc"], kv["Dr"]
    if dt == "f32":
        return pool.reshape(-1, Dc + Dr)[slots].astype(np.float64)
    if dt == "bf16":
        return decode_bf16(pool.reshape(-1, Dc + Dr)[slots])
    assert dt == "fp8"
    page = kv["page_size"]
    rows = pool.reshape(-1, Dc + 2 * Dr)[slots]
    codes = decode_e4m3(rows[:, :Dc])
    rope = decode_bf16(np.ascontiguousarray(rows[:, Dc:]).view(np.uint16))
    st, se = kv["scale_tokens"], kv["scale_elems"]
    tiles_per_page = (page // st) * (Dc // se)
    scale = np.asarray(kv["scale"], dtype=np.float64).reshape(-1)
    slots = np.asarray(slots, dtype=np.int64)
    p, i = slots // page, slots % page
    d_tile = np.arange(Dc) // se
    sidx = (p * tiles_per_page + (i // st) * (Dc // se))[:, None] + d_tile[None, :]
    latent = codes * scale[sidx]
    return np.concatenate([latent, rope], axis=1)


# ---------------------------------------------------------------------------
# Step 1: indexer scores
# ---------------------------------------------------------------------------
def index_scores_row(q_row, q_scale_row, w_row, keys, k_scale) -> np.ndarray:
    """Scores of one query against n visible keys, float64 [n].

    I[s] = sum_h w[h] * ReLU(q_scale[h] * k_scale[s] * <q[h], k[s]>)

    The indexer scores each history position per head, weights the per-head
    scores with the query's head weights and sums them ([P1, "Sparse Attention
    Pipeline Optimization"] pseudo-code; [P2, section 3.1]; [P5, section 3]).
    The ReLU per head before weighting is a reading; scales are the fp8
    dequantization factors (1 for float inputs).
    """
    dots = q_row @ keys.T                                   # [Hi, n]
    scaled = dots * q_scale_row[:, None] * k_scale[None, :]
    return (w_row[:, None] * np.maximum(scaled, 0.0)).sum(axis=0)


def _q_index_row(idx, t):
    q = idx["q"][t]
    if idx.get("q_mx") is not None:
        qv = mx_values(q, idx["q_mx"][t])
        qs = np.ones(q.shape[0])
    elif q.dtype == np.uint16:                       # bfloat16 path: no scales
        qv = decode_bf16(q)
        qs = np.ones(q.shape[0])
    elif q.dtype == np.uint8:
        qv = decode_e4m3(q)
        qs = np.asarray(idx["q_scale"][t], dtype=np.float64)
        qs = np.broadcast_to(qs, (q.shape[0],)) if qs.ndim == 0 else qs
    else:
        qv = q.astype(np.float64)
        qs = np.ones(q.shape[0])
    return qv, qs, idx["w"][t].astype(np.float64)


def index_scores(idx, seq, rows=None) -> dict:
    """Scores for query rows `rows` (default: all).  Returns {t: float32 [q_pos[t]+1]}.

    idx: dict with q [Tq,Hi,Di] (uint8 codes, uint16 bfloat16 bits or f32; the
    bfloat16 indexer path of [P2, section 3.2] and [P5, section 3.1] has no
    scales), q_scale ([Tq] or [Tq,Hi],
    fp8 only), w [Tq,Hi], k [P,page,Di], k_scale [P,page] (fp8 only); MXFP8
    instead gives q_mx [Tq,Hi,Di/32] and k_mx [P,page,Di/32] E8M0 bytes.
    seq: dict with q_seq, q_pos, block_table, page_size.
    Causal visibility: key s is visible to query t iff s <= q_pos[t] (a reading
    of the causal history the pages describe, [P1, "Prefill Context
    Parallelism"]).  The float64 result is rounded to float32, the dtype of the
    score buffer the pipeline hands to Top-K.
    """
    Tq = len(seq["q_pos"])
    rows = range(Tq) if rows is None else rows
    out = {}
    for t in rows:
        b, pos = int(seq["q_seq"][t]), int(seq["q_pos"][t])
        slots = physical_slots(seq["block_table"][b], np.arange(pos + 1), seq["page_size"])
        keys, ks = key_rows(idx["k"], idx.get("k_scale"), slots, idx.get("k_mx"))
        qv, qs, w = _q_index_row(idx, t)
        out[t] = index_scores_row(qv, qs, w, keys, ks).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Step 2: Top-K
# ---------------------------------------------------------------------------
def topk_row(scores_f32, K, order=0) -> np.ndarray:
    """Top-K of one row of float32 scores over positions 0..n-1, int32 [K].

    Keeps the first min(K, n) positions under the order (score descending,
    position ascending), with -0.0 equal to +0.0; pads with -1.  order=0 emits
    them in that order, order=1 in ascending position (same set).
    The pages keep the K best-scored history positions per query
    ([P1, "Sparse Attention Pipeline Optimization"]; [P2, section 3.2]); the
    tie-break toward the lower position is a reading.  Scores must be finite.
    """
    s = np.asarray(scores_f32, dtype=np.float32).astype(np.float64)
    assert np.all(np.isfinite(s)), "Top-K contract covers finite scores only"
    s = s + 0.0                                    # -0.0 + 0.0 == +0.0
    n = s.shape[0]
    perm = np.lexsort((np.arange(n), -s))          # primary: -s, secondary: position
    sel = perm[: min(K, n)]
    if order == 1:
        sel = np.sort(sel)
    out = np.full(K, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


def topk(scores: dict, K, order=0) -> dict:
    """Top-K for every row of a {t: float32 scores} dict -> {t: int32 [K]}."""
    return {t: topk_row(s, K, order) for t, s in scores.items()}


def topk_pages_row(scores_f32, K, page=64):
    """Block-aligned selection of one row of float32 scores, int32 [K].

    [P3, section 3.1] aligns the selection to cache blocks so that attention
    reads the cache in whole blocks.  The page does not say how a block is
    ranked; the reading taken here: a block of `page` consecutive positions
    scores the largest score among its visible positions (a block is kept when
    it holds one of the strongest positions), the first min(K / page, blocks)
    blocks under (block score descending, block index ascending) are kept, and
    every visible position of a kept block is emitted, blocks in ascending
    order, -1 padding up to K.  K must be a multiple of `page`.  With page = 1
    this is topk_row(order=1).  Scores must be finite.
    """
    assert K % page == 0, "block-aligned selection takes whole blocks"
    s = np.asarray(scores_f32, dtype=np.float32).astype(np.float64)
    assert np.all(np.isfinite(s)), "Top-K contract covers finite scores only"
    s = s + 0.0                                    # -0.0 + 0.0 == +0.0
    n = s.shape[0]
    n_blocks = -(-n // page)
    best = np.array([s[b * page: min(n, (b + 1) * page)].max() for b in range(n_blocks)])
    perm = np.lexsort((np.arange(n_blocks), -best))
    kept = np.sort(perm[: min(K // page, n_blocks)])
    out = np.full(K, -1, dtype=np.int32)
    at = 0
    for b in kept:
        cols = np.arange(b * page, min(n, (b + 1) * page))
        out[at: at + cols.shape[0]] = cols
        at += cols.shape[0]
    return out


def topk_pages(scores: dict, K, page=64) -> dict:
    """Block-aligned selection for every row of a {t: float32 scores} dict."""
    return {t: topk_pages_row(s, K, page) for t, s in scores.items()}


# ---------------------------------------------------------------------------
# Step 3: sparse MLA attention over the selected rows
# ---------------------------------------------------------------------------
def sparse_mla_row(q_row, rows, Dc, scale):
    """Attention of one token (all heads) over its selected latent rows.

    q_row [H, Dc+Dr], rows [m, Dc+Dr] (float64).  For each head h:
      l_j = scale * <q[h], row_j>            (key = whole latent+rope row)
      p = softmax(l), O[h] = sum_j p_j * row_j[:Dc]   (value = latent part)
      LSE[h] = log sum_j exp(l_j)
    The sparse kernel reads only the selected rows and runs ordinary blockwise
    attention over them ([P1, "Sparse Attention Pipeline Optimization"];
    [P3, section 3.2]); attention over a compressed latent cache per
    [P5, section 1].  Blockwise evaluation does not change the result, so the
    plain softmax is the definition.  With no rows, O = 0 and LSE = -inf.
    """
    H = q_row.shape[0]
    if rows.shape[0] == 0:
        return np.zeros((H, Dc)), np.full(H, -np.inf)
    logits = scale * (q_row @ rows.T)               # [H, m]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ rows[:, :Dc]) / l
    lse = (mx + np.log(l))[:, 0]
    return out, lse


def _q_mla_row(q, t):
    r = q[t]
    return decode_bf16(r) if r.dtype == np.uint16 else r.astype(np.float64)


def sparse_mla(q, kv, seq, sel: dict, scale) -> dict:
    """Sparse MLA for each row t of `sel` ({t: int32 [K] logical positions, -1 = none}).

    Returns {t: (out [H, Dc] float64, lse [H] float64)}.
    """
    res = {}
    for t, ids in sel.items():
        ids = np.asarray(ids)
        ids = ids[ids >= 0]
        b = int(seq["q_seq"][t])
        slots = physical_slots(seq["block_table"][b], ids, seq["page_size"])
        rows = kv_rows(kv, slots)
        res[t] = sparse_mla_row(_q_mla_row(q, t), rows, kv["Dc"], scale)
    return res


def merge_partials(outs, lses):
    """Exact merge of attention results over disjoint row subsets.

    outs [S, H, Dc] (each normalised over its subset), lses [S, H].  The merged
    output is sum_s exp(lse_s - LSE) * out_s with LSE = log sum_s exp(lse_s).
    This is the softmax identity the split evaluation relies on; empty subsets
    (lse = -inf) contribute nothing.
    """
    lses = np.asarray(lses, dtype=np.float64)
    mx = np.max(lses, axis=0)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    wts = np.exp(lses - mx_safe[None])
    tot = wts.sum(axis=0)
    out = (wts[:, :, None] * np.asarray(outs)).sum(axis=0) / np.where(tot > 0, tot, 1.0)[:, None]
    lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return out, lse


# ---------------------------------------------------------------------------
# The whole path
# ---------------------------------------------------------------------------
def index_select_attend(idx, q, kv, seq, K, scale, rows=None, order=0):
    """Scores -> Top-K -> sparse MLA for the given query rows.

    order 0 / 1: per-position Top-K in score / position order; order 2: the
    block-aligned selection of topk_pages_row with the cache's page size.
    Returns (scores {t: f32}, selected {t: int32 [K]}, attention {t: (out, lse)}).
    [P1, "Sparse Attention Pipeline Optimization"] pseudo-code: the indexer
    scores and weights, Top-K picks positions, the sparse kernel gathers and
    attends.
    """
    sc = index_scores(idx, seq, rows)
    sel = topk_pages(sc, K, seq["page_size"]) if order == 2 else topk(sc, K, order)
    att = sparse_mla(q, kv, seq, sel, scale)
    return sc, sel, att
