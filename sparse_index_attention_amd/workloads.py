"""Seeded synthetic inputs for sparse index attention.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scoring, selection or attention).  Both the HIP path and
the CPU oracle consume the arrays it returns.

Generation is chunked: rows of each tensor are drawn in blocks of CHUNK rows,
block c of tensor `tid` in config `cid` from SeedSequence([2026, cid, tid, c]).
A sampled row can therefore be re-drawn alone, and the blocks can be drawn by
several threads at once with bit-identical results.

Tensor ids: 0 indexer q, 1 indexer k, 2 head weights, 3 MLA q, 4 latent KV,
5 page permutation.

Distributions: indexer q/k, MLA q and latent KV ~ N(0,1); head weights ~ U(0,1).
fp8 tensors are quantized with a dynamic scale = amax/448 over the scale group
(amax 0 -> scale 1), codes = round-to-nearest-even(x/scale) saturated to +-448
(OCP e4m3fn).  MXFP8 tensors take one power-of-two scale per 32 consecutive
elements of the last axis, the smallest 2^e with amax <= 448 * 2^e, stored as
an E8M0 byte (amax 0 -> byte 0), and the same e4m3 rounding.  bf16 tensors are float32 draws rounded to nearest even.
Physical pages are a random permutation of the pool (shuffled block tables).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 4096
PAGE = 64

# Named workloads.  The first five are the measured configurations; the
# "*_tiny" ones keep the same dtypes and layouts at sizes a plain CPU
# implementation checks in seconds (ragged lengths, several tiles, short rows).
CONFIGS = {
    # one sequence, T=256, fp32 throughout
    "tiny_prefill": dict(cid=0, kind="prefill", T=256, Hi=4, Di=32, idx_dtype="f32", K=32,
                         H=8, Dc=64, Dr=16, kv_dtype="f32"),
    # 64 sequences x 32768 context, one query each
    "decode": dict(cid=1, kind="decode", B=64, ctx=32768, Hi=64, Di=128, idx_dtype="fp8",
                   K=2048, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    # one sequence of 65536 tokens, causal
    "long_prefill": dict(cid=2, kind="prefill", T=65536, Hi=64, Di=128, idx_dtype="fp8",
                         K=2048, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    # 16 sequences x 131072 context, fp8 latent KV with one scale per 64-token page
    "quant_decode": dict(cid=3, kind="decode", B=16, ctx=131072, Hi=64, Di=128, idx_dtype="fp8",
                         K=2048, H=128, Dc=512, Dr=64, kv_dtype="fp8", kv_scale=(64, 512)),
    # the same with the pages' KV tiling: one fp32 scale per token and 128-element tile
    "quant_decode_tile128": dict(cid=3, kind="decode", B=16, ctx=131072, Hi=64, Di=128, idx_dtype="fp8",
                                 K=2048, H=128, Dc=512, Dr=64, kv_dtype="fp8", kv_scale=(1, 128)),
    # rank 0 of a 16-way zigzag split of a 262144-token prefix: segments 0 and 31 of 32
    "cp_chunk_prefill": dict(cid=4, kind="zigzag", total=262144, segments=32, rank=0,
                             Hi=64, Di=128, idx_dtype="fp8", K=2048, H=128, Dc=512, Dr=64,
                             kv_dtype="bf16"),
    # --- small parity cases -------------------------------------------------
    "tiny_prefill_identity": dict(cid=0, kind="prefill", T=256, Hi=4, Di=32, idx_dtype="f32",
                                  K=32, H=8, Dc=64, Dr=16, kv_dtype="f32", identity_pages=True),
    "decode_tiny": dict(cid=11, kind="decode", B=6, ctx=[1, 63, 64, 700, 2100, 3001], Hi=64,
                        Di=128, idx_dtype="fp8", K=256, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    "prefill_tiny": dict(cid=12, kind="prefill", T=650, Hi=64, Di=128, idx_dtype="fp8", K=128,
                         H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    "quant_decode_tiny": dict(cid=13, kind="decode", B=4, ctx=[5, 300, 1111, 2500], Hi=64, Di=128,
                              idx_dtype="fp8", K=512, H=128, Dc=512, Dr=64, kv_dtype="fp8",
                              kv_scale=(64, 512)),
    "quant_decode_tile128_tiny": dict(cid=14, kind="decode", B=3, ctx=[90, 777, 1500], Hi=64,
                                      Di=128, idx_dtype="fp8", K=256, H=128, Dc=512, Dr=64,
                                      kv_dtype="fp8", kv_scale=(1, 128)),
    "cp_chunk_prefill_tiny": dict(cid=15, kind="zigzag", total=512, segments=32, rank=0, Hi=64,
                                  Di=128, idx_dtype="fp8", K=64, H=128, Dc=512, Dr=64,
                                  kv_dtype="bf16"),
    "decode_h64_tiny": dict(cid=16, kind="decode", B=3, ctx=[33, 500, 1300], Hi=32, Di=128,
                            idx_dtype="fp8", K=192, H=64, Dc=512, Dr=64, kv_dtype="bf16"),
    # bfloat16 indexer (the precision path), otherwise as decode / prefill
    "bf16_decode": dict(cid=6, kind="decode", B=64, ctx=32768, Hi=64, Di=128, idx_dtype="bf16",
                        K=2048, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    "bf16_decode_tiny": dict(cid=20, kind="decode", B=5, ctx=[1, 65, 500, 2100, 9000], Hi=64, Di=128,
                             idx_dtype="bf16", K=256, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    "bf16_prefill_tiny": dict(cid=21, kind="prefill", T=390, Hi=32, Di=128, idx_dtype="bf16", K=64,
                              H=64, Dc=512, Dr=64, kv_dtype="bf16"),
    "bf16_chunked_prefill_tiny": dict(cid=22, kind="chunked", ctx=[300, 1000, 77, 2100, 5],
                                      new=[37, 130, 77, 9, 2], Hi=64, Di=128, idx_dtype="bf16", K=128,
                                      H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    # MXFP8 indexer (32-element groups with E8M0 scales), otherwise as decode / prefill
    "mx_decode": dict(cid=5, kind="decode", B=64, ctx=32768, Hi=64, Di=128, idx_dtype="mxfp8",
                      K=2048, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    "mx_decode_tiny": dict(cid=18, kind="decode", B=5, ctx=[1, 64, 333, 2100, 9000], Hi=64, Di=128,
                           idx_dtype="mxfp8", K=256, H=128, Dc=512, Dr=64, kv_dtype="bf16"),
    "mx_prefill_tiny": dict(cid=19, kind="prefill", T=430, Hi=32, Di=128, idx_dtype="mxfp8", K=64,
                            H=64, Dc=512, Dr=64, kv_dtype="bf16"),
    # batched chunked prefill: sequence b holds ctx[b] tokens, the last new[b] of them are queries
    "chunked_prefill_tiny": dict(cid=17, kind="chunked", ctx=[300, 1000, 77, 2100, 5], new=[37, 130, 77, 9, 2],
                                 Hi=64, Di=128, idx_dtype="fp8", K=128, H=128, Dc=512, Dr=64,
                                 kv_dtype="bf16"),
}


@dataclass
class Workload:
    name: str
    cfg: dict
    # sequence map
    q_seq: np.ndarray
    q_pos: np.ndarray
    seq_lens: np.ndarray
    block_table: np.ndarray
    num_pages: int
    # indexer
    iq: np.ndarray = None          # [Tq, Hi, Di] uint8 codes or float32
    iq_scale: np.ndarray = None    # [Tq] float32 (fp8 only)
    iw: np.ndarray = None          # [Tq, Hi] float32
    ik: np.ndarray = None          # [P, PAGE, Di] uint8 codes or float32
    ik_scale: np.ndarray = None    # [P, PAGE] float32 (fp8 only)
    # MLA
    q: np.ndarray = None           # [Tq, H, Dc+Dr] uint16 (bf16 bits) or float32
    kv: np.ndarray = None          # [P, PAGE, Dc+Dr] uint16 / float32, or [P, PAGE, Dc+2Dr] uint8
    kv_scale: np.ndarray = None    # fp8 only
    extra: dict = field(default_factory=dict)

    @property
    def Tq(self):
        return int(self.q_pos.shape[0])

    @property
    def max_visible(self):
        return int(self.q_pos.max()) + 1

    @property
    def softmax_scale(self):
        return 1.0 / math.sqrt(self.cfg["Dc"] + self.cfg["Dr"])

    # dict views in the form the CPU oracle takes
    def oracle_seq(self):
        return dict(q_seq=self.q_seq, q_pos=self.q_pos, block_table=self.block_table,
                    page_size=PAGE)

    def oracle_indexer(self):
        if self.cfg["idx_dtype"] == "mxfp8":
            return dict(q=self.iq, q_mx=self.iq_scale, w=self.iw, k=self.ik, k_mx=self.ik_scale)
        if self.cfg["idx_dtype"] == "bf16":
            return dict(q=self.iq, w=self.iw, k=self.ik)
        return dict(q=self.iq, q_scale=self.iq_scale, w=self.iw, k=self.ik, k_scale=self.ik_scale)

    def oracle_kv(self):
        c = self.cfg
        d = dict(pool=self.kv, dtype=c["kv_dtype"], Dc=c["Dc"], Dr=c["Dr"], page_size=PAGE)
        if c["kv_dtype"] == "fp8":
            st, se = c["kv_scale"]
            d.update(scale=self.kv_scale, scale_tokens=st, scale_elems=se)
        return d


# ---------------------------------------------------------------------------
# random draws
# ---------------------------------------------------------------------------
def _rng(cid, tid, chunk):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, cid, tid, chunk])))


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _draw_rows(cid, tid, nrows, row_shape, kind, out=None, convert=None, out_dtype=None):
    """Draw `nrows` rows of shape row_shape, chunk by chunk (threaded).

    kind: 'normal' or 'uniform'.  `convert(chunk_f32, first_row)` maps a float32
    chunk to its stored form (bf16 bits, fp8 codes...) and may write side outputs.
    """
    row_elems = int(np.prod(row_shape))
    if out is None:
        out = np.empty((nrows,) + tuple(row_shape), dtype=out_dtype or np.float32)
    nchunks = (nrows + CHUNK - 1) // CHUNK

    def work(c):
        r0, r1 = c * CHUNK, min(nrows, (c + 1) * CHUNK)
        g = _rng(cid, tid, c)
        n = (r1 - r0) * row_elems
        x = g.standard_normal(n, dtype=np.float32) if kind == "normal" else g.random(n, dtype=np.float32)
        x = x.reshape((r1 - r0,) + tuple(row_shape))
        out[r0:r1] = convert(x, r0) if convert is not None else x

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def _e4m3_table():
    # non-negative finite e4m3fn values for codes 0x00..0x7E, from the format
    codes = np.arange(0x7F)
    e, m = codes >> 3, (codes & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    return v


_E4M3 = _e4m3_table()


def to_e4m3(x: np.ndarray) -> np.ndarray:
    """float -> OCP e4m3fn code, round to nearest (ties to even code), saturating."""
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(x), 0x80, 0).astype(np.uint8)


def quantize_mx(x: np.ndarray, group: int = 32):
    """MXFP8 along the last axis: (e4m3 codes, E8M0 scale bytes [..., n/group]).

    Scale 2^e with the smallest e such that amax <= 448 * 2^e (no element
    saturates); with amax = m * 2^E, m in [0.5, 1): e = E - 9 if m <= 0.875
    else E - 8.  amax = 0 gives byte 0."""
    g = x.reshape(*x.shape[:-1], x.shape[-1] // group, group).astype(np.float64)
    amax = np.max(np.abs(g), axis=-1)
    m, E = np.frexp(amax)
    e = np.where(m <= 0.875, E - 9, E - 8)
    e = np.where(amax > 0, e, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    codes = to_e4m3(g / np.ldexp(1.0, e)[..., None]).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def quantize_groups(x: np.ndarray, axes):
    """Dynamic fp8 quantization with one scale per group (the reduced `axes`)."""
    amax = np.max(np.abs(x), axis=axes, keepdims=True).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = to_e4m3(x / scale)
    return codes, np.squeeze(scale, axis=axes)


# ---------------------------------------------------------------------------
# workload construction
# ---------------------------------------------------------------------------
def _seqmap(cfg):
    kind = cfg["kind"]
    if kind == "prefill":
        T = cfg["T"]
        lens = np.array([T], dtype=np.int32)
        q_seq = np.zeros(T, dtype=np.int32)
        q_pos = np.arange(T, dtype=np.int32)
    elif kind == "decode":
        ctx = cfg["ctx"]
        lens = np.array(ctx if isinstance(ctx, list) else [ctx] * cfg["B"], dtype=np.int32)
        q_seq = np.arange(len(lens), dtype=np.int32)
        q_pos = lens - 1
    elif kind == "zigzag":
        total, nseg, r = cfg["total"], cfg["segments"], cfg["rank"]
        L = total // nseg
        lens = np.array([total], dtype=np.int32)
        q_pos = np.concatenate([np.arange(r * L, (r + 1) * L),
                                np.arange((nseg - 1 - r) * L, (nseg - r) * L)]).astype(np.int32)
        q_seq = np.zeros(q_pos.shape[0], dtype=np.int32)
    elif kind == "chunked":
        lens = np.array(cfg["ctx"], dtype=np.int32)
        new = cfg["new"]
        q_seq = np.concatenate([np.full(n, b) for b, n in enumerate(new)]).astype(np.int32)
        q_pos = np.concatenate([np.arange(L - n, L) for L, n in zip(lens, new)]).astype(np.int32)
    else:
        raise ValueError(kind)
    pages_per_seq = (lens + PAGE - 1) // PAGE
    maxp = int(pages_per_seq.max())
    B = len(lens)
    P = B * maxp
    if cfg.get("identity_pages"):
        perm = np.arange(P, dtype=np.int32)
    else:
        perm = _rng(cfg["cid"], 5, 0).permutation(P).astype(np.int32)
    block_table = perm.reshape(B, maxp)
    return q_seq, q_pos, lens, block_table, P


def make_workload(name: str, mla=True, indexer=True, overrides=None) -> Workload:
    """Build the named workload as host (NumPy) arrays.  `overrides` replaces
    configuration keys (e.g. {"ctx": 8192} for a decode context sweep); the
    random streams stay those of the named configuration."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides or {})
    cid = cfg["cid"]
    q_seq, q_pos, lens, block_table, P = _seqmap(cfg)
    wl = Workload(name, cfg, q_seq, q_pos, lens, block_table, P)
    Tq = q_pos.shape[0]
    Hi, Di, H, Dc, Dr = cfg["Hi"], cfg["Di"], cfg["H"], cfg["Dc"], cfg["Dr"]

    if indexer:
        if cfg["idx_dtype"] == "mxfp8":
            qsc = np.empty((Tq, Hi, Di // 32), dtype=np.uint8)
            ksc = np.empty((P * PAGE, Di // 32), dtype=np.uint8)

            def qconv(x, r0):
                codes, e = quantize_mx(x)
                qsc[r0:r0 + x.shape[0]] = e
                return codes

            def kconv(x, r0):
                codes, e = quantize_mx(x)
                ksc[r0:r0 + x.shape[0]] = e
                return codes

            wl.iq = _draw_rows(cid, 0, Tq, (Hi, Di), "normal", convert=qconv, out_dtype=np.uint8)
            wl.ik = _draw_rows(cid, 1, P * PAGE, (Di,), "normal", convert=kconv,
                               out_dtype=np.uint8).reshape(P, PAGE, Di)
            wl.iq_scale, wl.ik_scale = qsc, ksc.reshape(P, PAGE, Di // 32)
        elif cfg["idx_dtype"] == "bf16":
            wl.iq = _draw_rows(cid, 0, Tq, (Hi, Di), "normal", convert=lambda x, r0: to_bf16_bits(x),
                               out_dtype=np.uint16)
            wl.ik = _draw_rows(cid, 1, P * PAGE, (Di,), "normal", convert=lambda x, r0: to_bf16_bits(x),
                               out_dtype=np.uint16).reshape(P, PAGE, Di)
        elif cfg["idx_dtype"] == "f32":
            wl.iq = _draw_rows(cid, 0, Tq, (Hi, Di), "normal")
            wl.ik = _draw_rows(cid, 1, P * PAGE, (Di,), "normal").reshape(P, PAGE, Di)
        else:
            qsc = np.empty(Tq, dtype=np.float32)
            ksc = np.empty(P * PAGE, dtype=np.float32)

            def qconv(x, r0):
                codes, s = quantize_groups(x, axes=(1, 2))     # one scale per token
                qsc[r0:r0 + x.shape[0]] = s
                return codes

            def kconv(x, r0):
                codes, s = quantize_groups(x, axes=(1,))       # one scale per key token
                ksc[r0:r0 + x.shape[0]] = s
                return codes

            wl.iq = _draw_rows(cid, 0, Tq, (Hi, Di), "normal", convert=qconv, out_dtype=np.uint8)
            wl.ik = _draw_rows(cid, 1, P * PAGE, (Di,), "normal", convert=kconv,
                               out_dtype=np.uint8).reshape(P, PAGE, Di)
            wl.iq_scale, wl.ik_scale = qsc, ksc.reshape(P, PAGE)
        wl.iw = _draw_rows(cid, 2, Tq, (Hi,), "uniform")

    if mla:
        D = Dc + Dr
        if cfg["kv_dtype"] == "f32":
            wl.q = _draw_rows(cid, 3, Tq, (H, D), "normal")
            wl.kv = _draw_rows(cid, 4, P * PAGE, (D,), "normal").reshape(P, PAGE, D)
        else:
            wl.q = _draw_rows(cid, 3, Tq, (H, D), "normal",
                              convert=lambda x, r0: to_bf16_bits(x), out_dtype=np.uint16)
            if cfg["kv_dtype"] == "bf16":
                wl.kv = _draw_rows(cid, 4, P * PAGE, (D,), "normal",
                                   convert=lambda x, r0: to_bf16_bits(x),
                                   out_dtype=np.uint16).reshape(P, PAGE, D)
            else:
                st, se = cfg["kv_scale"]
                assert PAGE % st == 0 and CHUNK % PAGE == 0 and Dc % se == 0
                ntile_tok = PAGE // st
                scales = np.empty((P * PAGE // st, Dc // se), dtype=np.float32)

                def kvconv(x, r0):
                    n = x.shape[0]
                    lat = x[:, :Dc].reshape(n // st, st, Dc // se, se)
                    codes, s = quantize_groups(lat, axes=(1, 3))   # [n/st, Dc/se]
                    scales[r0 // st:(r0 + n) // st] = s
                    row = np.empty((n, Dc + 2 * Dr), dtype=np.uint8)
                    row[:, :Dc] = codes.reshape(n, Dc)
                    row[:, Dc:] = to_bf16_bits(x[:, Dc:]).view(np.uint8).reshape(n, 2 * Dr)
                    return row

                wl.kv = _draw_rows(cid, 4, P * PAGE, (D,), "normal", convert=kvconv,
                                   out=np.empty((P * PAGE, Dc + 2 * Dr), dtype=np.uint8)
                                   ).reshape(P, PAGE, Dc + 2 * Dr)
                # [P, PAGE/st, Dc/se]: tile (page, token group, latent group)
                wl.kv_scale = scales.reshape(P, ntile_tok, Dc // se)
    return wl


def sample_rows(wl: Workload, n: int, K: int, boundary: int = 8192) -> np.ndarray:
    """Deterministic sample of query rows for full-size checks.

    Always holds: the first two and last two rows; the rows at q_pos = K-2..K
    (where a row starts to see more than K keys); the first three rows after
    every jump of q_pos inside a sequence (the start of a zigzag segment) and
    the row before it; for every multiple m of `boundary` (the key ranges and
    page chunks of the indexer kernels) the first rows at q_pos = m-1 and m;
    plus max(n - those, n // 2) rows evenly spaced over the whole batch."""
    Tq = wl.Tq
    if Tq <= n:
        return np.arange(Tq)
    pos = wl.q_pos.astype(np.int64)
    seq = wl.q_seq.astype(np.int64)
    s = {0, 1, Tq - 2, Tq - 1}
    s |= set(int(x) for x in np.nonzero(np.abs(pos - (K - 1)) <= 1)[0][:3])
    jumps = np.nonzero((seq[1:] == seq[:-1]) & (pos[1:] - pos[:-1] > 1))[0]
    for j in jumps[:8]:
        s |= {int(j), int(j) + 1, int(j) + 2, int(j) + 3}
    if len(np.unique(pos)) > 1:
        for m in range(boundary, int(pos.max()) + 2, boundary):
            for want in (m - 1, m):
                hit = np.nonzero(pos == want)[0]
                if hit.size:
                    s.add(int(hit[0]))
    rest = max(n - len(s), n // 2)
    s |= set(int(x) for x in np.linspace(0, Tq - 1, rest + 2)[1:-1].round())
    return np.array(sorted(x for x in s if 0 <= x < Tq))
