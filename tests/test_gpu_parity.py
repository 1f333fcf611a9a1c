"""GPU parity: each libsia entry point against the CPU oracle on the same
seeded inputs, at sizes the oracle finishes in seconds (several tiles, ragged
tails, short rows).  Full-size configurations are in test_gpu_fullsize.py."""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from sparse_index_attention_amd import sia
from sparse_index_attention_amd import workloads as W

from gpu_support import (ATT_TOL, LSE_ATOL, check_attention, check_scores, dev, kind_of, page_band_ok, page_max,
                         tie_band_ok, to_np_out, upload, workload)

pytestmark = pytest.mark.gpu

TINY = ["tiny_prefill", "decode_tiny", "prefill_tiny", "quant_decode_tiny", "quant_decode_tile128_tiny",
        "cp_chunk_prefill_tiny", "decode_h64_tiny", "chunked_prefill_tiny", "mx_decode_tiny", "mx_prefill_tiny",
        "bf16_decode_tiny", "bf16_prefill_tiny", "bf16_chunked_prefill_tiny"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sia.lib()


@functools.lru_cache(maxsize=16)
def oracle_run(name):
    wl = workload(name)
    K = wl.cfg["K"]
    sc = O.index_scores(wl.oracle_indexer(), wl.oracle_seq())
    sel = O.topk(sc, K, 0)
    att = O.sparse_mla(wl.q, wl.oracle_kv(), wl.oracle_seq(), sel, wl.softmax_scale)
    return sc, sel, att


def ld_of(wl):
    return (wl.max_visible + 3) // 4 * 4


@pytest.mark.parametrize("name", TINY)
def test_index_scores(name):
    wl = workload(name)
    print(f"[scores] {name}", flush=True)
    seq, ix, _, _ = upload(wl)
    scores = sia.index_scores(ix, seq, ld=ld_of(wl))
    torch.cuda.synchronize()
    got = scores.cpu().numpy()
    sc, _, _ = oracle_run(name)
    check_scores(wl, range(wl.Tq), got, sc)


def oracle_score_buffer(wl, sc, fill=np.nan):
    buf = np.full((wl.Tq, ld_of(wl)), fill, dtype=np.float32)
    for t, row in sc.items():
        buf[t, : row.shape[0]] = row
    return buf


@pytest.mark.parametrize("name", TINY)
@pytest.mark.parametrize("order", [0, 1])
def test_topk_bit_exact_on_oracle_scores(name, order):
    wl = workload(name)
    print(f"[topk] {name} order={order}", flush=True)
    K = wl.cfg["K"]
    seq, _, _, _ = upload(wl)
    sc, _, _ = oracle_run(name)
    buf = dev(oracle_score_buffer(wl, sc))          # NaN beyond q_pos: must never be read
    idx, vals = sia.topk(buf, seq, K, order=order, with_vals=True)
    torch.cuda.synchronize()
    idx, vals = idx.cpu().numpy(), vals.cpu().numpy()
    for t in range(wl.Tq):
        exp = O.topk_row(sc[t], K, order)
        assert np.array_equal(idx[t], exp), f"row {t}"
        m = exp >= 0
        assert np.all(vals[t][m] == sc[t][exp[m]]) and np.all(np.isneginf(vals[t][~m]))


def _topk_rows_case(rows, K, order, max_visible=None):
    T = len(rows)
    n_max = max(len(r) for r in rows)
    mv = max_visible or n_max
    ld = (mv + 3) // 4 * 4
    buf = np.full((T, ld), np.nan, dtype=np.float32)
    for t, r in enumerate(rows):
        buf[t, : len(r)] = r
    pages = (mv + 63) // 64
    seq = sia.SeqMap(dev(np.zeros(T, np.int32)), dev(np.array([len(r) - 1 for r in rows], np.int32)),
                     dev(np.arange(pages, dtype=np.int32)[None]), pages, mv)
    idx = sia.topk(dev(buf), seq, K, order=order)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for t, r in enumerate(rows):
        exp = O.topk_row(r, K, order)
        assert np.array_equal(idx[t], exp), f"case row {t} (n={len(r)}, K={K})"


def _synthetic_rows(seed, ns):
    rng = np.random.default_rng(seed)
    rows = []
    for i, n in enumerate(ns):
        kind = i % 6
        if kind == 0:
            r = rng.standard_normal(n)
        elif kind == 1:
            r = np.round(rng.standard_normal(n) * 3)            # heavy ties
        elif kind == 2:
            r = np.where(rng.random(n) < 0.5, 0.0, -0.0)         # only signed zeros
        elif kind == 3:
            r = np.full(n, 7.25)                                  # all equal
        elif kind == 4:
            r = rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, size=n)   # wide range
        else:
            r = np.maximum(rng.standard_normal(n), 0)             # ReLU-like: many exact zeros
        rows.append(r.astype(np.float32))
    return rows


@pytest.mark.parametrize("K", [1, 7, 64, 2048])
@pytest.mark.parametrize("order", [0, 1])
def test_topk_edge_cases_cached_rows(K, order):
    print(f"[topk-edge] K={K} order={order}", flush=True)
    ns = [1, 2, 5, 63, 64, 65, 1000, 2047, 2048, 2049, 5000, 32768, 12345, 3, 4096, 30000, 777, 2100]
    _topk_rows_case(_synthetic_rows(K * 10 + order, ns), K, order)


@pytest.mark.parametrize("order", [0, 1])
def test_topk_many_rows_of_every_length_class(order):
    """Calls with many rows send each row to the variant that holds its length
    (keys per thread 8, 32, 64, or streamed), one launch per class.  Every row
    must be handled by exactly one launch: no row keeps the sentinel the output
    was filled with, each is a valid selection (distinct visible positions,
    -1 padding), and two rows of every length equal the oracle bit for bit."""
    K = 2048
    lens = [0, 1, 100, 2048, 8192, 8193, 20000, 32768, 32769, 50000, 65536, 65537, 70001]
    T = 1200
    print(f"[topk-classes] order={order}: {T} rows", flush=True)
    n = np.array([lens[t % len(lens)] for t in range(T)], np.int64)
    mv = int(n.max())
    ld = (mv + 3) // 4 * 4
    rng = np.random.default_rng(77 + order)
    scores = torch.from_numpy(rng.standard_normal((T, ld), dtype=np.float32)).cuda()
    pages = (mv + 63) // 64
    seq = sia.SeqMap(dev(np.zeros(T, np.int32)), dev((n - 1).astype(np.int32)),
                     dev(np.arange(pages, dtype=np.int32)[None]), pages, mv)
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    sia.topk(scores, seq, K, order=order, idx=idx)
    torch.cuda.synchronize()
    ids = idx.cpu().numpy()
    for t in range(T):
        m = min(int(n[t]), K)
        row = ids[t]
        assert np.all(row[m:] == -1), f"row {t} (n={n[t]}): padding"
        sel = row[:m]
        assert np.all((sel >= 0) & (sel < n[t])) and len(np.unique(sel)) == m, f"row {t} (n={n[t]}): selection"
    sc = None
    for t in range(2 * len(lens)):
        if sc is None or t % 4 == 0:
            sc = scores[t: t + 4].cpu().numpy()
        exp = O.topk_row(sc[t % 4][: int(n[t])], K, order)
        assert np.array_equal(ids[t], exp), f"row {t} (n={n[t]})"


@pytest.mark.parametrize("order", [0, 1])
def test_topk_long_rows_uncached(order):
    print(f"[topk-long] order={order}", flush=True)
    ns = [70000, 40000, 1, 2048, 65536, 100003]
    _topk_rows_case(_synthetic_rows(99 + order, ns), 2048, order, max_visible=100003)


@pytest.mark.parametrize("name", TINY)
@pytest.mark.parametrize("entry", ["decode", "prefill"])
def test_sparse_mla_on_oracle_indices(name, entry):
    wl = workload(name)
    print(f"[mla] {name} {entry}", flush=True)
    K = wl.cfg["K"]
    seq, _, q, kv = upload(wl)
    _, sel, att = oracle_run(name)
    idx = dev(np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32))
    lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
    fn = sia.sparse_mla_decode if entry == "decode" else sia.sparse_mla_prefill
    out = fn(q, kv, seq, idx, K, wl.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    check_attention(kind_of(wl), to_np_out(out), lse.cpu().numpy(), att, range(wl.Tq))


@pytest.mark.parametrize("name", ["decode_tiny", "quant_decode_tiny", "prefill_tiny"])
def test_sparse_mla_holes_and_permuted_lists(name):
    """-1 holes anywhere in the list, positions in arbitrary order."""
    wl = workload(name)
    print(f"[mla-holes] {name}", flush=True)
    K = wl.cfg["K"]
    rng = np.random.default_rng(5)
    _, sel, _ = oracle_run(name)
    ids = np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32)
    for t in range(wl.Tq):
        rng.shuffle(ids[t])
        ids[t][rng.random(K) < 0.3] = -1
    sel2 = {t: ids[t] for t in range(wl.Tq)}
    att = O.sparse_mla(wl.q, wl.oracle_kv(), wl.oracle_seq(), sel2, wl.softmax_scale)
    seq, _, q, kv = upload(wl)
    lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        out = fn(q, kv, seq, dev(ids), K, wl.softmax_scale, lse=lse)
        torch.cuda.synchronize()
        check_attention(kind_of(wl), to_np_out(out), lse.cpu().numpy(), att, range(wl.Tq))


def test_sparse_mla_all_invalid_row_gives_zero_and_neg_inf():
    wl = workload("decode_tiny")
    K = wl.cfg["K"]
    seq, _, q, kv = upload(wl)
    ids = np.full((wl.Tq, K), -1, np.int32)
    ids[1, 3] = 0
    lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        out = fn(q, kv, seq, dev(ids), K, wl.softmax_scale, lse=lse)
        torch.cuda.synchronize()
        o, l = to_np_out(out), lse.cpu().numpy()
        assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
        row0 = O.kv_rows(wl.oracle_kv(), O.physical_slots(wl.block_table[1], np.array([0]), 64))
        assert np.allclose(o[1], np.broadcast_to(row0[:, :512], (wl.cfg["H"], 512)), atol=1e-2, rtol=1e-2)


@pytest.mark.parametrize("name", ["decode_tiny", "quant_decode_tiny", "prefill_tiny"])
def test_dense_causal_attention_when_K_covers_the_context(name):
    """Rows whose visible count is at most K select every visible position
    (exactly, whatever the scores), so the fused call reduces to dense causal
    MLA attention there.  The reference is a float64 softmax over all visible
    rows, taken here with torch from the decoded cache rows, not through the
    oracle's sparse attention."""
    wl = workload(name)
    K, H, Dc = wl.cfg["K"], wl.cfg["H"], wl.cfg["Dc"]
    rows = [t for t in range(wl.Tq) if int(wl.q_pos[t]) + 1 <= K]
    print(f"[dense] {name}: {len(rows)} rows with K >= context", flush=True)
    assert rows, "the workload should have rows that K covers"
    seq, ix, q, kv = upload(wl)
    idx = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    lse = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
    out = sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, order=1, idx_out=idx, lse=lse)
    torch.cuda.synchronize()
    ids, o, l = idx.cpu().numpy(), to_np_out(out), lse.cpu().numpy()
    kvd = wl.oracle_kv()
    qd = torch.from_numpy(O.decode_bf16(wl.q).astype(np.float64))
    atol, rtol = ATT_TOL[kind_of(wl)]
    for t in rows:
        n = int(wl.q_pos[t]) + 1
        # order 1: every visible position in ascending order, then -1
        assert np.array_equal(ids[t][:n], np.arange(n)) and np.all(ids[t][n:] == -1), f"row {t}: selection"
        b = int(wl.q_seq[t])
        kr = torch.from_numpy(O.kv_rows(kvd, O.physical_slots(wl.block_table[b], np.arange(n), 64)).astype(np.float64))
        logits = wl.softmax_scale * (qd[t] @ kr.T)                    # [H, n]
        ref = torch.softmax(logits, dim=1) @ kr[:, :Dc]               # [H, Dc]
        ref_lse = torch.logsumexp(logits, dim=1)
        err = np.abs(o[t] - ref.numpy())
        assert np.all(err <= atol + rtol * np.abs(ref.numpy())), f"row {t}: max err {err.max()}"
        assert np.all(np.abs(l[t] - ref_lse.numpy()) <= LSE_ATOL[kind_of(wl)] + 1e-4 * np.abs(ref_lse.numpy())), \
            f"row {t}: lse"


@pytest.mark.parametrize("name", TINY)
def test_index_select_attend_end_to_end(name):
    wl = workload(name)
    print(f"[fused] {name}", flush=True)
    K = wl.cfg["K"]
    seq, ix, q, kv = upload(wl)
    idx = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
    out = sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, order=0, idx_out=idx, lse=lse)
    torch.cuda.synchronize()
    sc, sel, att = oracle_run(name)
    ids, o, l = idx.cpu().numpy(), to_np_out(out), lse.cpu().numpy()
    matched = []
    for t in range(wl.Tq):
        assert tie_band_ok(sc[t], K, ids[t], sel[t]), f"row {t}: index sets differ beyond the tie band"
        if set(ids[t]) == set(sel[t]):
            matched.append(t)
    assert len(matched) >= 0.9 * wl.Tq
    check_attention(kind_of(wl), o[matched], l[matched], att, matched)


@pytest.mark.parametrize("name", ["decode_tiny", "prefill_tiny", "chunked_prefill_tiny", "cp_chunk_prefill_tiny"])
def test_deterministic_reruns(name):
    """Two runs of the fused call give the same indices and output bits
    (decode splits and the prefill score-matrix path alike)."""
    wl = workload(name)
    print(f"[determinism] {name}", flush=True)
    K = wl.cfg["K"]
    seq, ix, q, kv = upload(wl)
    res = []
    for _ in range(2):
        idx = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
        lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
        out = sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, idx_out=idx, lse=lse)
        torch.cuda.synchronize()
        bits = out.view(torch.int16) if out.dtype != torch.float32 else out.view(torch.int32)
        res.append((idx.cpu().numpy(), bits.cpu().numpy(), lse.view(torch.int32).cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


def test_side_stream_without_workspace():
    """Calls on a caller-given stream without a caller workspace: the binding
    allocates the workspace and outputs on that stream, so memory the current
    stream allocates meanwhile never aliases buffers the kernels still use."""
    print("[side-stream]", flush=True)
    wl = workload("decode_tiny")
    K, H = wl.cfg["K"], wl.cfg["H"]
    seq, ix, q, kv = upload(wl)
    ref_idx = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    ref = sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, idx_out=ref_idx)
    torch.cuda.synchronize()
    n_ws = sia.workspace_size(sia.OP_INDEX_SELECT_ATTEND, seq, K, H, wl.cfg["Dc"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        outs.append(sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, stream=side))
        outs.append(sia.index_topk(ix, seq, K, stream=side))
        # the current stream takes and scribbles over fresh memory of the workspace's size
        junk = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        junk.fill_(0xFF)
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k in range(0, len(outs), 2):
        assert torch.equal(outs[k].view(torch.int16), ref.view(torch.int16))
        assert torch.equal(outs[k + 1], ref_idx)


def test_permuted_block_table_matches_identity():
    """Moving pages around the pool (and the table with them) changes nothing."""
    wl = workload("prefill_tiny")
    K = wl.cfg["K"]
    seq, ix, q, kv = upload(wl)
    idx_a = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    out_a = sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, idx_out=idx_a)
    tbl = wl.block_table[0]
    ix2 = sia.Indexer(ix.q, ix.w, dev(wl.ik[tbl]), ix.q_scale, dev(wl.ik_scale[tbl]))
    kv2 = sia.LatentKV(dev(wl.kv[tbl]), 512, 64)
    seq2 = sia.SeqMap(seq.q_seq, seq.q_pos, dev(np.arange(len(tbl), dtype=np.int32)[None]), len(tbl),
                      wl.max_visible)
    idx_b = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    out_b = sia.index_select_attend(ix2, q, kv2, seq2, K, wl.softmax_scale, idx_out=idx_b)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))


def test_sparse_mla_pool_beyond_4gib():
    """A bf16 latent pool under 4 GiB is gathered through 32-bit buffer offsets,
    a larger one through 64-bit addresses.  The same pages placed at the top of
    a 4.4 GB pool (offsets past 2^32, every other page NaN) give bit-identical
    outputs, and both match the oracle."""
    wl = workload("decode_tiny")
    K, H = wl.cfg["K"], wl.cfg["H"]
    seq, _, q, kv = upload(wl)
    _, sel, att = oracle_run("decode_tiny")
    idx = dev(np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32))
    P = wl.kv.shape[0]
    big_pages = 60000   # 60000 x 64 rows x 1152 bytes = 4.42 GB
    assert big_pages * 64 * 1152 > 2**32 and P < big_pages
    base = big_pages - P
    print(f"[mla-big-pool] {P} pages placed at {base}..{big_pages - 1}", flush=True)
    # every page the table does not name holds NaN: rows without a valid index
    # must not read them
    big = torch.full((big_pages,) + tuple(kv.pool.shape[1:]), float("nan"), dtype=kv.pool.dtype, device="cuda")
    big[base:].copy_(kv.pool)
    kv_big = sia.LatentKV(big, 512, 64)
    seq_big = sia.SeqMap(seq.q_seq, seq.q_pos, seq.block_table + base, big_pages, wl.max_visible)
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        la = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
        lb = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
        a = fn(q, kv, seq, idx, K, wl.softmax_scale, lse=la)
        b = fn(q, kv_big, seq_big, idx, K, wl.softmax_scale, lse=lb)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), fn.__name__
        assert torch.equal(la, lb), fn.__name__
        check_attention("bf16", to_np_out(b), lb.cpu().numpy(), att, range(wl.Tq))
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["quant_decode_tiny", "quant_decode_tile128_tiny"])
def test_sparse_mla_fp8_pool_beyond_4gib(name):
    """fp8 latent pools (640-byte rows) under 4 GiB are gathered through
    buffer descriptors, larger ones through 64-bit addresses.  The same pages
    and scales placed at the top of a 4.4 GB pool (every other page and scale
    NaN) give bit-identical outputs, and both match the oracle."""
    wl = workload(name)
    K, H = wl.cfg["K"], wl.cfg["H"]
    seq, _, q, kv = upload(wl)
    _, sel, att = oracle_run(name)
    idx = dev(np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32))
    P = kv.pool.shape[0]
    big_pages = 105000   # 105000 x 64 rows x 640 bytes = 4.30 GB
    assert big_pages * 64 * 640 > 2**32 and P < big_pages
    base = big_pages - P
    print(f"[mla-big-pool-fp8] {name}: {P} pages placed at {base}..{big_pages - 1}", flush=True)
    big = torch.full((big_pages,) + tuple(kv.pool.shape[1:]), 0xFF, dtype=torch.uint8, device="cuda")  # NaN codes
    big[base:].copy_(kv.pool)
    sbig = torch.full((big_pages,) + tuple(kv.scale.shape[1:]), float("nan"), dtype=torch.float32, device="cuda")
    sbig[base:].copy_(kv.scale)
    kv_big = sia.LatentKV(big, 512, 64, sbig, kv.scale_tokens, kv.scale_elems)
    seq_big = sia.SeqMap(seq.q_seq, seq.q_pos, seq.block_table + base, big_pages, wl.max_visible)
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        la = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
        lb = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
        a = fn(q, kv, seq, idx, K, wl.softmax_scale, lse=la)
        b = fn(q, kv_big, seq_big, idx, K, wl.softmax_scale, lse=lb)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), fn.__name__
        assert torch.equal(la, lb), fn.__name__
        check_attention("fp8", to_np_out(b), lb.cpu().numpy(), att, range(wl.Tq))
    del big, sbig
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_tiny", "quant_decode_tiny", "prefill_tiny"])
def test_sparse_mla_padding_rows_ignore_pool_contents(name):
    """Index lists padded with -1 (and holes) must not depend on what the pool
    holds in the row such entries would address: a NaN page placed at
    physical page 0 (every real page moved up by one) leaves the outputs
    bit-identical."""
    wl = workload(name)
    K, H = wl.cfg["K"], wl.cfg["H"]
    seq, _, q, kv = upload(wl)
    _, sel, _ = oracle_run(name)
    ids = np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32)
    ids[:, 1::7] = -1   # holes as well as trailing padding
    idx = dev(ids)
    print(f"[mla-nan-page0] {name}: {int((ids < 0).sum())} padded entries", flush=True)
    if kv.pool.dtype == torch.uint8:   # fp8 codes 0xff and bf16 0xffff are NaN
        pool2 = torch.cat([torch.full_like(kv.pool[:1], 0xFF), kv.pool])
        scale2 = torch.cat([torch.full_like(kv.scale[:1], float("nan")), kv.scale])
        kv2 = sia.LatentKV(pool2, kv.latent_dim, kv.rope_dim, scale2, kv.scale_tokens, kv.scale_elems)
    else:
        pool2 = torch.cat([torch.full_like(kv.pool[:1], float("nan")), kv.pool])
        kv2 = sia.LatentKV(pool2, kv.latent_dim, kv.rope_dim)
    seq2 = sia.SeqMap(seq.q_seq, seq.q_pos, seq.block_table + 1, seq.num_pages + 1, wl.max_visible)
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        la = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
        lb = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
        a = fn(q, kv, seq, idx, K, wl.softmax_scale, lse=la)
        b = fn(q, kv2, seq2, idx, K, wl.softmax_scale, lse=lb)
        torch.cuda.synchronize()
        assert torch.isfinite(b.float()).all(), fn.__name__
        assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a,
                           b.view(torch.int16) if b.dtype != torch.float32 else b), fn.__name__
        assert torch.equal(la, lb), fn.__name__


def test_split_count_invariance():
    """Decode splits each token's rows over several workgroups and merges the
    partials (O_s rounded to bf16, lse_s in float32).  Merged on the host in
    float64 from the workspace, they give the decode output up to its one bf16
    rounding.  The one-workgroup prefill output agrees with that merge up to:
    the bf16 rounding of the output, of the partials (the merge is a convex
    combination, so at most 2^-9 of max_s |O_s|), and of the softmax weights
    that feed the P.V MFMA (relative 2^-9 per weight on each side; a split
    changes each weight's reference maximum and so its rounding: at most 2^-8
    of max_j |v_j| per column), beyond float32 summation order."""
    wl = workload("decode_tiny")
    K, H, Dc = wl.cfg["K"], wl.cfg["H"], wl.cfg["Dc"]
    seq, _, q, kv = upload(wl)
    _, sel, _ = oracle_run("decode_tiny")
    idx = dev(np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32))
    n_ws = sia.workspace_size(sia.OP_MLA_DECODE, seq, K, H, Dc)
    T = wl.Tq
    S = (n_ws - 256) // (T * H * (2 * Dc + 4))
    assert S >= 2 and n_ws == T * S * H * (2 * Dc + 4) + 256, "decode_tiny should split its rows"
    ws = torch.zeros(n_ws, dtype=torch.uint8, device="cuda")
    a = sia.sparse_mla_decode(q, kv, seq, idx, K, wl.softmax_scale, ws=ws).float()
    b = sia.sparse_mla_prefill(q, kv, seq, idx, K, wl.softmax_scale).float()
    torch.cuda.synchronize()
    nb = T * S * H * Dc * 2
    po = ws[:nb].view(torch.bfloat16).float().cpu().numpy().astype(np.float64).reshape(T, S, H, Dc)
    pl = ws[nb: nb + T * S * H * 4].view(torch.float32).cpu().numpy().astype(np.float64).reshape(T, S, H)
    m = np.max(pl, axis=1, keepdims=True)
    wgt = np.where(np.isfinite(pl), np.exp(pl - np.where(np.isfinite(m), m, 0.0)), 0.0)
    tot = wgt.sum(axis=1)
    live = wgt[..., None] > 0
    merged = np.einsum("tsh,tshd->thd", wgt, np.where(live, po, 0.0)) / np.where(tot > 0, tot, 1.0)[..., None]
    a, b = a.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64)
    out_round = 2.0 ** -8 * np.abs(merged)         # one bf16 rounding of the output
    assert np.all(np.abs(a - merged) <= out_round + 1e-6), np.max(np.abs(a - merged))
    part_round = 2.0 ** -9 * np.max(np.where(live, np.abs(po), 0.0), axis=1)
    vmax = np.zeros((T, 1, Dc))
    for t in range(T):
        ids = sel[t][sel[t] >= 0]
        rows = O.kv_rows(wl.oracle_kv(), O.physical_slots(wl.block_table[int(wl.q_seq[t])], ids, 64))
        vmax[t, 0] = np.max(np.abs(rows[:, :Dc]), axis=0)
    p_round = 2.0 ** -8 * vmax
    err = np.abs(b - merged)
    assert np.all(err <= out_round + part_round + p_round + 1e-5), np.max(err - out_round - part_round - p_round)
    print(f"[split-invariance] S={S}: decode vs merge {np.max(np.abs(a - merged)):.3g}, prefill vs merge "
          f"{np.max(err):.3g}", flush=True)


@pytest.mark.parametrize("name", ["decode_tiny", "prefill_tiny"])
def test_sparse_mla_wide_logit_range(name):
    """Logits spread over hundreds of units (softmax scale 6): later tiles
    exceed the first tile's maximum by far more than 2^100, which takes the
    kernels' second pass with the overall maximum as the softmax reference.
    (bf16 caches only: the fp8 path rounds dequantized latent values to bf16,
    an error that logits of this size amplify beyond the attention tolerance.)"""
    wl = workload(name)
    print(f"[mla-wide-logits] {name}", flush=True)
    K, H = wl.cfg["K"], wl.cfg["H"]
    scale = 6.0
    _, sel, _ = oracle_run(name)
    att = O.sparse_mla(wl.q, wl.oracle_kv(), wl.oracle_seq(), sel, scale)
    # the one-split entry sees the listed rows in order: check that some token's
    # later rows really exceed its first 32 rows' maximum by > 100 (log2 units)
    kvd, seqd = wl.oracle_kv(), wl.oracle_seq()
    triggered = 0
    for t in range(wl.Tq):
        ids = sel[t][sel[t] >= 0]
        if len(ids) <= 32:
            continue
        rows = O.kv_rows(kvd, O.physical_slots(seqd["block_table"][int(seqd["q_seq"][t])], ids, 64))
        qd = O.decode_bf16(wl.q[t]) if wl.q.dtype == np.uint16 else wl.q[t].astype(np.float64)
        lg = (qd @ rows.T) * scale / np.log(2.0)
        triggered += int(np.any(lg[:, 32:].max(axis=1) > lg[:, :32].max(axis=1) + 100.0))
    assert triggered > 0
    seq, _, q, kv = upload(wl)
    idx = dev(np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32))
    lse = torch.empty(wl.Tq, H, dtype=torch.float32, device="cuda")
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        out = fn(q, kv, seq, idx, K, scale, lse=lse)
        torch.cuda.synchronize()
        check_attention(kind_of(wl), to_np_out(out), lse.cpu().numpy(), att, range(wl.Tq))


# ---------------------------------------------------------------------------
# Indexer scores + Top-K in one call (scores never leave the chip on fp8 paths)

def _unfused_topk(ix, seq, K, order):
    sc = sia.index_scores(ix, seq)
    idx, vals = sia.topk(sc, seq, K, order=order, with_vals=True)
    return sc, idx, vals


@pytest.mark.parametrize("name", TINY)
@pytest.mark.parametrize("order", [0, 1])
def test_index_topk_matches_scores_then_topk(name, order):
    """Same ids and values as sia_index_scores followed by sia_topk."""
    wl = workload(name)
    print(f"[index-topk] {name} order={order}", flush=True)
    K = wl.cfg["K"]
    seq, ix, _, _ = upload(wl)
    _, e_idx, e_vals = _unfused_topk(ix, seq, K, order)
    methods = [sia.INDEX_TOPK_AUTO, sia.INDEX_TOPK_SCORES]
    if wl.cfg["idx_dtype"] in ("fp8", "mxfp8"):
        methods.append(sia.INDEX_TOPK_ONCHIP)
    for m in methods:
        g_idx, g_vals = sia.index_topk(ix, seq, K, order=order, method=m, with_vals=True)
        torch.cuda.synchronize()
        assert torch.equal(g_idx, e_idx), f"method {m}"
        assert torch.equal(g_vals, e_vals), f"method {m}"
    # and against the oracle's own selection, up to ties within the score tolerance
    sc, sel, _ = oracle_run(name)
    ids = g_idx.cpu().numpy()
    for t in range(wl.Tq):
        assert tie_band_ok(sc[t], K, ids[t], sel[t]), f"row {t}"


def _long_indexer(seed, lens, distinct, Hi=64):
    """One query at the end of each sequence; key rows drawn from `distinct`
    e4m3 rows (0: every row independent), so scores tie across whole ranges."""
    rng = np.random.default_rng(seed)
    pages = [(n + 63) // 64 for n in lens]
    P = sum(pages)
    perm = rng.permutation(P).astype(np.int32)
    table = np.zeros((len(lens), max(pages)), np.int32)
    o = 0
    for b, n in enumerate(pages):
        table[b, :n] = perm[o:o + n]
        o += n
    if distinct:
        base = W.to_e4m3(rng.standard_normal((distinct, 128)))
        k = base[rng.integers(0, distinct, size=(P, 64))]
        ks = np.ones((P, 64), np.float32)
    else:
        k = W.to_e4m3(rng.standard_normal((P, 64, 128)))
        ks = rng.uniform(0.5, 2.0, (P, 64)).astype(np.float32)
    T = len(lens)
    q = W.to_e4m3(rng.standard_normal((T, Hi, 128)))
    qs = rng.uniform(0.5, 1.5, T).astype(np.float32)
    w = rng.random((T, Hi)).astype(np.float32)
    seq = sia.SeqMap(dev(np.arange(T, dtype=np.int32)), dev(np.array(lens, np.int32) - 1), dev(table), P,
                     max(lens))
    return seq, sia.Indexer(dev(q), dev(w), dev(k), dev(qs), dev(ks))


@pytest.mark.parametrize("distinct", [3, 0])
@pytest.mark.parametrize("K", [1, 100, 2048])
@pytest.mark.parametrize("order", [0, 1])
def test_index_topk_across_ranges(distinct, K, order):
    """Rows spanning several 8192-key ranges, ragged last ranges, rows shorter
    than K, and exact ties across range boundaries (lowest positions win)."""
    print(f"[index-topk-long] distinct={distinct} K={K} order={order}", flush=True)
    lens = [1, 64, 2047, 8191, 8192, 8193, 16389, 40000]
    seq, ix = _long_indexer(1000 + distinct, lens, distinct)
    sc, e_idx, e_vals = _unfused_topk(ix, seq, K, order)
    g_idx, g_vals = sia.index_topk(ix, seq, K, order=order, method=sia.INDEX_TOPK_ONCHIP, with_vals=True)
    torch.cuda.synchronize()
    assert torch.equal(g_idx, e_idx)
    assert torch.equal(g_vals, e_vals)
    # the selection rule itself, on the GPU's scores
    sc, ids = sc.cpu().numpy(), g_idx.cpu().numpy()
    for t, n in enumerate(lens):
        assert np.array_equal(ids[t], O.topk_row(sc[t, :n], K, order)), f"row {t} (n={n})"


def test_index_scores_independent_of_batching():
    """A query's scores are the same bits whether it is scored with the other
    queries of its sequence (key pages shared between them) or alone; blocks
    of queries that span sequences included."""
    wl = workload("chunked_prefill_tiny")
    print("[scores-batching] chunked_prefill_tiny", flush=True)
    seq, ix, _, _ = upload(wl)
    ld = ld_of(wl)
    full = sia.index_scores(ix, seq, ld=ld)
    torch.cuda.synchronize()
    full = full.cpu().numpy()
    for t in [0, 1, 35, 36, 37, 38, 100, 166, 167, 168, 200, 243, 244, 245, 252, 253, 254]:
        r = slice(t, t + 1)
        s1 = sia.SeqMap(dev(wl.q_seq[r]), dev(wl.q_pos[r]), seq.block_table, seq.num_pages, seq.max_visible)
        ix1 = sia.Indexer(ix.q[r].contiguous(), ix.w[r].contiguous(), ix.k_pool, ix.q_scale[r].contiguous(),
                          ix.k_scale)
        one = sia.index_scores(ix1, s1, ld=ld)
        torch.cuda.synchronize()
        n = int(wl.q_pos[t]) + 1
        assert np.array_equal(one.cpu().numpy()[0, :n].view(np.uint32), full[t, :n].view(np.uint32)), f"row {t}"


@pytest.mark.parametrize("name", ["prefill_tiny", "chunked_prefill_tiny", "decode_tiny", "cp_chunk_prefill_tiny"])
def test_index_scores_never_write_past_max_visible(name):
    """Entries at s >= max_visible of a padded score buffer keep their contents
    (pages straddling max_visible are computed whole)."""
    wl = workload(name)
    print(f"[scores-bounds] {name}", flush=True)
    seq, ix, _, _ = upload(wl)
    mv = wl.max_visible
    ld = (mv + 3) // 4 * 4 + 132
    buf = torch.full((wl.Tq, ld), 12345.0, dtype=torch.float32, device="cuda")
    sia.index_scores(ix, seq, buf)
    torch.cuda.synchronize()
    tail = buf[:, mv:].cpu().numpy()
    assert np.all(tail == 12345.0), f"{int(np.sum(tail != 12345.0))} entries past max_visible written"
    # and the visible part is written
    got = buf.cpu().numpy()
    for t in range(wl.Tq):
        n = int(wl.q_pos[t]) + 1
        assert np.all(np.isfinite(got[t, :n])), f"row {t}"


# ---------------------------------------------------------------------------
# Dynamic Q quantization (bf16 queries -> fp8 per token / MXFP8 per 32)

def _bf16_queries(seed, T, Hi, Di=128):
    """N(0,1) draws at mixed magnitudes, a token of zeros, tiny and large values."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, Hi, Di)).astype(np.float32)
    x *= (10.0 ** rng.integers(-4, 4, size=(T, 1, 1))).astype(np.float32)
    x[1] = 0.0
    x[2, :, :32] = 0.0                                   # all-zero MX groups
    x[3] *= np.float32(1e-30)                            # subnormal-range values
    x[4, 0, 0] = 3.0e38                                  # near the bf16 maximum
    return W.to_bf16_bits(x)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("Hi", [32, 64])
def test_quantize_q_matches_oracle(mx, Hi):
    print(f"[quantize-q] mx={mx} Hi={Hi}", flush=True)
    bits = _bf16_queries(30 + Hi + mx, 37, Hi)
    kpool = torch.zeros(1, 64, 128, dtype=torch.uint8, device="cuda")
    kscale = torch.zeros(1, 64, 4, dtype=torch.uint8, device="cuda") if mx else torch.ones(1, 64, device="cuda")
    ix = sia.Indexer(dev(bits), torch.ones(37, Hi, device="cuda"), kpool, None, kscale)
    codes, scales = sia.quantize_indexer_q(ix)
    torch.cuda.synchronize()
    e_codes, e_scales = O.quantize_q_mx(bits) if mx else O.quantize_q_fp8(bits)
    assert np.array_equal(codes.cpu().numpy(), e_codes)
    if mx:
        assert np.array_equal(scales.cpu().numpy(), e_scales)
    else:
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), e_scales.view(np.uint32))


@pytest.mark.parametrize("name", ["decode_tiny", "mx_decode_tiny", "prefill_tiny", "mx_prefill_tiny"])
def test_bf16_queries_quantized_in_the_call(name):
    """index_topk / index_select_attend given bf16 queries equal the same calls
    given the oracle's quantization of them (ids bit for bit)."""
    wl = workload(name)
    print(f"[bf16-q] {name}", flush=True)
    K, Hi = wl.cfg["K"], wl.cfg["Hi"]
    mx = wl.cfg["idx_dtype"] == "mxfp8"
    seq, ix, q, kv = upload(wl)
    bits = _bf16_queries(40, wl.Tq, Hi)
    codes, sc = O.quantize_q_mx(bits) if mx else O.quantize_q_fp8(bits)
    ix_b = sia.Indexer(dev(bits), ix.w, ix.k_pool, None, ix.k_scale)
    ix_q = sia.Indexer(dev(codes), ix.w, ix.k_pool, dev(sc), ix.k_scale)
    for m in (sia.INDEX_TOPK_ONCHIP, sia.INDEX_TOPK_SCORES):
        a_ids, a_vals = sia.index_topk(ix_b, seq, K, method=m, with_vals=True)
        b_ids, b_vals = sia.index_topk(ix_q, seq, K, method=m, with_vals=True)
        torch.cuda.synchronize()
        assert torch.equal(a_ids, b_ids) and torch.equal(a_vals, b_vals), f"method {m}"
    ia = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    ib = torch.empty_like(ia)
    oa = sia.index_select_attend(ix_b, q, kv, seq, K, wl.softmax_scale, idx_out=ia)
    ob = sia.index_select_attend(ix_q, q, kv, seq, K, wl.softmax_scale, idx_out=ib)
    torch.cuda.synchronize()
    assert torch.equal(ia, ib) and torch.equal(oa.view(torch.int16), ob.view(torch.int16))


# ---------------------------------------------------------------------------
# Block-aligned selection: whole 64-position pages ranked by their best score

def _pages_K(wl):
    return max(64, wl.cfg["K"] // 64 * 64)


@pytest.mark.parametrize("name", TINY)
def test_topk_pages_bit_exact_on_oracle_scores(name):
    wl = workload(name)
    K = _pages_K(wl)
    print(f"[topk-pages] {name} K={K}", flush=True)
    seq, _, _, _ = upload(wl)
    sc, _, _ = oracle_run(name)
    buf = dev(oracle_score_buffer(wl, sc))          # NaN beyond q_pos: must never be read
    idx, vals = sia.topk_pages(buf, seq, K, with_vals=True)
    torch.cuda.synchronize()
    idx, vals = idx.cpu().numpy(), vals.cpu().numpy()
    for t in range(wl.Tq):
        exp = O.topk_pages_row(sc[t], K)
        assert np.array_equal(idx[t], exp), f"row {t}"
        m = exp >= 0
        pm = page_max(sc[t] + np.float32(0))
        assert np.array_equal(vals[t][m], pm[exp[m] // 64]) and np.all(np.isneginf(vals[t][~m]))


@pytest.mark.parametrize("K", [64, 192, 2048])
def test_topk_pages_edge_rows(K):
    print(f"[topk-pages-edge] K={K}", flush=True)
    ns = [1, 2, 63, 64, 65, 127, 128, 129, 1000, 2047, 2048, 2049, 5000, 32768, 12345, 4096, 30000, 777]
    rows = _synthetic_rows(K + 5, ns)
    T, mv = len(rows), max(ns)
    ld = (mv + 3) // 4 * 4
    buf = np.full((T, ld), np.nan, dtype=np.float32)
    for t, r in enumerate(rows):
        buf[t, : len(r)] = r
    pages = (mv + 63) // 64
    seq = sia.SeqMap(dev(np.zeros(T, np.int32)), dev(np.array([len(r) - 1 for r in rows], np.int32)),
                     dev(np.arange(pages, dtype=np.int32)[None]), pages, mv)
    idx = sia.topk_pages(dev(buf), seq, K)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for t, r in enumerate(rows):
        assert np.array_equal(idx[t], O.topk_pages_row(r, K)), f"row {t} (n={len(r)})"


def test_topk_pages_many_pages():
    """Rows of up to 600 000 positions (9375 pages): the page Top-K takes its
    streamed path."""
    print("[topk-pages-long]", flush=True)
    ns = [600000, 70000, 1, 4096 * 64 + 3, 123457]
    rows = _synthetic_rows(7, ns)
    T, mv = len(rows), max(ns)
    ld = (mv + 3) // 4 * 4
    buf = np.full((T, ld), np.nan, dtype=np.float32)
    for t, r in enumerate(rows):
        buf[t, : len(r)] = r
    pages = (mv + 63) // 64
    seq = sia.SeqMap(dev(np.zeros(T, np.int32)), dev(np.array([len(r) - 1 for r in rows], np.int32)),
                     dev(np.arange(pages, dtype=np.int32)[None]), pages, mv)
    idx = sia.topk_pages(dev(buf), seq, 2048)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for t, r in enumerate(rows):
        assert np.array_equal(idx[t], O.topk_pages_row(r, 2048)), f"row {t} (n={len(r)})"


@pytest.mark.parametrize("name", TINY)
def test_index_topk_and_attend_with_page_selection(name):
    """sia_index_topk and sia_index_select_attend with SELECT_PAGES: the same
    ids as scores -> sia_topk_pages on the GPU, the oracle's page selection up
    to page-score ties, and attention over the oracle's pages."""
    wl = workload(name)
    K = _pages_K(wl)
    print(f"[pages-fused] {name} K={K}", flush=True)
    seq, ix, q, kv = upload(wl)
    e_idx = sia.topk_pages(sia.index_scores(ix, seq), seq, K)
    for m in (sia.INDEX_TOPK_AUTO, sia.INDEX_TOPK_SCORES):
        g_idx = sia.index_topk(ix, seq, K, order=sia.SELECT_PAGES, method=m)
        torch.cuda.synchronize()
        assert torch.equal(g_idx, e_idx), f"method {m}"
    idx = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
    lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
    out = sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, order=sia.SELECT_PAGES, idx_out=idx,
                                  lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(idx, e_idx)
    sc, _, _ = oracle_run(name)
    sel = O.topk_pages(sc, K)
    ids, o, l = idx.cpu().numpy(), to_np_out(out), lse.cpu().numpy()
    matched = []
    for t in range(wl.Tq):
        assert page_band_ok(sc[t], K, ids[t], sel[t]), f"row {t}: page sets differ beyond the tie band"
        if np.array_equal(ids[t], sel[t]):
            matched.append(t)
    assert len(matched) >= 0.9 * wl.Tq
    att = O.sparse_mla(wl.q, wl.oracle_kv(), wl.oracle_seq(), {t: sel[t] for t in matched}, wl.softmax_scale)
    check_attention(kind_of(wl), o[matched], l[matched], att, matched)


@pytest.mark.parametrize("name", ["decode_tiny", "quant_decode_tiny", "decode_h64_tiny", "tiny_prefill"])
@pytest.mark.parametrize("K", [1, 33, 100])
def test_sparse_mla_ragged_row_counts(name, K):
    """Index lists whose length is not a multiple of the 32-row tile (a
    partial last tile, and a single row), both entry points."""
    wl = workload(name)
    print(f"[mla-ragged] {name} K={K}", flush=True)
    sc, _, _ = oracle_run(name)
    sel = {t: O.topk_row(sc[t], K, 0) for t in range(wl.Tq)}
    ids = np.stack([sel[t] for t in range(wl.Tq)]).astype(np.int32)
    att = O.sparse_mla(wl.q, wl.oracle_kv(), wl.oracle_seq(), sel, wl.softmax_scale)
    seq, _, q, kv = upload(wl)
    lse = torch.empty(wl.Tq, wl.cfg["H"], dtype=torch.float32, device="cuda")
    for fn in (sia.sparse_mla_decode, sia.sparse_mla_prefill):
        out = fn(q, kv, seq, dev(ids), K, wl.softmax_scale, lse=lse)
        torch.cuda.synchronize()
        check_attention(kind_of(wl), to_np_out(out), lse.cpu().numpy(), att, range(wl.Tq))


def test_zero_token_calls_are_noops():
    """Every entry point accepts an empty batch on real device buffers and
    leaves its outputs untouched."""
    print("[zero-tokens]", flush=True)
    wl = workload("decode_tiny")
    seq_full, ix, q, kv = upload(wl)
    empty_i = torch.empty(0, dtype=torch.int32, device="cuda")
    seq = sia.SeqMap(empty_i, empty_i, seq_full.block_table, seq_full.num_pages, seq_full.max_visible)
    K = wl.cfg["K"]
    ix0 = sia.Indexer(ix.q[:0], ix.w[:0], ix.k_pool, ix.q_scale[:0], ix.k_scale)
    sentinel = torch.full((1, 8), 7.0, device="cuda")
    sc = sia.index_scores(ix0, seq, scores=sentinel, ld=8)
    assert sc.shape[0] == 1 and bool((sentinel == 7.0).all())
    assert sia.topk(sentinel, seq, K).shape == (0, K)
    assert sia.topk_pages(sentinel, seq, 64).shape == (0, 64)
    assert sia.index_topk(ix0, seq, K).shape == (0, K)
    out = sia.sparse_mla_decode(q[:0], kv, seq, empty_i.view(0, 1).expand(0, K).contiguous(), K, wl.softmax_scale)
    assert out.shape[0] == 0
    out = sia.index_select_attend(ix0, q[:0], kv, seq, K, wl.softmax_scale)
    assert out.shape[0] == 0
    torch.cuda.synchronize()
