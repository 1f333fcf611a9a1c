"""Pins for the CPU oracle: each oracle function is checked against something
other than itself (library routines, closed forms, brute force, invariants).

These tests run on the CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from sparse_index_attention_amd import workloads as W


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def test_e4m3_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2                       # 0x7F and 0xFF only


def test_e4m3_landmarks():
    """Format landmarks from tests/golden/e4m3_landmarks.txt (largest finite,
    one, smallest normal and subnormal, signed zeros, NaN)."""
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3_landmarks.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    codes = np.array([int(c, 16) for c, _ in rows], dtype=np.uint8)
    got = O.decode_e4m3(codes)
    for (c, want), g in zip(rows, got):
        if want == "nan":
            assert np.isnan(g), c
        else:
            w = float(want)
            assert g == w and np.signbit(g) == want.startswith("-"), (c, g, want)


def test_bf16_vs_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]     # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.decode_bf16(bits), ref)


def test_generator_codes_decode_near_input():
    # the workload quantizer and the oracle decoder agree within half an fp8 step
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    codes, sc = W.quantize_groups(x, axes=(1,))
    back = O.decode_e4m3(codes) * sc[:, None]
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -4 + sc[:, None] * 2 ** -9 + 1e-12)


# ---------------------------------------------------------------------------
# scores
# ---------------------------------------------------------------------------
def _brute_scores(q, qs, w, k, ks):
    Hi, Di = q.shape
    out = []
    for s in range(k.shape[0]):
        tot = 0.0
        for h in range(Hi):
            dot = math.fsum(float(q[h, d]) * float(k[s, d]) for d in range(Di))
            tot += float(w[h]) * max(0.0, float(qs[h]) * float(ks[s]) * dot)
        out.append(tot)
    return np.array(out)


def test_scores_brute_force_small():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 5))
    k = rng.standard_normal((9, 5))
    w = rng.random(3)
    qs = np.full(3, 0.7)
    ks = rng.random(9) + 0.1
    got = O.index_scores_row(q, qs, w, k, ks)
    assert np.allclose(got, _brute_scores(q, qs, w, k, ks), rtol=1e-12, atol=1e-12)


def test_scores_single_head_is_relu_matmul():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((40, 16))
    ref = torch.relu(torch.from_numpy(k) @ torch.from_numpy(q[0])).numpy()
    got = O.index_scores_row(q, np.ones(1), np.ones(1), k, np.ones(40))
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_scores_worked_case_unit_vectors():
    # q[h] = c_h e0, k = e0, unit scales: I = sum_h w_h max(c_h, 0)
    c = np.array([2.0, -1.0, 0.5, 3.0])
    w = np.array([0.25, 4.0, 2.0, 1.0])
    q = np.zeros((4, 8)); q[:, 0] = c
    k = np.zeros((1, 8)); k[0, 0] = 1.0
    got = O.index_scores_row(q, np.ones(4), w, k, np.ones(1))
    assert got[0] == 0.25 * 2.0 + 2.0 * 0.5 + 3.0      # = 4.5


def test_scores_scales_linear_and_nonnegative():
    rng = np.random.default_rng(4)
    q, k, w = rng.standard_normal((4, 8)), rng.standard_normal((20, 8)), rng.random(4)
    base = O.index_scores_row(q, np.ones(4), w, k, np.ones(20))
    assert np.all(base >= 0)
    scaled = O.index_scores_row(q, np.full(4, 2.0), w, k, np.full(20, 3.0))
    assert np.allclose(scaled, 6.0 * base)
    assert np.allclose(O.index_scores_row(q, np.ones(4), 2 * w, k, np.ones(20)), 2 * base)
    w2 = rng.random(4)
    assert np.allclose(O.index_scores_row(q, np.ones(4), w + w2, k, np.ones(20)),
                       base + O.index_scores_row(q, np.ones(4), w2, k, np.ones(20)))


def test_scores_paged_causal_rows_match_brute_force():
    wl = W.make_workload("tiny_prefill", mla=False)
    rows = [0, 1, 37, 63, 64, 200, 255]
    sc = O.index_scores(wl.oracle_indexer(), wl.oracle_seq(), rows)
    for t in rows:
        assert sc[t].shape == (t + 1,) and sc[t].dtype == np.float32
        slots = [wl.block_table[0][s // 64] * 64 + s % 64 for s in range(t + 1)]
        k = wl.ik.reshape(-1, 32)[slots].astype(np.float64)
        ref = _brute_scores(wl.iq[t].astype(np.float64), np.ones(4), wl.iw[t], k, np.ones(t + 1))
        assert np.array_equal(sc[t], ref.astype(np.float32))


def test_scores_fp8_rows_use_both_scales():
    wl = W.make_workload("decode_tiny", mla=False)
    t = 3
    sc = O.index_scores(wl.oracle_indexer(), wl.oracle_seq(), [t])[t]
    pos = wl.q_pos[t]
    s_list = [0, 17, pos]
    for s in s_list:
        slot = wl.block_table[t][s // 64] * 64 + s % 64
        kk = O.decode_e4m3(wl.ik.reshape(-1, 128)[slot])
        ks = float(wl.ik_scale.reshape(-1)[slot])
        qq = O.decode_e4m3(wl.iq[t])
        ref = _brute_scores(qq, np.full(64, wl.iq_scale[t]), wl.iw[t], kk[None], np.array([ks]))[0]
        assert sc[s] == np.float32(ref)


def test_e8m0_landmarks():
    """Shared-scale landmarks from tests/golden/e8m0_landmarks.txt."""
    path = os.path.join(os.path.dirname(__file__), "golden", "e8m0_landmarks.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        code, val = line.split()
        got = O.decode_e8m0(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)


def _brute_mx_scores(qc, qe, w, kc, ke):
    """MXFP8 scores by explicit loops: element d of a row is decode(code) *
    2^(e[d // 32] - 127)."""
    def val(c, e, d):
        return float(O.decode_e4m3(np.array([c], dtype=np.uint8))[0]) * math.ldexp(1.0, int(e[d // 32]) - 127)
    Hi, Di = qc.shape
    out = []
    for s in range(kc.shape[0]):
        tot = 0.0
        for h in range(Hi):
            dot = math.fsum(val(qc[h, d], qe[h], d) * val(kc[s, d], ke[s], d) for d in range(Di))
            tot += float(w[h]) * max(0.0, dot)
        out.append(tot)
    return np.array(out)


def _mx_inputs(rng, Hi, n, Di=64):
    codes = lambda shape: np.where(rng.random(shape) < 0.5, 0, 0x80).astype(np.uint8) | \
        rng.integers(0, 0x7f, size=shape).astype(np.uint8)        # finite e4m3 codes of both signs
    return (codes((Hi, Di)), rng.integers(110, 140, size=(Hi, Di // 32)).astype(np.uint8), rng.random(Hi),
            codes((n, Di)), rng.integers(110, 140, size=(n, Di // 32)).astype(np.uint8))


def test_mx_scores_brute_force_small():
    rng = np.random.default_rng(11)
    qc, qe, w, kc, ke = _mx_inputs(rng, 3, 7)
    idx = dict(q=qc[None], q_mx=qe[None], w=w[None], k=kc[None], k_mx=ke[None])
    seq = dict(q_seq=np.zeros(1, np.int32), q_pos=np.array([6], np.int32), block_table=np.zeros((1, 1), np.int64),
               page_size=64)
    got = O.index_scores(idx, seq)[0]
    ref = _brute_mx_scores(qc, qe, w, kc, ke)
    assert np.array_equal(got, ref.astype(np.float32))


def test_mx_with_one_exponent_per_row_is_per_token_fp8():
    """When every group of a query head shares one exponent (and of a key), MXFP8
    scores equal the per-token fp8 scores with those powers of two as scales."""
    rng = np.random.default_rng(12)
    qc, _, w, kc, _ = _mx_inputs(rng, 4, 9)
    eq = rng.integers(120, 135, size=4)
    ek = rng.integers(120, 135, size=9)
    qe = np.repeat(eq[:, None], 2, axis=1).astype(np.uint8)
    ke = np.repeat(ek[:, None], 2, axis=1).astype(np.uint8)
    mx = O.index_scores_row(O.mx_values(qc, qe), np.ones(4), w, O.mx_values(kc, ke), np.ones(9))
    fp8 = O.index_scores_row(O.decode_e4m3(qc), np.ldexp(1.0, eq - 127), w, O.decode_e4m3(kc), np.ldexp(1.0, ek - 127))
    assert np.allclose(mx, fp8, rtol=1e-14, atol=0)


def test_mx_group_scales_apply_to_their_32_elements():
    """Raising the exponent of one group of a key doubles exactly that group's
    contribution: q = e4m3 1.0 everywhere, k = 1.0 in group 0 and 2.0 in group 1."""
    Di = 64
    qc = np.full((1, Di), 0x38, np.uint8)                 # 1.0
    kc = np.full((1, Di), 0x38, np.uint8)
    qe = np.full((1, 2), 127, np.uint8)
    ke = np.array([[127, 128]], np.uint8)                 # group 1 scaled by 2
    got = O.index_scores_row(O.mx_values(qc, qe), np.ones(1), np.ones(1), O.mx_values(kc, ke), np.ones(1))
    assert got[0] == 32 * 1.0 + 32 * 2.0


def test_mx_generator_roundtrip():
    """Generated MXFP8 data decodes to within one e4m3 step of the draw and never saturates."""
    x = np.random.default_rng(13).standard_normal((200, 128)).astype(np.float32)
    codes, e = W.quantize_mx(x)
    back = O.mx_values(codes, e)
    scale = np.repeat(O.decode_e8m0(e), 32, axis=-1)
    assert np.all(np.abs(O.decode_e4m3(codes)) <= 448)
    assert np.all(np.abs(back - x) <= np.maximum(np.abs(x) * 2.0 ** -4, scale * 2.0 ** -9) + 1e-12)
    amax = np.max(np.abs(x.reshape(200, 4, 32)), axis=-1)
    s = O.decode_e8m0(e)
    assert np.all(amax <= 448 * s) and np.all(amax > 224 * s)   # the smallest power of two that fits


def test_bf16_indexer_rows_brute_force():
    """bfloat16 queries and keys: the score of the exact decoded values, no scales."""
    wl = W.make_workload("bf16_decode_tiny", mla=False)
    t = 2
    sc = O.index_scores(wl.oracle_indexer(), wl.oracle_seq(), [t])[t]
    qv = O.decode_bf16(wl.iq[t])
    assert np.array_equal(qv.astype(np.float32), qv)                     # bf16 values are exact in f32
    for s in [0, 1, 63, 64, int(wl.q_pos[t])]:
        slot = wl.block_table[t][s // 64] * 64 + s % 64
        kk = O.decode_bf16(wl.ik.reshape(-1, 128)[slot])
        ref = _brute_scores(qv, np.ones(64), wl.iw[t], kk[None], np.ones(1))[0]
        assert sc[s] == np.float32(ref)


def test_encode_e4m3_grid_ties_and_saturation():
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]
    assert np.array_equal(O.encode_e4m3(O.decode_e4m3(finite)), finite)        # every value maps to its code
    # midpoints between neighbours round to the even code
    for c in range(0x00, 0x7E):
        mid = (O.decode_e4m3(np.uint8(c)) + O.decode_e4m3(np.uint8(c + 1))) / 2
        assert O.encode_e4m3(mid) == (c if c % 2 == 0 else c + 1), c
    assert O.encode_e4m3(1e6) == 0x7E and O.encode_e4m3(-500.0) == 0xFE and O.encode_e4m3(460.0) == 0x7E
    assert O.encode_e4m3(2.0 ** -11) == 0x00 and O.encode_e4m3(-0.0) == 0x80


def _bf16_bits(x):
    return W.to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_quantize_q_fp8_per_token():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, 4, 32)).astype(np.float32) * np.array([1, 10, 0.01, 1e-3, 0])[:, None, None]
    bits = _bf16_bits(x)
    codes, scale = O.quantize_q_fp8(bits)
    xv = O.decode_bf16(bits)
    for t in range(4):
        amax = np.max(np.abs(xv[t]))
        assert scale[t] == np.float32(np.float32(amax) / np.float32(448))
        back = O.decode_e4m3(codes[t]) * scale[t]
        assert np.max(np.abs(O.decode_e4m3(codes[t]))) == 448.0                  # the extreme element hits the top
        assert np.all(np.abs(back - xv[t]) <= np.abs(xv[t]) * 2.0 ** -4 + scale[t] * 2.0 ** -10 + 1e-30)
    assert scale[4] == 1.0 and np.all(O.decode_e4m3(codes[4]) == 0)


def test_quantize_q_mx_scale_rule_brute_force():
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((3, 2, 64)) * 10.0 ** rng.integers(-6, 6, size=(3, 2, 1))).astype(np.float32)
    x[2, 1, 32:] = 0.0
    bits = _bf16_bits(x)
    codes, e8 = O.quantize_q_mx(bits)
    xv = O.decode_bf16(bits).reshape(3, 2, 2, 32)
    for idx in np.ndindex(3, 2, 2):
        amax = np.max(np.abs(xv[idx]))
        if amax == 0:
            assert e8[idx] == 0
            continue
        e = next(k for k in range(-140, 140) if amax <= 448 * 2.0 ** k)   # smallest fitting power of two
        assert int(e8[idx]) == e + 127
        c = codes.reshape(3, 2, 2, 32)[idx]
        assert np.array_equal(c, O.encode_e4m3(xv[idx] * 2.0 ** -e))


# ---------------------------------------------------------------------------
# Top-K
# ---------------------------------------------------------------------------
def _brute_topk(s, K):
    order = sorted(range(len(s)), key=lambda i: (-float(s[i]), i))
    out = order[:K] + [-1] * max(0, K - len(s))
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("n,K", [(1, 4), (7, 7), (50, 8), (300, 32), (33, 32)])
def test_topk_vs_sorted_bruteforce(n, K):
    rng = np.random.default_rng(n * 31 + K)
    s = rng.standard_normal(n).astype(np.float32)
    s[rng.integers(0, n, size=n // 3)] = 0.0            # ties
    assert np.array_equal(O.topk_row(s, K), _brute_topk(s, K))


def test_topk_negative_zero_ties_to_lower_position():
    s = np.array([1.0, -0.0, 0.0, -0.0, 2.0, -1.0], dtype=np.float32)
    assert list(O.topk_row(s, 4)) == [4, 0, 1, 2]
    assert list(O.topk_row(s, 4, order=1)) == [0, 1, 2, 4]


def test_topk_invariants():
    rng = np.random.default_rng(5)
    s = np.round(rng.standard_normal(500) * 4).astype(np.float32)   # many ties
    for K in (1, 16, 100, 499, 500, 600):
        idx = O.topk_row(s, K)
        sel = idx[idx >= 0]
        assert len(sel) == min(K, 500) and len(set(sel)) == len(sel)
        assert np.all((sel >= 0) & (sel < 500))
        unsel = np.setdiff1d(np.arange(500), sel)
        for j in sel[:50]:
            better = (s[unsel] > s[j]) | ((s[unsel] == s[j]) & (unsel < j))
            assert not better.any()
    small, big = O.topk_row(s, 50), O.topk_row(s, 200)
    assert set(small) <= set(big)
    assert np.array_equal(np.sort(O.topk_row(s, 77)), O.topk_row(s, 77, order=1))


# ---------------------------------------------------------------------------
# block-aligned selection ([P3, section 3.1]; block score = the largest score
# among the block's visible positions, a reading)
# ---------------------------------------------------------------------------
def _brute_pages(s, K, page):
    """Block selection by rank counting with plain loops: block b is kept when
    fewer than K/page blocks beat it (higher best score, or equal and lower)."""
    n = len(s)
    nb = (n + page - 1) // page
    best = []
    for b in range(nb):
        m = None
        for i in range(b * page, min(n, b * page + page)):
            v = float(s[i]) + 0.0
            m = v if m is None or v > m else m
        best.append(m)
    out = []
    for b in range(nb):
        beaten_by = sum(1 for c in range(nb) if best[c] > best[b] or (best[c] == best[b] and c < b))
        if beaten_by < K // page:
            out.extend(range(b * page, min(n, b * page + page)))
    return np.array(out + [-1] * (K - len(out)), dtype=np.int32)


@pytest.mark.parametrize("n,K,page", [(1, 4, 4), (10, 8, 4), (37, 12, 4), (64, 16, 8), (130, 64, 64),
                                      (200, 64, 16), (1000, 128, 64)])
def test_topk_pages_vs_rank_counting(n, K, page):
    rng = np.random.default_rng(n * 7 + K + page)
    s = np.round(rng.standard_normal(n) * 3).astype(np.float32)     # many ties
    assert np.array_equal(O.topk_pages_row(s, K, page), _brute_pages(s, K, page))


def test_topk_pages_worked_case_max_not_sum():
    # four blocks of 4: maxima 9, 5, 8, 1 and sums 9, 20, 8, 4.  Two blocks are
    # kept: by the maximum blocks 0 and 2; a sum rule would keep 1 and 0, and the
    # per-position Top-8 would mix all four blocks.
    s = np.array([0, 0, 0, 9, 5, 5, 5, 5, 8, 0, 0, 0, 1, 1, 1, 1], dtype=np.float32)
    assert list(O.topk_pages_row(s, 8, 4)) == [0, 1, 2, 3, 8, 9, 10, 11]
    assert sorted(O.topk_row(s, 8)) != [0, 1, 2, 3, 8, 9, 10, 11]


def test_topk_pages_partial_last_block_and_ties():
    # 10 visible positions in blocks of 4: the last block holds positions 8, 9
    s = np.array([1, 1, 1, 1, 0, 0, 0, 0, 3, 2], dtype=np.float32)
    assert list(O.topk_pages_row(s, 8, 4)) == [0, 1, 2, 3, 8, 9, -1, -1]
    # equal block maxima (including -0.0 against +0.0) go to the lower block
    t = np.array([0, -0.0, 0, 0, 0, 0, 0, 0, -0.0, -0.0, 0, 0], dtype=np.float32)
    assert list(O.topk_pages_row(t, 4, 4)) == [0, 1, 2, 3]
    assert list(O.topk_pages_row(t, 8, 4)) == [0, 1, 2, 3, 4, 5, 6, 7]


def test_topk_pages_block_of_one_is_position_topk():
    rng = np.random.default_rng(11)
    for n, K in ((1, 1), (9, 4), (300, 32), (50, 64)):
        s = np.round(rng.standard_normal(n) * 2).astype(np.float32)
        assert np.array_equal(O.topk_pages_row(s, K, 1), O.topk_row(s, K, order=1))


def test_topk_pages_invariants():
    rng = np.random.default_rng(12)
    page = 64
    for n in (1, 63, 64, 65, 2047, 2048, 2049, 5000):
        s = rng.standard_normal(n).astype(np.float32)
        for K in (64, 256, 2048):
            idx = O.topk_pages_row(s, K, page)
            sel = idx[idx >= 0]
            assert np.all(idx[len(sel):] == -1)                      # padding trails
            assert np.all(np.diff(sel) > 0) and np.all(sel < n)      # ascending, visible
            blocks = np.unique(sel // page)
            assert len(blocks) == min(K // page, -(-n // page))
            for b in blocks:                                         # whole blocks
                assert np.array_equal(sel[sel // page == b], np.arange(b * page, min(n, b * page + page)))
            if n <= K:
                assert np.array_equal(sel, np.arange(n))
            best = np.array([s[b * page: b * page + page].max() for b in range(-(-n // page))])
            kept_min = best[blocks].min()
            others = np.setdiff1d(np.arange(len(best)), blocks)
            assert not np.any(best[others] > kept_min)
            # the block holding the best position is always kept
            assert int(np.argmax(s)) in set(sel.tolist())


# ---------------------------------------------------------------------------
# sparse MLA
# ---------------------------------------------------------------------------
def test_mla_dense_equals_sdpa_when_K_covers_context():
    rng = np.random.default_rng(6)
    T, H, Dc, Dr = 40, 4, 16, 8
    q = rng.standard_normal((T, H, Dc + Dr))
    kv = rng.standard_normal((T, Dc + Dr))
    scale = 1 / math.sqrt(Dc + Dr)
    seq = dict(q_seq=np.zeros(T, np.int32), q_pos=np.arange(T, dtype=np.int32),
               block_table=np.arange(1, dtype=np.int32)[None], page_size=64)
    kvd = dict(pool=kv.reshape(1, T, Dc + Dr), dtype="f32", Dc=Dc, Dr=Dr, page_size=64)
    sel = {t: O.topk_row(np.zeros(t + 1, np.float32), 64) for t in range(T)}
    kvp = np.zeros((1, 64, Dc + Dr)); kvp[0, :T] = kv
    kvd["pool"] = kvp
    res = O.sparse_mla(q, kvd, seq, sel, scale)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                 # [1,H,T,D]
    kt = torch.from_numpy(kv)[None, None].expand(1, H, T, Dc + Dr)
    vt = torch.from_numpy(kv[:, :Dc])[None, None].expand(1, H, T, Dc)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    logits = torch.einsum("htd,sd->hts", torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(kv)) * scale
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    lse_ref = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1).numpy()  # [H,T]
    for t in range(T):
        assert np.allclose(res[t][0], ref[t], rtol=1e-12, atol=1e-12)
        assert np.allclose(res[t][1], lse_ref[:, t], rtol=1e-12, atol=1e-12)


def test_mla_single_row_and_constant_values():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 10))
    row = rng.standard_normal((1, 10))
    out, lse = O.sparse_mla_row(q, row, 6, 0.3)
    assert np.array_equal(out, np.broadcast_to(row[:, :6], (3, 6)))
    assert np.allclose(lse, 0.3 * (q @ row[0]))
    rows = np.ones((25, 10)); rows[:, 6:] = rng.standard_normal((25, 4))
    out, _ = O.sparse_mla_row(q, rows, 6, 0.3)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-14)


def test_mla_permutation_invariant_and_merge():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((5, 12))
    rows = rng.standard_normal((30, 12))
    out, lse = O.sparse_mla_row(q, rows, 8, 0.5)
    p = rng.permutation(30)
    out2, lse2 = O.sparse_mla_row(q, rows[p], 8, 0.5)
    assert np.allclose(out, out2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)
    parts = [O.sparse_mla_row(q, rows[a:b], 8, 0.5) for a, b in [(0, 7), (7, 8), (8, 8), (8, 30)]]
    mo, ml = O.merge_partials([x[0] for x in parts], [x[1] for x in parts])
    assert np.allclose(mo, out, atol=1e-13) and np.allclose(ml, lse, atol=1e-13)


def test_mla_empty_selection():
    out, lse = O.sparse_mla_row(np.ones((2, 4)), np.zeros((0, 4)), 3, 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_kv_fp8_tiles_brute_force():
    for name in ("quant_decode_tiny", "quant_decode_tile128_tiny"):
        wl = W.make_workload(name, indexer=False)
        kv = wl.oracle_kv()
        st, se = wl.cfg["kv_scale"]
        rng = np.random.default_rng(9)
        slots = rng.integers(0, wl.num_pages * 64, size=12)
        got = O.kv_rows(kv, slots)
        for r, slot in enumerate(slots):
            p, i = divmod(int(slot), 64)
            raw = wl.kv[p, i]
            for d in (0, 1, 127, 128, 300, 511):
                sc = wl.kv_scale[p, i // st, d // se]
                assert got[r, d] == O.decode_e4m3(raw[d:d + 1])[0] * float(sc)
            rope = torch.from_numpy(raw[512:].copy().view(np.int16)).view(torch.bfloat16)
            assert np.array_equal(got[r, 512:], rope.to(torch.float64).numpy())


def test_kv_fp8_closed_form_page():
    # every code 1.0 (0x38) with page scale 2 -> latent 2; rope bf16 1.5 (0x3FC0)
    pool = np.zeros((2, 64, 512 + 128), np.uint8)
    pool[:, :, :512] = 0x38
    pool[:, :, 512:] = np.frombuffer(np.full(64, 0x3FC0, np.uint16).tobytes(), np.uint8)
    kv = dict(pool=pool, dtype="fp8", Dc=512, Dr=64, page_size=64,
              scale=np.array([2.0, 0.5], np.float32).reshape(2, 1, 1), scale_tokens=64, scale_elems=512)
    rows = O.kv_rows(kv, np.array([5, 64 + 9]))
    assert np.all(rows[0, :512] == 2.0) and np.all(rows[1, :512] == 0.5)
    assert np.all(rows[:, 512:] == 1.5)


# ---------------------------------------------------------------------------
# paging and the zigzag chunk
# ---------------------------------------------------------------------------
def test_paging_identity_vs_permuted_tables():
    wl = W.make_workload("tiny_prefill")
    idx, seq, kv = wl.oracle_indexer(), wl.oracle_seq(), wl.oracle_kv()
    # rebuild the pools so logical page i sits at physical page i
    tbl = wl.block_table[0]
    idx2 = dict(idx, k=wl.ik[tbl])
    kv2 = dict(kv, pool=wl.kv[tbl])
    seq2 = dict(seq, block_table=np.arange(len(tbl), dtype=np.int32)[None])
    rows = [0, 31, 32, 100, 255]
    a = O.index_select_attend(idx, wl.q, kv, seq, 32, wl.softmax_scale, rows)
    b = O.index_select_attend(idx2, wl.q, kv2, seq2, 32, wl.softmax_scale, rows)
    for t in rows:
        assert np.array_equal(a[0][t], b[0][t])
        assert np.array_equal(a[1][t], b[1][t])
        assert np.array_equal(a[2][t][0], b[2][t][0])


def test_zigzag_chunk_rows_equal_full_causal_rows():
    # rank 0 of 32 segments over T=512 holds positions 0..15 and 496..511
    full = W.make_workload("prefill_tiny", mla=False)     # T = 650 >= 512
    pos = np.concatenate([np.arange(16), np.arange(496, 512)]).astype(np.int32)
    seq_full = full.oracle_seq()
    seq_chunk = dict(seq_full, q_seq=np.zeros(32, np.int32), q_pos=pos)
    idx = full.oracle_indexer()
    idx_chunk = dict(idx, q=idx["q"][pos], q_scale=idx["q_scale"][pos], w=idx["w"][pos])
    a = O.index_scores(idx, seq_full, list(pos))
    b = O.index_scores(idx_chunk, seq_chunk)
    for j, t in enumerate(pos):
        assert np.array_equal(a[int(t)], b[j])
    assert list(W._seqmap(W.CONFIGS["cp_chunk_prefill_tiny"])[1]) == list(pos)
