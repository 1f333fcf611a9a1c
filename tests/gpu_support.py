"""Helpers shared by the GPU parity tests: upload a workload, run the oracle on
the same inputs, and compare with the stated tolerances."""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle as O
from sparse_index_attention_amd import sia
from sparse_index_attention_amd import workloads as W

# Score tolerance (the stated "1e-3 relative"): |g - o| <= 1e-3 |o| + 1e-6 max_s |o[t, s]|
# per row.  The floor only matters for exact and near-exact zeros (ReLU), where
# a different summation order may flip the sign of a head's dot product.
SCORE_REL = 1e-3
SCORE_FLOOR = 1e-6
# Attention tolerance: |g - o| <= ATOL + RTOL |o| elementwise.
ATT_TOL = {"bf16": (2e-2, 1e-2), "fp8": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}
LSE_ATOL = {"bf16": 2e-2, "fp8": 2e-2, "f32": 1e-4}


def dev(x: np.ndarray, device="cuda"):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


@functools.lru_cache(maxsize=8)
def workload(name):
    return W.make_workload(name)


def upload(wl: W.Workload, device="cuda"):
    c = wl.cfg
    seq = sia.SeqMap(dev(wl.q_seq), dev(wl.q_pos), dev(wl.block_table), wl.num_pages, wl.max_visible)
    if c["idx_dtype"] in ("f32", "bf16"):
        ix = sia.Indexer(dev(wl.iq), dev(wl.iw), dev(wl.ik))
    else:
        ix = sia.Indexer(dev(wl.iq), dev(wl.iw), dev(wl.ik), dev(wl.iq_scale), dev(wl.ik_scale))
    if c["kv_dtype"] == "fp8":
        st, se = c["kv_scale"]
        kv = sia.LatentKV(dev(wl.kv), c["Dc"], c["Dr"], dev(wl.kv_scale), st, se)
    else:
        kv = sia.LatentKV(dev(wl.kv), c["Dc"], c["Dr"])
    return seq, ix, dev(wl.q), kv


def score_bound_row(wl: W.Workload, t: int) -> np.ndarray:
    """A[t, s] for s <= q_pos[t]: the score taken on absolute values,
    sum_h |w_h| qs ks sum_d |q_hd k_sd|, the magnitude any summation-order or
    accumulator rounding error scales with (reported, not asserted)."""
    idx = wl.oracle_indexer()
    b, pos = int(wl.q_seq[t]), int(wl.q_pos[t])
    slots = O.physical_slots(wl.block_table[b], np.arange(pos + 1), W.PAGE)
    keys, ks = O.key_rows(idx["k"], idx.get("k_scale"), slots, idx.get("k_mx"))
    q = idx["q"][t]
    if idx.get("q_mx") is not None:
        qv, qs = O.mx_values(q, idx["q_mx"][t]), np.ones(q.shape[0])
    elif q.dtype == np.uint16:
        qv, qs = O.decode_bf16(q), np.ones(q.shape[0])
    elif q.dtype == np.uint8:
        qv = O.decode_e4m3(q)
        qs = np.full(q.shape[0], float(idx["q_scale"][t]))
    else:
        qv, qs = q.astype(np.float64), np.ones(q.shape[0])
    return O.index_scores_row(np.abs(qv), qs, np.abs(idx["w"][t].astype(np.float64)), np.abs(keys), ks)


def check_scores(wl, rows, got: np.ndarray, exp: dict, label=None, bound_rows=64):
    """Assert |g - o| <= 1e-3 |o| + 1e-6 max|o| on every entry of every row and
    print the worst observed errors: the ratio to that bound, the relative
    error over entries above the floor, and (on up to `bound_rows` rows) the
    error over A (score_bound_row)."""
    worst_ratio, worst_rel, worst_a, n = 0.0, 0.0, 0.0, 0
    first_bad = None
    for i, t in enumerate(rows):
        n_vis = int(wl.q_pos[t]) + 1
        o = exp[t].astype(np.float64)
        g = got[i, :n_vis].astype(np.float64)
        floor = SCORE_FLOOR * float(np.max(np.abs(o)))
        err = np.abs(g - o)
        tol = SCORE_REL * np.abs(o) + floor
        ratio = err / np.maximum(tol, 1e-300)
        bad = np.nonzero(~(err <= tol))[0]
        if bad.size and first_bad is None:
            first_bad = (t, bad.size, int(bad[0]), g[bad[0]], o[bad[0]])
        worst_ratio = max(worst_ratio, float(np.max(ratio)))
        big = np.abs(o) > floor
        if big.any():
            worst_rel = max(worst_rel, float(np.max(err[big] / np.abs(o[big]))))
        if i < bound_rows:
            A = score_bound_row(wl, t)
            pos = A > 0
            if pos.any():
                worst_a = max(worst_a, float(np.max(err[pos] / A[pos])))
        n += n_vis
    name = label or wl.name
    print(f"[score-err] {name} ({wl.cfg['idx_dtype']}): {n} scores; worst |g-o|/bound {worst_ratio:.3g}, "
          f"worst |g-o|/|o| {worst_rel:.3g}, worst |g-o|/A {worst_a:.3g}", flush=True)
    assert first_bad is None, (f"row {first_bad[0]}: {first_bad[1]} scores beyond 1e-3|o| + 1e-6 max|o|, "
                               f"first s={first_bad[2]} g={first_bad[3]} o={first_bad[4]}")
    return worst_ratio


def check_attention(kind, got_out, got_lse, exp: dict, rows):
    atol, rtol = ATT_TOL[kind]
    for i, t in enumerate(rows):
        o, l = exp[t]
        g = got_out[i].astype(np.float64)
        bad = ~(np.abs(g - o) <= atol + rtol * np.abs(o))
        assert not bad.any(), f"row {t}: {bad.sum()} outputs out of tolerance, max err {np.max(np.abs(g - o))}"
        if got_lse is not None:
            gl = got_lse[i].astype(np.float64)
            fin = np.isfinite(l)
            assert np.array_equal(fin, np.isfinite(gl)), f"row {t}: lse finiteness differs"
            assert np.all(np.abs(gl[fin] - l[fin]) <= LSE_ATOL[kind] + 1e-4 * np.abs(l[fin])), f"row {t}: lse"


def to_np_out(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy()


def tie_band_ok(oracle_scores_row: np.ndarray, K: int, got_ids: np.ndarray, exp_ids: np.ndarray) -> bool:
    """Index sets equal except for positions whose oracle score lies within
    1e-3 relative of the K-th oracle score (exact zeros when that score is 0)."""
    a = set(int(x) for x in got_ids if x >= 0)
    b = set(int(x) for x in exp_ids if x >= 0)
    if len(a) != len(b):
        return False
    diff = a ^ b
    if not diff:
        return True
    sK = float(np.sort(oracle_scores_row.astype(np.float64))[::-1][min(K, len(oracle_scores_row)) - 1])
    band = 1e-3 * abs(sK)
    return all(abs(float(oracle_scores_row[j]) - sK) <= band for j in diff)


def page_max(row):
    """Largest score of each 64-position page of a row."""
    n = row.shape[0]
    return np.array([row[b * 64: b * 64 + 64].max() for b in range((n + 63) // 64)], dtype=np.float32)


def page_band_ok(oracle_scores_row, K, got_ids, exp_ids):
    """Both lists are whole visible pages in ascending order, and the kept page
    sets differ only in pages whose oracle page score lies within 1e-3 relative
    of the (K/64)-th best page score."""
    n = oracle_scores_row.shape[0]
    for ids in (got_ids, exp_ids):
        pages = sorted(set(int(x) // 64 for x in ids if x >= 0))
        whole = [p for b in pages for p in range(b * 64, min(n, b * 64 + 64))]
        if list(ids[: len(whole)]) != whole or np.any(ids[len(whole):] != -1):
            return False
    pm = page_max(oracle_scores_row.astype(np.float64))
    a = set(int(x) // 64 for x in got_ids if x >= 0)
    b = set(int(x) // 64 for x in exp_ids if x >= 0)
    if len(a) != len(b):
        return False
    diff = a ^ b
    if not diff:
        return True
    sK = float(np.sort(pm)[::-1][min(K // 64, len(pm)) - 1])
    return all(abs(float(pm[p]) - sK) <= 1e-3 * abs(sK) for p in diff)


def kind_of(wl):
    return wl.cfg["kv_dtype"]
