"""sia_index_select_attend_noalloc, called through the C ABI, against
sia_index_select_attend with a caller workspace: the same kernels on the same
inputs, so indices, outputs and LSE must agree bit for bit.  Two calls in a
row share the library's per-GPU array, the second on a smaller batch."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_index_attention_amd import sia
from sparse_index_attention_amd import workloads as W

from gpu_support import upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    sia.lib()


def noalloc_raw(ix, q, kv, seq, K, scale, order, idx, out, lse):
    a, s, k = ix.c(), seq.c(), kv.c()
    return sia.lib().sia_index_select_attend_noalloc(
        ctypes.byref(a), sia._ptr(q), sia.dtype_code(q), q.shape[1], ctypes.byref(k), ctypes.byref(s), K, order,
        float(scale), sia._ptr(idx), sia._ptr(out), sia._ptr(lse), sia._stream(None))


def compare(name, order):
    print(f"[noalloc] {name} order={order}: generating", flush=True)
    wl = W.make_workload(name)
    K, H, Dc = wl.cfg["K"], wl.cfg["H"], wl.cfg["Dc"]
    seq, ix, q, kv = upload(wl)
    n = sia.workspace_size(sia.OP_INDEX_SELECT_ATTEND, seq, K, H, Dc)
    assert n <= sia.NOALLOC_WORKSPACE_BYTES
    res = []
    for use_ws in (True, False):
        idx = torch.full((wl.Tq, K), -7, dtype=torch.int32, device="cuda")
        lse = torch.full((wl.Tq, H), 7.0, dtype=torch.float32, device="cuda")
        out = torch.full((wl.Tq, H, Dc), 7.0, dtype=q.dtype, device="cuda")
        if use_ws:
            sia.index_select_attend(ix, q, kv, seq, K, wl.softmax_scale, order=order, idx_out=idx, out=out, lse=lse)
        else:
            rc = noalloc_raw(ix, q, kv, seq, K, wl.softmax_scale, order, idx, out, lse)
            assert rc == 0, sia.lib().sia_status_string(rc)
        torch.cuda.synchronize()
        res.append((idx.cpu().numpy(), out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
    print(f"[noalloc] {name} order={order}: identical to the workspace call ({n / 2**20:.1f} MiB)", flush=True)


def test_noalloc_matches_workspace_call_twice():
    compare("decode", 0)          # the benchmarked decode batch
    compare("decode_tiny", 0)     # then a smaller batch on the same array


def test_noalloc_small_prefill_and_page_selection():
    compare("chunked_prefill_tiny", 1)
    compare("quant_decode_tiny", 2)


def test_noalloc_replays_from_a_captured_graph():
    """The callers this entry point is for include code under HIP graph
    capture.  The call is captured once and replayed three times, with eager
    work (the outputs overwritten, an unrelated kernel) and synchronisations
    between replays; every replay must give the eager call's bits."""
    name, order = "decode_tiny", 0
    print(f"[noalloc-graph] {name}: eager reference", flush=True)
    wl = W.make_workload(name)
    K, H, Dc = wl.cfg["K"], wl.cfg["H"], wl.cfg["Dc"]
    seq, ix, q, kv = upload(wl)
    idx = torch.empty((wl.Tq, K), dtype=torch.int32, device="cuda")
    lse = torch.empty((wl.Tq, H), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.Tq, H, Dc), dtype=q.dtype, device="cuda")
    # eager call first: it also looks up the array's address, outside the capture
    assert noalloc_raw(ix, q, kv, seq, K, wl.softmax_scale, order, idx, out, lse) == 0
    torch.cuda.synchronize()
    ref = (idx.cpu().numpy(), out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = noalloc_raw(ix, q, kv, seq, K, wl.softmax_scale, order, idx, out, lse)
    assert rc == 0, sia.lib().sia_status_string(rc)
    torch.cuda.synchronize()
    junk = torch.ones(1 << 20, device="cuda")
    for rep in range(3):
        idx.fill_(-7)
        out.fill_(7.0)
        lse.fill_(7.0)
        junk.mul_(1.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (idx.cpu().numpy(), out.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy())
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager call"
        print(f"[noalloc-graph] replay {rep}: identical", flush=True)
