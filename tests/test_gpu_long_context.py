"""The long-context decode workload (256 requests x 128K positions, page 64: 524,288
block-table entries, 137 GB of bf16 K/V made on the device from the page hash) through
the C ABI: device pools equal the host generator bit for bit on sampled pages; parity
with the oracle on a scaled-down copy (every element) and on sampled requests of the full
size, the full-size run captured in a HIP graph."""
import sys

import numpy as np
import pytest

import oracle
from varlen_paged_attention_amd import api, workloads as W

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    api.lib()
    yield
    torch.cuda.empty_cache()


def _oracle_request(w, r, rows=None):
    """Oracle rows of request r from its own pages, regenerated on the host."""
    npg = -(-int(w.kv_len[r]) // w.page_size)
    K, V = W.host_kv_pages(w, w.block_table[r][:npg])
    bt = np.arange(npg, dtype=np.int32)[None, :]
    return oracle.attention_rows(w.q, K, V, bt, np.array([w.q_start[r]], np.int32), np.array([w.q_end[r]], np.int32),
                                 np.array([w.kv_len[r]], np.int32), w.page_size, 0, rows)


def test_device_pages_equal_host_generator():
    import torch
    w = W.config(8, scale=64)
    _say(f"[gpu] hashed pools scale 64: {w.num_pages} pages")
    k, v = W.hashed_pools_device(w, "cuda", pages_per_chunk=100)
    torch.cuda.synchronize()
    pages = np.array([0, 1, 99, 100, w.num_pages - 1])
    kh, vh = W.host_kv_pages(w, pages)
    assert np.array_equal(k[torch.from_numpy(pages).cuda()].view(torch.int16).cpu().numpy().view(np.uint16), kh)
    assert np.array_equal(v[torch.from_numpy(pages).cuda()].view(torch.int16).cpu().numpy().view(np.uint16), vh)


def test_long_context_scaled_elementwise():
    w = W.config(8, scale=128)                      # 2 requests x 1024 positions
    _say(f"[gpu] long-context scaled: {w.num_reqs} x {int(w.kv_len[0])}")
    out, plan = api.run_workload(w)
    got = out.float().cpu().numpy()
    worst = 0.0
    for r in range(w.num_reqs):
        for h, o in _oracle_request(w, r).items():
            worst = max(worst, float(np.abs(got[int(w.q_start[r]):int(w.q_end[r]), h, :] - o).max()))
    _say(f"[parity] long-context/128: max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL


def test_long_context_full_size_graph_sampled():
    import torch
    w = W.config(8)
    _say(f"[gpu] long-context full: {w.num_reqs} x {int(w.kv_len[0])}, {w.num_pages} pages")
    plan = api.plan_for(w)
    st = api.varlen_attn_plan_stats(plan)
    assert st["table_bytes"] == 524288 * 4
    q, k, v, bt = api.to_device(w)
    out = torch.zeros_like(q)
    ws = api.new_workspace(plan)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call = api.RunCall(plan, q, k, v, bt, out, ws, stream=s)
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    got = out.float().cpu().numpy()
    del k, v, g
    torch.cuda.empty_cache()
    worst = 0.0
    for r in (0, w.num_reqs - 1):
        for h, o in _oracle_request(w, r).items():
            worst = max(worst, float(np.abs(got[int(w.q_start[r]), h, :] - o[0]).max()))
    _say(f"[parity] long-context full (graph replay), requests 0 and last: max|gpu-oracle| = {worst:.3e}")
    assert np.isfinite(got).all()
    assert worst <= TOL


def test_long_context_focused_full_size_graph_sampled():
    """The full 128K workload on the focused companion inputs (outputs O(1)), run through a
    HIP graph replay.  Sampled requests include the one holding the highest page id; their
    hot keys lie on pages above id 2^16 whose K and V bytes sit more than 4 GiB into the
    pools, so 32-bit page offsets would show.  Each request's comparison comes with its
    negative controls (an all-zero output, a dropped or doubled hot 64-key step must fail)."""
    import torch
    import sampled
    w = W.focus(W.config(8))
    _say(f"[gpu] long-context focused full: {w.num_reqs} x {int(w.kv_len[0])}, {w.num_pages} pages")
    plan = api.plan_for(w)
    q, k, v, bt = api.to_device(w)
    page_bytes = k[0].numel() * k.element_size()
    out = torch.zeros_like(q)
    ws = api.new_workspace(plan)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call = api.RunCall(plan, q, k, v, bt, out, ws, stream=s)
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del k, v, g
    torch.cuda.empty_cache()
    R, Hkv = w.num_reqs, w.num_kv_heads
    gq = w.num_q_heads // Hkv
    top = int(np.argmax(w.block_table.max(axis=1)))
    reqs = sorted({0, R - 1, top, 97})
    worst, margin, high = 0.0, np.inf, 0
    for r in reqs:
        kvhs = sorted({r % Hkv, (r * 5 + 3) % Hkv})
        heads = [kvh * gq + c for kvh in kvhs for c in range(gq)]
        for kvh in kvhs:
            for c in range(gq):
                pos = w.notes["hot"][(r, kvh, c)]
                pages = w.block_table[r, pos // w.page_size].astype(np.int64)
                high += int(((pages >= 1 << 16) & (pages * page_bytes >= 1 << 32)).sum())
        got_rows = {h: got[int(w.q_start[r]):int(w.q_start[r]) + 1, h, :] for h in heads}
        e, mg = sampled.check_request(w, r, [0], heads, got_rows, TOL)
        worst, margin = max(worst, e), min(margin, mg)
        _say(f"[parity] long-context focused request {r} (max page {int(w.block_table[r].max())}): "
             f"max|gpu-oracle| = {e:.3e}, control margin {mg:.3e}")
    _say(f"[parity] long-context focused full (graph replay): max|gpu-oracle| = {worst:.3e}; "
         f"{high} sampled hot keys on pages above id 2^16 and 4 GiB")
    assert high >= 32
    assert int(w.block_table[top].max()) >= w.num_pages - 64
    assert worst <= TOL and margin > TOL
