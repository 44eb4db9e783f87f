"""Short requests (decodes, speculative-decode verify rows) on the MFMA prefill tiles.

The planner puts them there by itself on bf16 plans whose tiles fill the GPU (the full-size
parity tests cover those); here ``prefill_min_rows=1`` forces every request onto tiles at
small sizes, also cut into key chunks, and every output element is compared with the
oracle: head_dim 64 and 128, page sizes 16 to 256, kv lengths around page and 16-key slice
boundaries (1, 15, 16, 17, 63, 64, 65, ...), NaN-poisoned page tails, bf16 and fp8 pools."""
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


def _oracle_full(w):
    if w.dtype == "fp8":
        K, V = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
    else:
        K, V = w.k_pool, w.v_pool
    return oracle.varlen_paged_attention(w.q, K, V, w.block_table, w.q_start, w.q_end, w.kv_len, w.page_size,
                                         w.softmax_scale or None)


def _edge(d, ps, dtype):
    kv = [1, 15, 16, 17, 63, 64, 65, 200, 1000, 1500]
    rows = [1] * 8 + [3, 5]                    # decodes and two verify steps
    return W.build("edge", rows, kv, num_q_heads=8, num_kv_heads=2, head_dim=d, page_size=ps, seed=31,
                   dtype=dtype, poison_tail=True, extra_pages=2)


CASES = [
    ("decode-heavy/8", lambda dt: W.config(3, scale=8, poison_tail=True, dtype=dt)),
    ("spec-decode-mtp3/8", lambda dt: W.config(6, scale=8, poison_tail=True, dtype=dt)),
    ("spec-decode-mtp7/8", lambda dt: W.config(7, scale=8, poison_tail=True, dtype=dt)),
    ("edge d128 ps16", lambda dt: _edge(128, 16, dt)),
    ("edge d64 ps128", lambda dt: _edge(64, 128, dt)),
    ("edge d128 ps256", lambda dt: _edge(128, 256, dt)),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("split", [0, 64], ids=["whole", "cut64"])
@pytest.mark.parametrize("label,make", CASES, ids=[c[0] for c in CASES])
def test_short_requests_on_tiles_elementwise(label, make, split, dtype):
    w = make(dtype)
    plan = api.plan_for(w, prefill_min_rows=1, prefill_split_len=split)
    st = api.varlen_attn_plan_stats(plan)
    assert st["split_items"] == 0 and st["prefill_tiles"] > 0
    if split:
        assert st["prefill_split_tiles"] > 0
    _say(f"[gpu] short requests on tiles: {label} {dtype} split={split} tiles={st['prefill_tiles']} "
         f"cut={st['prefill_split_tiles']}")
    out, _ = api.run_workload(w, plan=plan)
    got = out.float().cpu().numpy().astype(np.float64)
    ref = _oracle_full(w)
    worst = 0.0
    for r in range(w.num_reqs):
        a, b = int(w.q_start[r]), int(w.q_end[r])
        assert np.isfinite(got[a:b]).all(), f"{label}: non-finite output in request {r}"
        worst = max(worst, float(np.abs(got[a:b] - ref[a:b]).max()))
    _say(f"[parity] short requests on tiles {label} {dtype} split={split}: max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL


def test_auto_decode_tiles_equal_split_items_full_size():
    """The decode-heavy iteration at full size: tiles (chosen by the planner) and split-KV
    items (VA_FLAG_NO_DECODE_TILES) agree within the bf16 tolerance on every element."""
    w = W.config(3)
    p_tiles, p_items = api.plan_for(w), api.plan_for(w, flags=api.VA_FLAG_NO_DECODE_TILES)
    assert api.varlen_attn_plan_stats(p_tiles)["split_items"] == 0
    assert api.varlen_attn_plan_stats(p_items)["prefill_tiles"] == 0
    a, _ = api.run_workload(w, plan=p_tiles)
    b, _ = api.run_workload(w, plan=p_items)
    diff = float((a.float() - b.float()).abs().max())
    _say(f"[parity] decode-heavy tiles vs split-KV items: max diff {diff:.3e}")
    assert diff <= TOL


def test_shared_prefix_members_own_keys_on_tiles_elementwise():
    """64 requests sharing 4 leading pages, with 1-5 new rows each (decodes and verify
    steps, causal among their own rows): group tiles score the shared pages and column-list
    tiles each member's own keys, in one launch; every element against the oracle."""
    rows = [1 + (r % 5) for r in range(64)]
    kv = [256 + 40 + 7 * r for r in range(64)]
    w = W.build("shared-rows", rows, kv, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64, seed=23,
                shared_prefix_pages=4, poison_tail=True)
    plan = api.plan_for(w, flags=api.VA_FLAG_SHARED_PREFIX)
    st = api.varlen_attn_plan_stats(plan)
    assert st["shared_groups"] == 1 and st["shared_tiles"] > 0 and st["split_items"] == 0
    _say(f"[gpu] shared prefix, members on tiles: {st['prefill_tiles']} tiles ({st['shared_tiles']} group)")
    out, _ = api.run_workload(w, plan=plan)
    got = out.float().cpu().numpy().astype(np.float64)
    ref = _oracle_full(w)
    assert np.isfinite(got).all()
    worst = float(np.abs(got - ref).max())
    _say(f"[parity] shared prefix, members on tiles: max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL


def test_stream_read_probe_runs():
    """The HBM read-rate probe reads a buffer; for data that is all ones the XOR of every
    lane's words is 0, so the sink keeps its value."""
    import torch
    buf = torch.ones(1 << 24, dtype=torch.int32, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    api.varlen_attn_debug_stream_read(buf, sink)
    api.varlen_attn_debug_stream_read(buf[:12], sink)         # 3 words: fewer than the grid has lanes
    torch.cuda.synchronize()
    assert int(sink.item()) == 7
