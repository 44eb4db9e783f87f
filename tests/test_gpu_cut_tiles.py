"""Prefill tiles cut into key chunks (a short chunk of new rows on a long cached prefix):
every chunk tile writes partial results that the combine pass merges.  Parity with the
oracle on every element at small sizes (chunk length forced, ragged chunks, NaN-poisoned
page tails, bf16 / fp8 / head_dim 64) and on sampled rows of a long chunk the planner cuts
by itself; the cut and uncut plans of that chunk also agree within the bf16 tolerance."""
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


def _oracle_full(w):
    if w.dtype == "fp8":
        K, V = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
    else:
        K, V = w.k_pool, w.v_pool
    return oracle.varlen_paged_attention(w.q, K, V, w.block_table, w.q_start, w.q_end, w.kv_len, w.page_size,
                                         w.softmax_scale or None)


SMALL = [
    # label, workload, prefill_split_len
    ("g4 chunks of 1024 + decodes", lambda d: W.build("c", [300, 1, 40], [5000, 77, 2100], num_q_heads=8,
                                                       num_kv_heads=2, head_dim=128, page_size=16, seed=7,
                                                       dtype=d, poison_tail=True), 1000),
    ("g1 d64 chunks of 64", lambda d: W.build("c", [130, 64], [700, 64], num_q_heads=2, num_kv_heads=2,
                                              head_dim=64, page_size=32, seed=8, dtype=d, poison_tail=True), 64),
    ("g8 chunk-mix/8 chunks of 256", lambda d: W.config(4, scale=8, poison_tail=True, dtype=d), 256),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("label,make,split", SMALL, ids=[s[0] for s in SMALL])
def test_cut_tiles_elementwise(label, make, split, dtype):
    w = make(dtype)
    plan = api.plan_for(w, prefill_split_len=split)
    st = api.varlen_attn_plan_stats(plan)
    _say(f"[gpu] cut tiles {label} {dtype}: {st['prefill_split_tiles']} of {st['prefill_tiles']} tiles cut")
    assert st["prefill_split_tiles"] > 0
    out, _ = api.run_workload(w, plan=plan)
    got = out.float().cpu().numpy().astype(np.float64)
    ref = _oracle_full(w)
    worst = 0.0
    for r in range(w.num_reqs):
        a, b = int(w.q_start[r]), int(w.q_end[r])
        assert np.isfinite(got[a:b]).all(), f"{label}: non-finite output in request {r}"
        worst = max(worst, float(np.abs(got[a:b] - ref[a:b]).max()))
    _say(f"[parity] cut tiles {label} {dtype}: max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL


def test_long_chunk_auto_cut_sampled():
    """256 new rows on 65,536 cached positions (32 query heads over 8 KV heads): 64 tiles
    become 512 chunk tiles."""
    import torch
    w = W.build("lc", [256, 1], [65536 + 256, 3000], num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=64,
                seed=6)
    plan = api.plan_for(w)
    st = api.varlen_attn_plan_stats(plan)
    _say(f"[gpu] long chunk: {st['prefill_split_tiles']} of {st['prefill_tiles']} tiles cut")
    assert st["prefill_split_tiles"] == 512
    out, _ = api.run_workload(w, plan=plan)
    whole, _ = api.run_workload(w, prefill_split_len=-1)
    assert api.varlen_attn_plan_stats(api.plan_for(w, prefill_split_len=-1))["prefill_split_tiles"] == 0
    got = out.float().cpu().numpy()
    diff = float((out.float() - whole.float()).abs().max())
    _say(f"[parity] long chunk cut vs whole tiles: max diff {diff:.3e}")
    assert np.isfinite(got).all() and diff <= TOL
    del whole
    torch.cuda.empty_cache()
    worst = 0.0
    for rows in ([0, 1, 77, 128, 200, 255],):
        ref = oracle.attention_rows(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                    w.page_size, 0, rows)
        for h, o in ref.items():
            worst = max(worst, float(np.abs(got[np.asarray(rows), h, :] - o).max()))
    _say(f"[parity] long chunk sampled rows: max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL


def test_long_chunk_auto_cut_focused():
    """The same automatically cut chunk on the focused companion inputs (outputs O(1)):
    sampled rows and heads against the oracle, with negative controls (an all-zero output,
    a dropped or doubled hot 64-key step must fail the comparison)."""
    import sampled
    w = W.focus(W.build("lc", [256, 1], [65536 + 256, 3000], num_q_heads=32, num_kv_heads=8, head_dim=128,
                        page_size=64, seed=6))
    plan = api.plan_for(w)
    assert api.varlen_attn_plan_stats(plan)["prefill_split_tiles"] == 512
    out, _ = api.run_workload(w, plan=plan)
    got = out.float().cpu().numpy()
    worst, margin = 0.0, np.inf
    for r, rows, heads in ((0, [0, 1, 77, 128, 200, 255], [0, 3, 9, 17, 30, 31]), (1, [0], [0, 5, 31])):
        got_rows = {h: got[int(w.q_start[r]) + np.asarray(rows), h, :] for h in heads}
        e, mg = sampled.check_request(w, r, rows, heads, got_rows, TOL)
        worst, margin = max(worst, e), min(margin, mg)
    _say(f"[parity] long chunk focused: max|gpu-oracle| = {worst:.3e}; smallest negative-control error {margin:.3e}")
    assert margin > TOL
