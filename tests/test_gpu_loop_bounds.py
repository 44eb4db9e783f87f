"""GPU parity at the boundaries of the prefill kernel's loop: tiles of 1 to 8 64-key steps
with ragged ends (lengths one short of, equal to and one past a multiple of 64), causal
diagonals that start and end at every position within a step, workgroups whose later
waves see no keys (a one-row prompt has one column), key-chunk tiles whose first key is
not 0, and decode tiles, in bf16 and fp8 storage at head dims 64 and 128.  These are
the shapes where the kernel switches between its loop forms (unmasked / masked, whole
tiles / tiles with a tail, the last tile of a wave, the copy-only steps after it).
Every output row is compared with the oracle (tolerance 2e-2 bf16, 1e-2 fp8); slots
past each request's length hold NaN."""
import sys

import numpy as np
import pytest

import oracle
from varlen_paged_attention_amd import api, workloads as W

pytestmark = pytest.mark.gpu


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


# (q_rows, kv_len) per request: uncached prompts, chunks on cached prefixes, decodes
PROMPTS = [(1, 1), (63, 63), (64, 64), (65, 65), (130, 130), (191, 191), (256, 256), (257, 257)]
CHUNKS = [(16, 79), (100, 163), (128, 320), (129, 449), (64, 513), (30, 250)]
DECODES = [(1, 63), (1, 64), (1, 65), (1, 191), (1, 192), (1, 193), (1, 257), (1, 512)]
CASES = [(d, g, dt) for dt in ("bf16", "fp8") for d in (128, 64) for g in (1, 4)]


def _build(d, g, dtype, reqs, seed):
    rows, kv = zip(*reqs)
    return W.build(f"loop-bounds-d{d}-g{g}-{dtype}", rows, kv, num_q_heads=2 * g, num_kv_heads=2, head_dim=d,
                   page_size=16 if d == 128 else 64, dtype=dtype, seed=seed, poison_tail=True)


def _check(w, flags, kw, label):
    out, plan = api.run_workload(w, flags=flags, **kw)
    got = out.float().cpu().numpy().astype(np.float64)
    if w.dtype == "fp8":
        K, V = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
        tol = 1e-2
    else:
        K, V, tol = w.k_pool, w.v_pool, 2e-2
    ref = oracle.varlen_paged_attention(w.q, K, V, w.block_table, w.q_start, w.q_end, w.kv_len, w.page_size)
    rows = np.zeros(w.total_q_rows, bool)
    for r in range(w.num_reqs):
        rows[w.q_start[r]:w.q_end[r]] = True
    e = float(np.abs(got[rows] - ref[rows]).max())
    st = api.varlen_attn_plan_stats(plan)
    _say(f"[parity] {label}: tiles {st['prefill_tiles']} (cut {st['prefill_split_tiles']}), items "
         f"{st['split_items']}: max|gpu-oracle| = {e:.3e} (tol {tol})")
    assert np.isfinite(got[rows]).all(), f"{label}: non-finite output"
    assert e <= tol, f"{label}: max error {e}"


@pytest.mark.parametrize("d,g,dtype", CASES, ids=[f"d{d}-g{g}-{dt}" for d, g, dt in CASES])
def test_loop_bounds_whole_tiles(d, g, dtype):
    """Prompts, chunks and decodes (decodes as tiles) in one plan: whole tiles only."""
    w = _build(d, g, dtype, PROMPTS + CHUNKS + DECODES, seed=d + g)
    _say(f"[gpu] loop bounds, whole tiles: d{d} g{g} {dtype}")
    _check(w, 0, {}, f"whole tiles d{d} g{g} {dtype}")


@pytest.mark.parametrize("d,g,dtype", CASES, ids=[f"d{d}-g{g}-{dt}" for d, g, dt in CASES])
def test_loop_bounds_key_chunks(d, g, dtype):
    """The same requests with every tile cut into 128-key chunks (key-chunk tiles start at
    kbeg > 0 and end where the next chunk starts; the last chunk holds the diagonal)."""
    w = _build(d, g, dtype, PROMPTS + CHUNKS + DECODES, seed=d + g + 1)
    _say(f"[gpu] loop bounds, 128-key chunks: d{d} g{g} {dtype}")
    _check(w, 0, {"prefill_split_len": 128}, f"key chunks d{d} g{g} {dtype}")


@pytest.mark.parametrize("d,g", [(128, 1), (128, 4), (64, 4)])
def test_loop_bounds_decode_tiles(d, g):
    """Enough decodes (lengths around multiples of 64) that the planner runs them as tiles
    of g columns each: a tile's first wave holds every column, the other three see no keys
    and only copy their slices."""
    reqs = PROMPTS[:4] + [DECODES[i % len(DECODES)] for i in range(320)]
    w = _build(d, g, "bf16", reqs, seed=7 + d + g)
    _say(f"[gpu] loop bounds, decode tiles: d{d} g{g}")
    st = api.varlen_attn_plan_stats(api.plan_for(w))
    assert st["split_items"] == 0, f"decodes expected as tiles: {st}"
    _check(w, 0, {}, f"decode tiles d{d} g{g}")
