"""The attention kernel's own staging of bf16 K/V pages (the buffer-resource DMA
addressing every bf16 tile uses) copied out in logical order by
varlen_attn_debug_stage_gather, compared bit for bit with NumPy fancy indexing of the
pools: small iterations over every page size and both head dims with NaN-poisoned page
tails, and one request of 131,072 positions whose pages all lie more than 4 GiB into
pools of about 6 GiB (page sizes 16 and 256; 0.5 GB of output)."""
import sys

import numpy as np
import pytest

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
    torch.cuda.empty_cache()


def _staged(w, k, v, bt):
    import torch
    plan = api.plan_for(w)
    ko = torch.full((int(w.kv_len.sum()), w.num_kv_heads, w.head_dim), 7.0, dtype=torch.bfloat16, device="cuda")
    vo = torch.full_like(ko, 7.0)
    api.varlen_attn_debug_stage_gather(plan, k, v, bt, ko, vo)
    torch.cuda.synchronize()
    return ko.view(torch.int16).cpu().numpy().view(np.uint16), vo.view(torch.int16).cpu().numpy().view(np.uint16)


def _logical(kp, vp, pages, L, ps):
    """[L, Hkv, D] K and V of one request from its pages (host arrays), by fancy indexing."""
    j = np.arange(L)
    return kp[pages[j // ps], :, j % ps, :], vp[pages[j // ps], :, :, j % ps]


SMALL = [
    ("orca/4 ps16", lambda: W.config(2, scale=4, poison_tail=True)),
    ("decode-heavy/8 ps64", lambda: W.config(3, scale=8, poison_tail=True)),
    ("d64 ps32", lambda: W.build("g", [30, 1, 1], [300, 77, 1], num_q_heads=6, num_kv_heads=3, head_dim=64,
                                 page_size=32, seed=4, poison_tail=True, extra_pages=2)),
    ("ps128", lambda: W.build("g", [1, 9], [1000, 130], num_q_heads=8, num_kv_heads=2, head_dim=128,
                              page_size=128, seed=5, poison_tail=True)),
    ("ps256", lambda: W.build("g", [1, 1, 3], [700, 256, 5], num_q_heads=4, num_kv_heads=4, head_dim=128,
                              page_size=256, seed=6, poison_tail=True)),
]


@pytest.mark.parametrize("label,make", SMALL, ids=[s[0] for s in SMALL])
def test_stage_gather_bit_exact(label, make):
    w = make()
    _say(f"[gpu] staged gather {label}")
    q, k, v, bt = api.to_device(w)
    gk, gv = _staged(w, k, v, bt)
    wk, wv = [], []
    for r in range(w.num_reqs):
        a, b = _logical(w.k_pool, w.v_pool, w.block_table[r].astype(np.int64), int(w.kv_len[r]), w.page_size)
        wk.append(a)
        wv.append(b)
    assert np.array_equal(gk, np.concatenate(wk)) and np.array_equal(gv, np.concatenate(wv))


@pytest.mark.parametrize("ps,pool_pages", [(16, 200_000), (256, 12_000)])
def test_stage_gather_128k_request_above_4gib(ps, pool_pages):
    import torch
    L = 131072
    w = W.build("g128k", [1], [L], num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=ps, seed=12,
                hashed_kv=True)
    npg = L // ps
    page_bytes = 8 * ps * 128 * 2
    lo = (4 << 30) // page_bytes + 1                   # every page starts more than 4 GiB into the pool
    rng = np.random.default_rng(ps)
    pages = rng.choice(np.arange(lo, pool_pages), size=npg, replace=False).astype(np.int32)
    w.num_pages = pool_pages
    w.block_table = pages[None, :].copy()
    _say(f"[gpu] staged gather 128K ps={ps}: pool {pool_pages} pages ({pool_pages * page_bytes / 2**30:.1f} GiB), "
         f"page ids {pages.min()}..{pages.max()}")
    q, k, v, bt = api.to_device(w)
    gk, gv = _staged(w, k, v, bt)
    del k, v
    torch.cuda.empty_cache()
    kh, vh = W.host_kv_pages(w, pages)                 # the request's pages, in table order
    j = np.arange(L)
    assert np.array_equal(gk, kh[j // ps, :, j % ps, :])
    assert np.array_equal(gv, vh[j // ps, :, :, j % ps])
