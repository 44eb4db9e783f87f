"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.  Tolerances: max |gpu - oracle| <= 2e-2 for bf16 inputs/outputs with fp32
accumulation, <= 1e-4 for fp32; the page gather is compared bit for bit."""
import functools
import sys

import numpy as np
import pytest

import oracle
from varlen_paged_attention_amd import api, workloads as W

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


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


@functools.lru_cache(maxsize=4)
def _cfg(cid, scale=1, poison=False):
    return W.config(cid, scale=scale, poison_tail=poison)


def _oracle_full(w):
    return oracle.varlen_paged_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                         w.page_size, w.softmax_scale or None)


def _covered_rows(w):
    rows = np.zeros(w.total_q_rows, bool)
    for r in range(w.num_reqs):
        rows[w.q_start[r]:w.q_end[r]] = True
    return rows


def _check_full(w, out, label):
    got = out.float().cpu().numpy().astype(np.float64)
    ref = _oracle_full(w)
    rows = _covered_rows(w)
    err = np.abs(got[rows] - ref[rows])
    e = float(err.max()) if err.size else 0.0
    _say(f"[parity] {label}: max|gpu-oracle| = {e:.3e} (tol {TOL[w.dtype]})")
    assert np.isfinite(got[rows]).all(), f"{label}: non-finite output"
    assert e <= TOL[w.dtype], f"{label}: max error {e}"
    return e


SMALL = [
    ("tiny-f32", 1, 1, 0),
    ("orca-mixed/4", 2, 4, 0),
    ("orca-mixed/4 split-only", 2, 4, api.VA_FLAG_NO_PREFILL_KERNEL),
    ("decode-heavy/8", 3, 8, 0),
    ("chunk-mix/8", 4, 8, 0),
    ("shared-6", 5, 1, api.VA_FLAG_SHARED_PREFIX),
    ("shared-6 plain", 5, 1, 0),
    ("shared-6 split items", 5, 1, api.VA_FLAG_SHARED_PREFIX | api.VA_FLAG_NO_PREFILL_KERNEL),
    ("shared-64/8", 51, 8, api.VA_FLAG_SHARED_PREFIX),
    ("spec-decode-mtp3/8", 6, 8, 0),
    ("spec-decode-mtp7/8", 7, 8, 0),
    ("long-prefix-chunk/8", 9, 8, 0),
]


@pytest.mark.parametrize("label,cid,scale,flags", SMALL, ids=[s[0] for s in SMALL])
def test_parity_small_elementwise(label, cid, scale, flags):
    """Every output element at reduced lengths (several tiles and splits, ragged tails)."""
    w = W.config(cid, scale=scale, poison_tail=True)
    _say(f"[gpu] run {label} rows={w.total_q_rows} kv={list(w.kv_len[:4])}...")
    out, plan = api.run_workload(w, flags=flags)
    _check_full(w, out, label)


def _sample_rows(w, rng, nreq, nrows):
    """(request, rows) samples: the first/last requests, the longest, and random ones."""
    R = w.num_reqs
    reqs = {0, R - 1, int(np.argmax(w.kv_len)), int(np.argmin(w.kv_len))}
    reqs |= set(int(x) for x in rng.choice(R, size=min(R, nreq), replace=False))
    out = []
    for r in sorted(reqs):
        m = int(w.q_end[r] - w.q_start[r])
        rows = {0, m - 1} | set(int(x) for x in rng.choice(m, size=min(m, nrows), replace=False))
        out.append((r, sorted(rows)))
    return out


FULL = [("orca-mixed", 2, 0), ("decode-heavy", 3, 0), ("chunk-mix", 4, 0), ("shared-6", 5, api.VA_FLAG_SHARED_PREFIX),
        ("shared-64", 51, api.VA_FLAG_SHARED_PREFIX), ("spec-decode-mtp3", 6, 0), ("spec-decode-mtp7", 7, 0),
        ("long-prefix-chunk", 9, 0),
        # the short requests of these run as prefill tiles by default; also on split-KV items
        ("decode-heavy split-KV", 3, api.VA_FLAG_NO_DECODE_TILES),
        ("spec-decode-mtp7 split-KV", 7, api.VA_FLAG_NO_DECODE_TILES),
        ("orca-mixed split-KV decodes", 2, api.VA_FLAG_NO_DECODE_TILES)]


@pytest.mark.parametrize("label,cid,flags", FULL, ids=[f[0] for f in FULL])
def test_parity_full_size_sampled(label, cid, flags):
    """Full-size workloads in the launch configuration the bench times; sampled rows (all
    heads) computed one by one by the oracle."""
    w = _cfg(cid)
    _say(f"[gpu] run full {label}: reqs={w.num_reqs} rows={w.total_q_rows} pages={w.num_pages}")
    out, plan = api.run_workload(w, flags=flags)
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(100 + cid)
    worst = 0.0
    for r, rows in _sample_rows(w, rng, 10, 12):
        ref = oracle.attention_rows(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                    w.page_size, r, rows)
        for h, o in ref.items():
            g = got[int(w.q_start[r]) + np.asarray(rows), h, :]
            assert np.isfinite(g).all()
            worst = max(worst, float(np.abs(g - o).max()))
    _say(f"[parity] full {label}: sampled max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL[w.dtype]


@functools.lru_cache(maxsize=2)
def _focused(cid):
    return W.focus(_cfg(cid))


def _focused_check(w, out, label, seed, nreq=6, nrows=8, nheads=8):
    """Sampled rows of a focused full-size run against the oracle, each sampled request's
    comparison with its negative controls (an all-zero output and a dropped or doubled hot
    64-key step must fail it) where the request has cached keys."""
    import sampled
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(seed)
    Hq = w.num_q_heads
    worst, margin = 0.0, np.inf
    for r, rows in _sample_rows(w, rng, nreq, nrows):
        heads = sorted({0, Hq - 1} | set(int(x) for x in rng.choice(Hq, size=min(Hq, nheads), replace=False)))
        got_rows = {h: got[int(w.q_start[r]) + np.asarray(rows), h, :] for h in heads}
        m = int(w.q_end[r] - w.q_start[r])
        ctrl = int(w.kv_len[r]) - m >= sampled.STEP
        e, mg = sampled.check_request(w, r, rows, heads, got_rows, TOL[w.dtype], with_controls=ctrl)
        worst = max(worst, e)
        if mg is not None:
            margin = min(margin, mg)
    _say(f"[parity] focused full {label}: sampled max|gpu-oracle| = {worst:.3e}; "
         f"smallest negative-control error {margin:.3e}")
    assert margin > TOL[w.dtype]
    return worst


FOCUSED = [("decode-heavy", 3, 0), ("decode-heavy split-KV", 3, api.VA_FLAG_NO_DECODE_TILES), ("chunk-mix", 4, 0),
           ("long-prefix-chunk", 9, 0), ("shared-64", 51, api.VA_FLAG_SHARED_PREFIX), ("spec-decode-mtp7", 7, 0),
           ("orca-mixed", 2, 0)]


@pytest.mark.parametrize("label,cid,flags", FOCUSED, ids=[f[0] for f in FOCUSED])
def test_parity_full_size_focused(label, cid, flags):
    """The full-size workloads on the focused companion inputs (attention concentrated on a
    few keys spread over each context, outputs O(1)): sampled rows against the oracle, with
    negative controls showing the comparison would catch a lost or doubled key step."""
    w = _focused(cid)
    _say(f"[gpu] run full focused {label}: reqs={w.num_reqs} rows={w.total_q_rows}")
    out, plan = api.run_workload(w, flags=flags)
    _focused_check(w, out, label, 300 + cid)


def _raw_gather(w):
    """Logical-order K and V of every request by numpy fancy indexing (raw bits)."""
    ks, vs = [], []
    for r in range(w.num_reqs):
        j = np.arange(int(w.kv_len[r]))
        pages = w.block_table[r][j // w.page_size]
        slots = j % w.page_size
        ks.append(w.k_pool[pages, :, slots, :])                       # [L, Hkv, D]
        vs.append(w.v_pool[pages, :, :, slots])                      # [L, Hkv, D]
    return np.concatenate(ks), np.concatenate(vs)


@pytest.mark.parametrize("cid,scale", [(1, 1), (2, 1), (3, 8), (5, 1)])
def test_gather_bit_exact(cid, scale):
    import torch
    w = W.config(cid, scale=scale, poison_tail=True)
    _say(f"[gpu] gather config {cid}/{scale}")
    plan = api.plan_for(w)
    q, k, v, bt = api.to_device(w)
    total = int(w.kv_len.sum())
    ko = torch.empty(total, w.num_kv_heads, w.head_dim, dtype=k.dtype, device="cuda")
    vo = torch.empty_like(ko)
    api.varlen_attn_debug_gather(plan, k, v, bt, ko, vo)
    torch.cuda.synchronize()
    kr, vr = _raw_gather(w)
    view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if w.dtype == "bf16" else \
        (lambda t: t.cpu().numpy())
    gk, gv = view(ko), view(vo)
    assert gk.shape == kr.shape and gv.shape == vr.shape
    assert np.array_equal(gk.view(np.uint8), np.ascontiguousarray(kr).view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), np.ascontiguousarray(vr).view(np.uint8))


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.int32)


def test_page_permutation_bitwise():
    """Physical page placement changes no output bit (same plan shape, same kernel order)."""
    w = W.config(2, scale=4)
    _say("[gpu] page permutation")
    a, _ = api.run_workload(w)
    perm = np.random.default_rng(5).permutation(w.num_pages)
    w2 = W.Workload(**{**w.__dict__})
    w2.k_pool = np.empty_like(w.k_pool)
    w2.v_pool = np.empty_like(w.v_pool)
    w2.k_pool[perm] = w.k_pool
    w2.v_pool[perm] = w.v_pool
    bt = w.block_table.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    w2.block_table = bt
    b, _ = api.run_workload(w2)
    assert np.array_equal(_bits(a), _bits(b))


def test_request_isolation_bitwise():
    w = W.config(3, scale=8)
    _say("[gpu] isolation")
    a, _ = api.run_workload(w)
    w2 = W.Workload(**{**w.__dict__})
    w2.q = w.q.copy()
    w2.k_pool = w.k_pool.copy()
    w2.v_pool = w.v_pool.copy()
    r = 3
    w2.q[w.q_start[r]:w.q_end[r]] ^= np.uint16(0x0040)
    npg = (int(w.kv_len[r]) + w.page_size - 1) // w.page_size
    pages = w.block_table[r, :npg]
    w2.k_pool[pages] ^= np.uint16(0x0040)
    w2.v_pool[pages] ^= np.uint16(0x0040)
    b, _ = api.run_workload(w2)
    A, B = _bits(a), _bits(b)
    others = np.ones(w.total_q_rows, bool)
    others[w.q_start[r]:w.q_end[r]] = False
    assert np.array_equal(A[others], B[others])
    assert not np.array_equal(A[~others], B[~others])


def test_deterministic():
    w = W.config(4, scale=8)
    _say("[gpu] determinism")
    a, plan = api.run_workload(w)
    b, _ = api.run_workload(w, plan=plan)
    assert np.array_equal(_bits(a), _bits(b))


EDGE = [
    ("gap+zero-row+kv1", dict(q_rows=[3, 0, 1, 1, 5], kv=[3, 9, 1, 2, 40], hq=4, hkv=4, d=64, ps=16)),
    ("g16-multi-row", dict(q_rows=[3, 1], kv=[700, 257], hq=32, hkv=2, d=128, ps=256)),
    ("mtp-g8-ps32", dict(q_rows=[5, 4, 1], kv=[300, 64, 31], hq=16, hkv=2, d=128, ps=32)),
    ("long-decode", dict(q_rows=[1, 1], kv=[40000, 77], hq=8, hkv=1, d=128, ps=64)),
    ("d64-bf16-prefill", dict(q_rows=[130, 2], kv=[200, 2], hq=6, hkv=3, d=64, ps=16)),
    ("f32-d128", dict(q_rows=[17, 1], kv=[40, 90], hq=4, hkv=2, d=128, ps=16, dtype="f32")),
    # prefill tiles plus decode items written directly (short kv) and split (long kv)
    ("prefill+direct+split", dict(q_rows=[600, 1, 1, 1], kv=[700, 100, 160, 30000], hq=8, hkv=2, d=128, ps=32)),
]


@pytest.mark.parametrize("label,spec", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(label, spec):
    import torch
    w = W.build(label, spec["q_rows"], spec["kv"], num_q_heads=spec["hq"], num_kv_heads=spec["hkv"],
                head_dim=spec["d"], page_size=spec["ps"], dtype=spec.get("dtype", "bf16"), seed=17,
                poison_tail=True, extra_pages=2)
    # leave two untouched rows between requests 0 and 1
    w.q_start = w.q_start.copy()
    w.q_end = w.q_end.copy()
    w.q_start[1:] += 2
    w.q_end[1:] += 2
    w.q = np.concatenate([w.q[:w.q_end[0]], np.zeros((2,) + w.q.shape[1:], w.q.dtype), w.q[w.q_end[0]:]])
    _say(f"[gpu] edge {label}")
    plan = api.plan_for(w)
    q, k, v, bt = api.to_device(w)
    out = torch.full_like(q, 7.0)
    ws = api.new_workspace(plan)
    api.varlen_attn_run(plan, q, k, v, bt, out, ws)
    torch.cuda.synchronize()
    _check_full(w, out, label)
    gap = out[w.q_end[0]:w.q_start[1]].float().cpu().numpy()
    assert (gap == 7.0).all(), "rows outside every request were written"


def test_run_errors():
    import torch
    w = W.config(1)
    plan = api.plan_for(w, split_len=64)      # several parts per output: a workspace is needed
    assert plan.workspace_bytes > 0
    q, k, v, bt = api.to_device(w)
    out = torch.zeros_like(q)
    small = torch.empty(max(1, plan.workspace_bytes - 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(api.VarlenAttnError) as ei:
        api.varlen_attn_run(plan, q, k, v, bt, out, small)
    assert ei.value.status == api.VA_ERR_WORKSPACE_TOO_SMALL
    L = api.lib()
    assert L.varlen_attn_run(plan.handle, None, None, None, None, None, None, 0, None) == api.VA_ERR_INVALID_ARG


# ------------------------------------------------------------------ KV append --

def _new_rows_kv(w):
    """The new rows' K/V ([total_q_rows, Hkv, D], raw element bits) read from the pools by
    the definition: row q_start[r] + i is position kv_len[r] - q_rows + i."""
    k_new = np.zeros((w.total_q_rows, w.num_kv_heads, w.head_dim), w.k_pool.dtype)
    v_new = np.zeros_like(k_new)
    for r in range(w.num_reqs):
        m = int(w.q_end[r] - w.q_start[r])
        S0 = int(w.kv_len[r]) - m
        for i in range(m):
            pos = S0 + i
            page, slot = w.block_table[r][pos // w.page_size], pos % w.page_size
            k_new[w.q_start[r] + i] = w.k_pool[page, :, slot, :]
            v_new[w.q_start[r] + i] = w.v_pool[page, :, :, slot]
    return k_new, v_new


def _to_dev(a):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).cuda()


def _raw(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.cpu().numpy()


APPEND_LAYOUTS = {
    # new rows starting mid-page: every V column written element by element
    "mid-page": ([37, 1, 5, 0, 200], [90, 300, 5, 10, 200]),
    # an uncached prefill first: its tokens fill whole pages from slot 0 (16-byte V stores)
    "page-aligned": ([200, 37, 1, 5, 0], [200, 90, 300, 5, 10]),
}


@pytest.mark.parametrize("layout", list(APPEND_LAYOUTS))
@pytest.mark.parametrize("dtype,d,ps", [("bf16", 128, 16), ("bf16", 64, 64), ("f32", 128, 32), ("bf16", 128, 256)])
def test_append_bit_exact(dtype, d, ps, layout):
    """GPU append == oracle append, bit for bit, with padding (-1) and random new values."""
    import torch
    q_rows, kv = APPEND_LAYOUTS[layout]
    w = W.build("ap", q_rows, kv, num_q_heads=8, num_kv_heads=4, head_dim=d,
                page_size=ps, dtype=dtype, seed=23, extra_pages=3)
    _say(f"[gpu] append {dtype} d={d} ps={ps} {layout}")
    plan = api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    loc = api.varlen_attn_plan_slots(plan)
    rng = np.random.default_rng(5)
    shape = (w.total_q_rows, w.num_kv_heads, w.head_dim)
    if dtype == "bf16":
        k_new = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        v_new = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    else:
        k_new = rng.standard_normal(shape).astype(np.float32)
        v_new = rng.standard_normal(shape).astype(np.float32)
    loc[3] = -1                                          # a padding row inside a request
    want_k, want_v = oracle.append_kv(w.k_pool, w.v_pool, k_new, v_new, loc, w.page_size)
    kp, vp = _to_dev(w.k_pool), _to_dev(w.v_pool)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.varlen_attn_append_kv(num_kv_heads=w.num_kv_heads, head_dim=d, page_size=ps, num_pages=w.num_pages,
                              k_new=_to_dev(k_new), v_new=_to_dev(v_new), out_cache_loc=torch.from_numpy(loc).cuda(),
                              k_pool=kp, v_pool=vp, bad_loc_count=bad, dtype=dtype)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert np.array_equal(_raw(kp).view(np.uint8), np.ascontiguousarray(want_k).view(np.uint8))
    assert np.array_equal(_raw(vp).view(np.uint8), np.ascontiguousarray(want_v).view(np.uint8))


def test_append_out_of_range_counted_and_skipped():
    import torch
    w = W.build("ob", [4], [20], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, seed=3)
    _say("[gpu] append out of range")
    n = w.num_pages * w.page_size
    loc = np.array([n, 5, n + 100, 17], np.int64)
    k_new = np.full((4, 2, 64), 0x3F80, np.uint16)
    v_new = np.full((4, 2, 64), 0x4000, np.uint16)
    want_k, want_v = oracle.append_kv(w.k_pool, w.v_pool, k_new, v_new, np.where(loc < n, loc, -1), w.page_size)
    kp, vp = _to_dev(w.k_pool), _to_dev(w.v_pool)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.varlen_attn_append_kv(num_kv_heads=2, head_dim=64, page_size=16, num_pages=w.num_pages, k_new=_to_dev(k_new),
                              v_new=_to_dev(v_new), out_cache_loc=torch.from_numpy(loc).cuda(), k_pool=kp, v_pool=vp,
                              bad_loc_count=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 2
    assert np.array_equal(_raw(kp), want_k) and np.array_equal(_raw(vp), want_v)


@pytest.mark.parametrize("cid,scale", [(2, 8), (4, 16), (3, 16)])
def test_append_then_attend(cid, scale):
    """Poison the new rows' slots, append their K/V on the GPU, run attention: the result
    matches the oracle on the original pools (the append puts every new row where the
    attention reads it)."""
    import torch
    w = W.config(cid, scale=scale)
    _say(f"[gpu] append then attend config {cid}/{scale}")
    plan = api.plan_for(w)
    loc = api.varlen_attn_plan_slots(plan)
    k_new, v_new = _new_rows_kv(w)
    poison = np.uint16(0x7FC0) if w.dtype == "bf16" else np.float32(np.nan)
    kb, vb = w.k_pool.copy(), w.v_pool.copy()
    for l in loc[loc >= 0]:
        kb[l // w.page_size, :, l % w.page_size, :] = poison
        vb[l // w.page_size, :, :, l % w.page_size] = poison
    q, _, _, bt = api.to_device(w)
    kp, vp = _to_dev(kb), _to_dev(vb)
    api.varlen_attn_append_kv(num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                              num_pages=w.num_pages, k_new=_to_dev(k_new), v_new=_to_dev(v_new),
                              out_cache_loc=torch.from_numpy(loc).cuda(), k_pool=kp, v_pool=vp, dtype=w.dtype)
    out = torch.zeros_like(q)
    api.varlen_attn_run(plan, q, kp, vp, bt, out, api.new_workspace(plan))
    torch.cuda.synchronize()
    assert np.array_equal(_raw(kp).view(np.uint8), np.ascontiguousarray(w.k_pool).view(np.uint8))
    assert np.array_equal(_raw(vp).view(np.uint8), np.ascontiguousarray(w.v_pool).view(np.uint8))
    _check_full(w, out, f"append+attend {cid}/{scale}")


def _uneven(kind, dtype=None):
    """Decodes whose tables share runs of pages unevenly (the planner's shared-prefix groups
    then follow the tree of common runs)."""
    dtype = dtype or "bf16"
    if kind == "many-nested":
        # 64 decodes of 2048 positions, g = 4, 8 KV heads: all share 8 pages, requests 0-31
        # share 24, requests 32-63 share 16 (members' own keys then run as tiles)
        w = W.build("many-nested", [1] * 64, [2048] * 64, num_q_heads=32, num_kv_heads=8, head_dim=128,
                    page_size=64, seed=31, dtype=dtype)
        return W.share_runs(w, [(0, list(range(1, 64)), 0, 8), (0, list(range(1, 32)), 8, 24),
                                (32, list(range(33, 64)), 8, 16)])
    if kind == "leader-outlier":
        w = W.build("leader-outlier", [1] * 6, [900] * 6, num_q_heads=8, num_kv_heads=2, head_dim=64,
                    page_size=16, seed=9, dtype=dtype)
        return W.share_runs(w, [(3, [1, 2, 4, 5], 0, 40), (3, [0], 0, 1)])
    w = W.build(f"uneven-{kind}", [1] * 8, [1500] * 8, num_q_heads=16, num_kv_heads=4, head_dim=128,
                page_size=64, seed=7, dtype=dtype)
    if kind == "outlier":
        return W.share_runs(w, [(1, [2, 3, 4, 5, 6, 7], 0, 16), (1, [0], 0, 1)])
    return W.share_runs(w, [(0, [1, 2, 3], 0, 16), (0, [4, 5, 6, 7], 0, 4), (4, [5, 6, 7], 4, 12)])


@pytest.mark.parametrize("kind,dtype", [("outlier", None), ("nested", None), ("leader-outlier", None),
                                        ("many-nested", None), ("nested", "fp8")])
def test_shared_prefix_uneven_groups_elementwise(kind, dtype):
    """Shared-prefix groups chosen over the tree of common page runs, elementwise against the
    oracle (fp8 pools: against the dequantised pools, at the fp8 tolerance)."""
    base = _uneven(kind, dtype)
    # the N(0,1) input and its focused companion (O(1) outputs: a lost or doubled key range
    # of a group would move them far past the tolerance)
    for w in (base, W.focus(base)):
        _say(f"[gpu] shared-prefix uneven groups {w.name} {w.dtype}")
        out, plan = api.run_workload(w, flags=api.VA_FLAG_SHARED_PREFIX)
        st = api.varlen_attn_plan_stats(plan)
        assert st["shared_groups"] >= 1 and st["shared_tiles"] > 0, st
        got = out.float().cpu().numpy().astype(np.float64)
        if dtype == "fp8":
            K, V = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
            tol = 1e-2
        else:
            K, V, tol = w.k_pool, w.v_pool, TOL[w.dtype]
        ref = oracle.varlen_paged_attention(w.q, K, V, w.block_table, w.q_start, w.q_end, w.kv_len, w.page_size)
        e = float(np.abs(got - ref).max())
        _say(f"[parity] shared-prefix uneven {w.name} {w.dtype} ({st['shared_groups']} groups, "
             f"{st['shared_tiles']} group tiles; max|oracle| = {np.abs(ref).max():.2f}): "
             f"max|gpu-oracle| = {e:.3e} (tol {tol})")
        assert np.isfinite(got).all() and e <= tol


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_shared_prefix_multirow_members_in_key_chunks_elementwise(dtype):
    """Six members of a 4096-key shared prefix, each with 15 verify rows (60 columns per KV
    head) and 1032 private keys: the private keys run as column-list tiles cut into 256-key
    chunks, and since the last 8 keys lie past some rows' limits the last chunk starts where
    every row still sees keys and runs on through the diagonal (fp8: the private keys are
    small, so they ride in the same launch too)."""
    base = W.build(f"shared-mtp15-{dtype}", [15] * 6, [4096 + 1032] * 6, num_q_heads=32, num_kv_heads=8,
                   head_dim=128, page_size=64, seed=31, shared_prefix_pages=64, dtype=dtype, poison_tail=True)
    for w in (base, W.focus(base)):
        _say(f"[gpu] shared-prefix multi-row members {w.name} {w.dtype}")
        out, plan = api.run_workload(w, flags=api.VA_FLAG_SHARED_PREFIX)
        st = api.varlen_attn_plan_stats(plan)
        tiles = api.varlen_attn_plan_export(plan, 3)
        own = tiles[(tiles[:, 10] & 1) == 1]
        own = own[own[:, 11] == 0]                       # column-list tiles of private keys
        assert st["shared_groups"] == 1 and st["split_items"] == 0 and len(own) == 6 * 8 * 4, st
        assert set((own[:, 6] - own[:, 7]).tolist()) == {256, 264}   # three 256-key chunks, the last 264
        got = out.float().cpu().numpy().astype(np.float64)
        if dtype == "fp8":
            K, V = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
            tol = 1e-2
        else:
            K, V, tol = w.k_pool, w.v_pool, TOL[w.dtype]
        ref = oracle.varlen_paged_attention(w.q, K, V, w.block_table, w.q_start, w.q_end, w.kv_len, w.page_size)
        e = float(np.abs(got - ref).max())
        _say(f"[parity] shared-prefix multi-row members {w.name} {w.dtype}: max|gpu-oracle| = {e:.3e} (tol {tol})")
        assert np.isfinite(got).all() and e <= tol


def test_readme_example_runs():
    """The usage example in README.md runs as printed and its output matches the oracle."""
    import os
    import re
    import torch
    text = open(os.path.join(os.path.dirname(__file__), "..", "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    bt = env["block_table"]
    K = env["k_pool"].float().cpu().numpy().astype(np.float64)
    V = env["v_pool"].float().cpu().numpy().astype(np.float64)
    Q = env["q"].float().cpu().numpy().astype(np.float64)
    ref = oracle.varlen_paged_attention(Q, K, V, bt, np.array(env["q_start"]), np.array(env["q_end"]),
                                        np.array(env["kv_len"]), env["ps"])
    e = float(np.abs(env["out"].float().cpu().numpy() - ref).max())
    _say(f"[parity] README example: max|gpu-oracle| = {e:.3e}")
    assert e <= TOL["bf16"]

