"""CPU tests of the C-ABI library: it loads, exports what the header declares, validates
metadata, and plans work that covers every visible (row, head, position) exactly once.
No compute call is made (plans are built with VA_FLAG_HOST_ONLY)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from varlen_paged_attention_amd import api, workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = api.VA_FLAG_HOST_ONLY


def _declared_functions():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(varlen_attn_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    L = api.lib()
    declared = _declared_functions()
    assert len(declared) >= 8
    for name in declared:
        assert hasattr(L, name), f"{name} declared in include/ but not exported"
    assert sorted(api.EXPORTED) == declared


def _plan(w, flags=HOST, **kw):
    return api.plan_for(w, flags=flags | HOST, **kw)


def _small():
    return W.build("s", [5, 1, 3], [9, 40, 3], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, seed=1)


def _expect(status, **over):
    w = _small()
    args = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, num_pages=w.num_pages,
                q_start=w.q_start, q_end=w.q_end, kv_len=w.kv_len, block_table=w.block_table, flags=HOST)
    args.update(over)
    with pytest.raises(api.VarlenAttnError) as ei:
        api.varlen_attn_plan(**args)
    assert ei.value.status == status, str(ei.value)
    return str(ei.value)


def test_plan_validation_errors():
    w = _small()
    E, U = api.VA_ERR_INVALID_ARG, api.VA_ERR_UNSUPPORTED
    assert "q_rows > kv_len" in _expect(E, kv_len=np.array([4, 40, 3]))
    assert "q_start" in _expect(E, q_end=np.array([4, 10, 13]) - 5)
    assert "overlap" in _expect(E, q_start=np.array([0, 4, 6]), q_end=np.array([5, 5, 9]))
    bt = w.block_table.copy()
    bt[1, 0] = w.num_pages
    assert "outside" in _expect(E, block_table=bt)
    bt[1, 0] = -1
    assert "outside" in _expect(E, block_table=bt)
    assert "max_pages_per_req" in _expect(E, kv_len=np.array([9, 16 * w.block_table.shape[1] + 1, 3]))
    assert "multiple" in _expect(E, num_q_heads=3)
    _expect(U, head_dim=96)
    _expect(U, page_size=24)
    _expect(E, num_pages=0)


def test_status_strings_and_null_args():
    L = api.lib()
    for s in (0, -1, -2, -3, -4, -5):
        assert L.varlen_attn_status_string(s)
    h = ctypes.c_void_p()
    assert L.varlen_attn_plan(None, 0, None, None, None, None, ctypes.byref(h), None) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_run(None, None, None, None, None, None, None, 0, None) == api.VA_ERR_INVALID_ARG
    p = _plan(_small())
    # a host-only plan refuses to run
    assert L.varlen_attn_run(p.handle, None, None, None, None, None, None, 0, None) == api.VA_ERR_INVALID_ARG
    assert b"HOST_ONLY" in L.varlen_attn_last_error()


def test_empty_and_zero_row_requests_plan():
    w = W.build("z", [0, 3, 0], [5, 7, 0], num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, seed=2)
    plan = _plan(w)
    st = api.varlen_attn_plan_stats(plan)
    items = api.varlen_attn_plan_export(plan, 0)
    direct_cols = int(sum(it[3] for it in items if it[7] & 2))
    assert st["combine_rows"] + direct_cols == 3 * 2
    assert st["visible_pairs"] == 3 * 4 + 6


def check_coverage(w, plan):
    """Every visible (row, head, position) is scored exactly once, by a prefill tile or by
    one split item, and the items' slots of each output are distinct and in range."""
    items = api.varlen_attn_plan_export(plan, 0)
    cols = api.varlen_attn_plan_export(plan, 1)
    comb = api.varlen_attn_plan_export(plan, 2)
    tiles = api.varlen_attn_plan_export(plan, 3)
    Hq, g, ps = w.num_q_heads, w.num_q_heads // w.num_kv_heads, w.page_size
    req_of_row = np.full(w.total_q_rows, -1)
    for r in range(w.num_reqs):
        req_of_row[w.q_start[r]:w.q_end[r]] = r
    cover = {}                 # (row, head) -> list of (k0, k1) intervals
    slots = {}
    comb_map = {(int(c[0]), int(c[1])): (int(c[2]), int(c[3])) for c in comb}
    direct = {}
    for it in items:
        req, kvh, col0, ncols, k0, k1, slot, flags = (int(x) for x in it)
        assert 1 <= ncols <= (16 if w.dtype == "f32" else 32) and k0 < k1 and k0 % 16 == 0   # 16-key runs in one page
        for c in cols[col0:col0 + ncols]:
            row, head, limit, pbase = (int(x) for x in c)
            r = req_of_row[row]
            assert head // g == kvh
            m = int(w.q_end[r] - w.q_start[r])
            assert limit == int(w.kv_len[r]) - m + (row - int(w.q_start[r]))
            # the table used must hold the column's own pages over [k0, min(k1, limit+1))
            hi = min(k1, limit + 1)
            if hi > k0:
                pages = range(k0 // ps, (hi - 1) // ps + 1)
                assert all(w.block_table[req, p] == w.block_table[r, p] for p in pages)
                cover.setdefault((row, head), []).append((k0, hi))
            if flags & 2:          # written directly: the item is the output's only part
                assert (row, head) not in comb_map and pbase == -1
                direct[(row, head)] = direct.get((row, head), 0) + 1
            else:
                pb, npart = comb_map[(row, head)]
                assert pb == pbase and 0 <= slot < npart
                slots.setdefault((row, head), []).append(slot)
            if not (flags & 1):
                assert k1 - 1 <= limit
    assert all(n == 1 for n in direct.values())
    assert not (set(direct) & set(slots))
    listed = api.varlen_attn_plan_export(plan, 4)          # copies of the column-list tiles
    assert len(listed) == (int((tiles[:, 10] & 1).sum()) if len(tiles) else 0)
    for t in tiles:
        if not t[10] & 1:
            continue
        # column-list tile: a shared-prefix group tile or a member's own keys after them
        req, kvh, col0, ncols, slot, k0, k1, kbeg = (int(x) for x in t[:8])
        assert kbeg == k0 and t[8] == -1
        assert 1 <= ncols <= 128 and k0 < k1
        for c in cols[col0:col0 + ncols]:
            row, head, limit, pbase = (int(x) for x in c)
            r = req_of_row[row]
            assert head // g == kvh and k0 <= limit
            hi = min(k1, limit + 1)
            pages = range(k0 // ps, (hi - 1) // ps + 1)
            assert all(w.block_table[req, p] == w.block_table[r, p] for p in pages)
            cover.setdefault((row, head), []).append((k0, hi))
            pb, npart = comb_map[(row, head)]
            assert pb == pbase and 0 <= slot < npart
            slots.setdefault((row, head), []).append(slot)
    for t in tiles:
        if t[10] & 1:
            continue
        req, kvh, c0, ncols, q0, S0, kv_end, kbeg, pbase, pstride = (int(x) for x in t[:10])
        assert kbeg % 64 == 0 and 1 <= ncols <= 128
        for col in range(ncols):
            i, hh = divmod(c0 + col, g)
            row, head = q0 + i, kvh * g + hh
            assert kbeg <= S0 + i, "a key chunk with no visible key for a column"
            if pbase < 0:                                  # whole tile: output written directly
                assert kbeg == 0 and kv_end >= S0 + i + 1 and (row, head) not in comb_map
                cover.setdefault((row, head), []).append((0, S0 + i + 1))
            else:                                          # one key chunk of a cut tile
                cover.setdefault((row, head), []).append((kbeg, min(kv_end, S0 + i + 1)))
                pb, npart = comb_map[(row, head)]
                assert 0 <= pbase + col * pstride - pb < npart and npart == pstride
                slots.setdefault((row, head), []).append(pbase + col * pstride - pb)
    for (row, head), s in slots.items():
        assert len(s) == len(set(s)), f"slot reused for {(row, head)}"
    for r in range(w.num_reqs):
        m = int(w.q_end[r] - w.q_start[r])
        S0 = int(w.kv_len[r]) - m
        for i in range(m):
            for h in range(Hq):
                iv = sorted(cover.get((int(w.q_start[r]) + i, h), []))
                assert iv, f"row {i} head {h} of request {r} not covered"
                assert iv[0][0] == 0 and iv[-1][1] == S0 + i + 1
                for a, b in zip(iv, iv[1:]):
                    assert a[1] == b[0], f"gap/overlap {a} {b}"


CASES = [
    ("tiny", lambda: W.config(1), 0),
    ("orca-small", lambda: W.config(2, scale=16), 0),
    ("orca-small-split-only", lambda: W.config(2, scale=16), api.VA_FLAG_NO_PREFILL_KERNEL),
    ("decode", lambda: W.config(3, scale=16), 0),
    ("chunk-mix", lambda: W.config(4, scale=16), 0),
    ("shared", lambda: W.config(5), api.VA_FLAG_SHARED_PREFIX),
    ("shared-scaled", lambda: W.config(51, scale=8), api.VA_FLAG_SHARED_PREFIX),
    ("shared-split-items", lambda: W.config(5), api.VA_FLAG_SHARED_PREFIX | api.VA_FLAG_NO_PREFILL_KERNEL),
    ("mtp-g8", lambda: W.build("m", [4, 3, 1], [100, 64, 33], num_q_heads=16, num_kv_heads=2, head_dim=128,
                               page_size=32, seed=3), 0),
    ("prefill+decodes", lambda: W.build("fd", [2048, 1, 1, 1], [2048, 100, 160, 3000], num_q_heads=8, num_kv_heads=2,
                                     head_dim=128, page_size=32, seed=4), 0),
    ("orca-full", lambda: W.config(2), 0),
    ("chunk-like", lambda: W.build("cl", [2048, 1, 1, 1, 1], [32768, 600, 5000, 16384, 70], num_q_heads=8,
                                   num_kv_heads=1, head_dim=128, page_size=64, seed=5), 0),
    ("spec-decode-mtp3", lambda: W.config(6, scale=16), 0),
    ("spec-decode-mtp7", lambda: W.config(7, scale=16), 0),
    ("orca-small-fp8", lambda: W.config(2, scale=16, dtype="fp8"), 0),
    ("decode-fp8", lambda: W.config(3, scale=16, dtype="fp8"), 0),
    ("shared-fp8", lambda: W.config(5, dtype="fp8"), api.VA_FLAG_SHARED_PREFIX),
    ("long-prefix-chunk", lambda: W.config(9), 0),
    ("long-prefix-chunk/8", lambda: W.config(9, scale=8), 0),
]


@pytest.mark.parametrize("name,make,flags", CASES, ids=[c[0] for c in CASES])
def test_plan_covers_every_visible_pair_once(name, make, flags):
    w = make()
    check_coverage(w, _plan(w, flags))


FOLD_CASES = [
    # (name, workload, flags, short requests expected on tiles)
    ("decode-heavy", lambda: W.config(3), 0, True),                       # 2048 tiles fill 512 slots
    ("decode-heavy no-decode-tiles", lambda: W.config(3), api.VA_FLAG_NO_DECODE_TILES, False),
    ("decode-heavy/16", lambda: W.config(3, scale=16), 0, False),          # 128 tiles: items stay
    ("decode-heavy fp8", lambda: W.config(3, dtype="fp8"), 0, False),      # fp8 tiles widen every code
    # fp8 plans with prefill tiles take their decodes into that launch when the decodes' KV is
    # small: ORCA's two (27 MB of codes and scales) ride as tiles, the chunk mix's 64 (1.15 GB)
    # stay items
    ("orca fp8", lambda: W.config(2, dtype="fp8"), 0, True),
    ("chunk-mix fp8", lambda: W.config(4, dtype="fp8"), 0, False),
    ("spec-decode-mtp7", lambda: W.config(7), 0, True),
    ("orca", lambda: W.config(2), 0, True),
    ("few long decodes (cut)", lambda: W.build("fl", [1] * 4, [32768] * 4, num_q_heads=32, num_kv_heads=8,
                                               head_dim=128, page_size=64, seed=3), 0, True),
    # members' own keys after the shared pages: column-list tiles (bf16; fp8 when their codes
    # and scales are small), else split items
    ("shared-prefix-64", lambda: W.config(51), api.VA_FLAG_SHARED_PREFIX, True),
    ("shared-prefix-64 fp8", lambda: W.config(51, dtype="fp8"), api.VA_FLAG_SHARED_PREFIX, False),
    # 6 members: their private keys (13 MB of codes and scales) ride in the group tiles' launch
    ("shared-prefix-6", lambda: W.config(5), api.VA_FLAG_SHARED_PREFIX, True),
    ("shared-prefix-6 fp8", lambda: W.config(5, dtype="fp8"), api.VA_FLAG_SHARED_PREFIX, True),
]


@pytest.mark.parametrize("name,make,flags,folded", FOLD_CASES, ids=[c[0] for c in FOLD_CASES])
def test_short_requests_as_tiles(name, make, flags, folded):
    w = make()
    plan = _plan(w, flags)
    st = api.varlen_attn_plan_stats(plan)
    m = w.q_end - w.q_start
    g = w.num_q_heads // w.num_kv_heads
    short = [r for r in range(w.num_reqs) if 0 < m[r] and m[r] * g < 64]
    tiles = api.varlen_attn_plan_export(plan, 3)
    # tiles scoring a request's own keys (not a shared-prefix group tile: record field 11, "group")
    on_tiles = set(int(t[0]) for t in tiles if not (t[10] & 1 and t[11]))
    if folded:
        assert all(r in on_tiles for r in short) and st["split_items"] == 0
        assert st["prefill_tiles"] >= 512
    else:
        assert not any(r in on_tiles for r in short) and st["split_items"] > 0
    check_coverage(w, plan)


@pytest.mark.parametrize("cid,tp,dp", [(4, 8, 1), (2, 8, 1), (3, 1, 8), (51, 1, 8)])
def test_one_gpu_share_of_a_workload(cid, tp, dp):
    """One GPU's share under tensor parallelism (heads / tp, at least one KV head) or data
    parallelism (every dp-th request) plans and covers every visible pair."""
    full = W.config(cid, scale=16)
    w = W.config(cid, scale=16, tp=tp, dp=dp)
    assert w.num_q_heads == full.num_q_heads // tp
    assert w.num_kv_heads == max(1, full.num_kv_heads // tp)
    assert w.num_reqs == len(range(0, full.num_reqs, dp))
    assert np.array_equal(w.kv_len, full.kv_len[::dp])
    flags = api.VA_FLAG_SHARED_PREFIX if cid == 51 else 0
    check_coverage(w, _plan(w, flags))


def _long_chunk(m=256, S0=65536, hq=32, hkv=8, extra=()):
    """A chunk of m new rows on S0 cached positions (plus optional decodes)."""
    rows = [m] + [1] * len(extra)
    return W.build("lc", rows, [S0 + m] + list(extra), num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                   page_size=64, seed=6)


CUT_CASES = [
    # (name, workload, prefill_split_len, expect cut tiles)
    ("forced-1000", lambda: W.build("c", [300, 1, 40], [5000, 77, 2100], num_q_heads=8, num_kv_heads=2,
                                    head_dim=128, page_size=16, seed=7), 1000, True),
    ("forced-g1", lambda: W.build("c", [130, 64], [700, 64], num_q_heads=2, num_kv_heads=2, head_dim=64,
                                  page_size=32, seed=8), 64, True),
    ("auto-long-chunk", lambda: _long_chunk(), 0, True),
    ("auto-long-chunk+decodes", lambda: _long_chunk(512, 131072, 64, 8, extra=(900, 40000, 3)), 0, True),
    ("auto-long-prefix-chunk+64-decodes", lambda: W.config(9), 0, True),
    ("auto-orca-stays-whole", lambda: W.config(2), 0, False),
    ("auto-chunk-mix-stays-whole", lambda: W.config(4), 0, False),
    ("never", lambda: _long_chunk(), -1, False),
]


@pytest.mark.parametrize("name,make,split,cut", CUT_CASES, ids=[c[0] for c in CUT_CASES])
def test_cut_prefill_tiles_cover_every_visible_pair_once(name, make, split, cut):
    w = make()
    plan = _plan(w, prefill_split_len=split)
    st = api.varlen_attn_plan_stats(plan)
    assert (st["prefill_split_tiles"] > 0) == cut
    check_coverage(w, plan)
    tiles = api.varlen_attn_plan_export(plan, 3)
    work = tiles[:, 6] - tiles[:, 7]
    if cut and split > 0:
        L = -(-split // 64) * 64
        assert np.all(work[tiles[:, 8] >= 0] <= L + 128)   # the last chunk also holds the diagonal
    if name == "auto-long-prefix-chunk+64-decodes":
        # the 64 tiles of 256 rows x 4 heads on 65,536 cached keys take 8192-key chunks (4096
        # models about as fast but measured 7 % slower); the decode tiles (<= 16,384 keys,
        # i.e. <= 2 chunks) stay whole
        assert st["prefill_split_tiles"] == 512 and st["prefill_tiles"] == 512 + 64 * 8
        assert set((tiles[tiles[:, 8] >= 0, 7] % 8192).tolist()) == {0}
    if name == "auto-long-chunk":
        # 64 tiles of ~65.8K keys on 512 resident slots: chunks of 8192 keys (the largest
        # power of two <= 64 * 65.8K / 512), 8 per tile (the remainder of 1 key is absorbed)
        assert st["prefill_tiles"] == 512 and st["prefill_split_tiles"] == 512
        assert st["combine_rows"] == 256 * 32
        assert sorted(set((tiles[:, 7] // 8192).tolist())) == list(range(8))
        # 64 groups of 8 tiles reading one key chunk of one KV head, 8 groups per XCD:
        # every group sits at launch positions of one XCD (position % 8); each XCD's first
        # 32 positions (one per CU) hold its heaviest tiles heaviest first, the next 32 (each
        # CU's second slot) the rest of its 64 heaviest lightest first, so that XCD positions
        # c and c + 32, which start on one CU, pair heavy with light; later positions heaviest
        # first
        xcd = {}
        for p, t in enumerate(tiles):
            assert xcd.setdefault((int(t[1]), int(t[7])), p % 8) == p % 8
        for x in range(8):
            wx = work[x::8]
            assert np.array_equal(np.concatenate([wx[:32], wx[32:64][::-1]]), np.sort(wx[:64])[::-1])
            assert np.all(np.diff(wx[64:]) <= 0) and (len(wx) <= 64 or wx[64:].max() <= wx[:64].min())


@pytest.mark.parametrize("name,make,flags", CASES, ids=[c[0] for c in CASES])
def test_plan_counters_match_oracle(name, make, flags):
    w = make()
    st = api.varlen_attn_plan_stats(_plan(w, flags))
    m = w.q_end - w.q_start
    assert st["visible_pairs"] == oracle.visible_pairs(m, w.kv_len)
    assert st["flops"] == oracle.attention_flops(m, w.kv_len, w.num_q_heads, w.head_dim)
    assert st["logical_kv_bytes"] == oracle.logical_kv_bytes(w.kv_len, w.num_kv_heads, w.head_dim, w.elem_bytes,
                                                             scale_bytes=w.scale_bytes)
    assert st["physical_kv_bytes"] == oracle.physical_kv_bytes(w.block_table, w.kv_len, w.page_size,
                                                               w.num_kv_heads, w.head_dim, w.elem_bytes,
                                                               scale_bytes=w.scale_bytes)
    if w.dtype == "fp8":
        assert st["q_bytes"] == int(m.sum()) * w.num_q_heads * w.head_dim * 2      # bf16 rows


def test_shared_prefix_groups_found():
    w = W.config(5)
    st = api.varlen_attn_plan_stats(_plan(w, api.VA_FLAG_SHARED_PREFIX))
    assert st["shared_groups"] == 1 and st["shared_tiles"] > 0 and st["shared_items"] == 0
    assert st["physical_kv_bytes"] == 40 * 2 ** 20 and st["logical_kv_bytes"] == 120 * 2 ** 20
    assert st["shared_tile_flops"] == 4 * 128 * (6 * 4) * 4096 * 8
    # the private ranges run as column-list tiles in the same launch: 128 group tiles (256-key
    # chunks of the 4096 shared keys, 8 KV heads) leave 384 of the 512 resident slots, so the
    # 6 x 8 private ranges of 1024 keys are cut into 128-key chunks (384 tiles); no split items
    assert st["split_items"] == 0 and st["split_item_kv_bytes"] == 0 and st["split_item_flops"] == 0
    assert st["prefill_tiles"] == 128 + 6 * 8 * 1024 // 128
    # with 64 members the 256 group tiles leave 256 slots, and the 512 private ranges stay
    # whole tiles (cut, they would need 2048-key chunks)
    st64 = api.varlen_attn_plan_stats(_plan(W.config(51), api.VA_FLAG_SHARED_PREFIX))
    assert st64["split_items"] == 0 and st64["split_item_kv_bytes"] == 0 and st64["split_item_flops"] == 0
    assert st64["prefill_tiles"] == 256 + 64 * 8
    # decode tiles off: the private ranges are split-KV items reading only those ranges
    # (6 x 1024 positions, 8 KV heads, K and V, bf16)
    sti = api.varlen_attn_plan_stats(_plan(w, api.VA_FLAG_SHARED_PREFIX | api.VA_FLAG_NO_DECODE_TILES))
    assert sti["split_item_kv_bytes"] == 6 * 1024 * 8 * 128 * 2 * 2
    assert sti["split_item_flops"] == 4 * 128 * 32 * 6 * 1024
    st0 = api.varlen_attn_plan_stats(_plan(w))
    assert st0["shared_groups"] == 0 and st0["split_item_kv_bytes"] == st0["physical_kv_bytes"]


def _uneven_sharing(kind):
    """Eight decodes (g = 4, page 64, 23 full pages each) whose tables share runs of pages
    unevenly: "outlier" -- requests 1-7 share 16 pages, request 0 only the first;
    "nested" -- all share 4 pages, requests 0-3 share 16, requests 4-7 share 12."""
    w = W.build(f"uneven-{kind}", [1] * 8, [1500] * 8, num_q_heads=16, num_kv_heads=4, head_dim=128,
                page_size=64, seed=7)
    if kind == "outlier":
        return W.share_runs(w, [(1, [2, 3, 4, 5, 6, 7], 0, 16), (1, [0], 0, 1)])
    return W.share_runs(w, [(0, [1, 2, 3], 0, 16), (0, [4, 5, 6, 7], 0, 4), (4, [5, 6, 7], 4, 12)])


def _groups_of(w, plan):
    """{requests of a group: its shared keys} from the plan's group tiles."""
    tiles = api.varlen_attn_plan_export(plan, 3)
    cols = api.varlen_attn_plan_export(plan, 1)
    req_of_row = {}
    for r in range(w.num_reqs):
        for row in range(int(w.q_start[r]), int(w.q_end[r])):
            req_of_row[row] = r
    groups = {}
    for t in tiles:
        if t[10] & 1 and t[11] == 1:
            col0, ncols, k1 = int(t[2]), int(t[3]), int(t[6])
            reqs = frozenset(req_of_row[int(c[0])] for c in cols[col0:col0 + ncols])
            key = (reqs, int(t[1]))
            groups[key] = max(groups.get(key, 0), k1)
    out = {}
    for (reqs, kvh), k1 in groups.items():
        out.setdefault(reqs, set()).add(k1)
    return {reqs: ks.pop() for reqs, ks in out.items() if len(ks) == 1}


@pytest.mark.parametrize("kind,expect", [
    ("outlier", {frozenset(range(1, 8)): 16 * 64}),
    ("nested", {frozenset(range(0, 4)): 16 * 64, frozenset(range(4, 8)): 12 * 64}),
])
def test_shared_prefix_groups_uneven(kind, expect):
    """Groups follow the tree of common page runs: a member sharing one page does not shorten
    the others' run, and nested prefixes get groups of their own when that saves more page
    reads than one wider, shallower group (the choice maximises pages read once for all)."""
    w = _uneven_sharing(kind)
    plan = _plan(w, HOST | api.VA_FLAG_SHARED_PREFIX)
    check_coverage(w, plan)
    st = api.varlen_attn_plan_stats(plan)
    assert st["shared_groups"] == len(expect)
    assert _groups_of(w, plan) == expect
    assert st["physical_kv_bytes"] == oracle.physical_kv_bytes(w.block_table, w.kv_len, w.page_size,
                                                               w.num_kv_heads, w.head_dim, w.elem_bytes)


def test_shared_prefix_groups_leader_outlier():
    """The lowest-numbered request sharing only the first page does not set the group."""
    w = W.build("uneven-lead", [1] * 6, [900] * 6, num_q_heads=8, num_kv_heads=2, head_dim=64,
                page_size=16, seed=9)
    w = W.share_runs(w, [(3, [1, 2, 4, 5], 0, 40), (3, [0], 0, 1)])
    plan = _plan(w, HOST | api.VA_FLAG_SHARED_PREFIX)
    check_coverage(w, plan)
    assert _groups_of(w, plan) == {frozenset([1, 2, 3, 4, 5]): 40 * 16}


def test_config_shapes():
    """The workloads match the configurations they stand for."""
    w = W.config(2)
    assert list(w.q_end - w.q_start) == [4096, 1, 1] and list(w.kv_len) == [4096, 1500, 1700]
    assert w.num_pages == 256 + 94 + 107
    w = W.config(5)
    assert w.num_pages == 64 + 6 * 16 and w.shared_prefix_pages == 64


@pytest.mark.parametrize("name,make,flags", CASES[:6], ids=[c[0] for c in CASES[:6]])
def test_plan_slots_match_oracle(name, make, flags):
    """The plan's out_cache_loc equals the oracle's slot mapping of the new rows."""
    w = make()
    got = api.varlen_attn_plan_slots(_plan(w, flags))
    want = oracle.slots_for_new_rows(w.q_start, w.q_end, w.kv_len, w.block_table, w.page_size, w.total_q_rows)
    assert np.array_equal(got, want)


def test_append_argument_errors():
    L = api.lib()
    assert L.varlen_attn_append_kv(None, 1, None, None, None, None, None, None, None) == api.VA_ERR_INVALID_ARG
    p = api.VaParams(0, 2, 64, 16, 8, 0, api.VA_DTYPE_BF16, 0.0, 0, 0, 0)
    assert L.varlen_attn_append_kv(p, -1, None, None, None, None, None, None, None) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_append_kv(p, 0, None, None, None, None, None, None, None) == api.VA_OK
    assert L.varlen_attn_append_kv(p, 3, None, None, None, None, None, None, None) == api.VA_ERR_INVALID_ARG
    p.head_dim = 96
    assert L.varlen_attn_append_kv(p, 3, None, None, None, None, None, None, None) == api.VA_ERR_UNSUPPORTED


def test_fp8_run_entry_points_check_the_plan_dtype():
    """An fp8 plan is refused by varlen_attn_run / run_events and a bf16 plan by
    varlen_attn_run_fp8, before any device work."""
    L = api.lib()
    wf = W.config(3, scale=64, dtype="fp8")
    pf = _plan(wf)
    assert L.varlen_attn_run(pf.handle, None, None, None, None, None, None, 0, None) == api.VA_ERR_INVALID_ARG
    assert "varlen_attn_run_fp8" in L.varlen_attn_last_error().decode()
    ev = (ctypes.c_void_p * api.VA_RUN_EVENTS)(1, 1, 1, 1)
    assert L.varlen_attn_run_events(pf.handle, None, None, None, None, None, None, 0, None, ev) == \
        api.VA_ERR_INVALID_ARG
    pb = _plan(W.config(3, scale=64))
    assert L.varlen_attn_run_fp8(pb.handle, None, None, None, None, None, None, None, None, 0, None, None) == \
        api.VA_ERR_INVALID_ARG
    assert "VA_DTYPE_FP8_E4M3" in L.varlen_attn_last_error().decode()
    # host-only fp8 plan: refused for lack of a device buffer
    assert L.varlen_attn_run_fp8(pf.handle, None, None, None, None, None, None, None, None, 0, None, None) == \
        api.VA_ERR_INVALID_ARG


def test_fp8_debug_convert_argument_errors():
    L = api.lib()
    assert L.varlen_attn_debug_fp8_to_bf16(None, None, 12, None) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_debug_fp8_to_bf16(None, None, -8, None) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_debug_fp8_to_bf16(None, None, 0, None) == api.VA_OK
    assert L.varlen_attn_debug_fp8_to_bf16(None, None, 8, None) == api.VA_ERR_INVALID_ARG


def test_stream_read_argument_errors():
    """The read-rate probe checks its arguments on the host (no launch happens here)."""
    L = api.lib()
    assert L.varlen_attn_debug_stream_read(None, 0, None, None) == api.VA_OK          # nothing to read
    assert L.varlen_attn_debug_stream_read(None, 64, None, None) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_debug_stream_read(16, 64, None, None) == api.VA_ERR_INVALID_ARG  # sink NULL
    assert L.varlen_attn_debug_stream_read(16, 60, 32, None) == api.VA_ERR_INVALID_ARG    # not whole words
    assert L.varlen_attn_debug_stream_read(8, 64, 32, None) == api.VA_ERR_INVALID_ARG     # misaligned
    assert b"16-byte" in L.varlen_attn_last_error()


def test_fp8_append_argument_errors():
    """fp8 pools take varlen_attn_append_kv_fp8 (codes and scales), and it takes only them."""
    L = api.lib()
    p = api.VaParams(0, 2, 64, 16, 8, 0, api.VA_DTYPE_FP8_E4M3, 0.0, 0, 0, 0)
    assert L.varlen_attn_append_kv(p, 3, None, None, None, None, None, None, None) == api.VA_ERR_INVALID_ARG
    assert "varlen_attn_append_kv_fp8" in L.varlen_attn_last_error().decode()
    n = (None,) * 9
    assert L.varlen_attn_append_kv_fp8(None, 1, *n) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_append_kv_fp8(p, -1, *n) == api.VA_ERR_INVALID_ARG
    assert L.varlen_attn_append_kv_fp8(p, 0, *n) == api.VA_OK
    assert L.varlen_attn_append_kv_fp8(p, 3, *n) == api.VA_ERR_INVALID_ARG
    pb = api.VaParams(0, 2, 64, 16, 8, 0, api.VA_DTYPE_BF16, 0.0, 0, 0, 0)
    assert L.varlen_attn_append_kv_fp8(pb, 3, *n) == api.VA_ERR_INVALID_ARG
    p.head_dim = 96
    assert L.varlen_attn_append_kv_fp8(p, 3, *n) == api.VA_ERR_UNSUPPORTED


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; asked for more it exits with status 2 and says why."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# ---- the binding checks every buffer's shape against the plan before a kernel sees it --

def _cpu_buffers(w, plan):
    import torch
    p = plan.params
    bf = torch.bfloat16
    return dict(q=torch.zeros(w.total_q_rows, p.num_q_heads, p.head_dim, dtype=bf),
                k_pool=torch.zeros(p.num_pages, p.num_kv_heads, p.page_size, p.head_dim, dtype=bf),
                v_pool=torch.zeros(p.num_pages, p.num_kv_heads, p.head_dim, p.page_size, dtype=bf),
                block_table_dev=torch.zeros(w.num_reqs, p.max_pages_per_req, dtype=torch.int32),
                out=torch.zeros(w.total_q_rows, p.num_q_heads, p.head_dim, dtype=bf))


@pytest.mark.parametrize("name,shape_fn", [
    ("q", lambda b: (b["q"].shape[0] - 1,) + tuple(b["q"].shape[1:])),
    ("out", lambda b: (b["out"].shape[0], b["out"].shape[1] - 1, b["out"].shape[2])),
    ("k_pool", lambda b: (b["k_pool"].shape[0] - 1,) + tuple(b["k_pool"].shape[1:])),
    ("v_pool", lambda b: tuple(b["k_pool"].shape)),              # a K-shaped V pool (pages not transposed)
    ("block_table_dev", lambda b: (b["block_table_dev"].shape[0] - 1, b["block_table_dev"].shape[1])),
])
def test_binding_rejects_buffers_smaller_than_the_plan(name, shape_fn):
    """A buffer that does not have the plan's shape is refused on the host (no kernel would
    read past it)."""
    import torch
    w = W.build("sh", [5, 1], [40, 70], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=32, seed=1,
                extra_pages=1)
    plan = api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    b = _cpu_buffers(w, plan)
    b[name] = torch.zeros(shape_fn(b), dtype=b[name].dtype)
    with pytest.raises(ValueError, match=name):
        api.varlen_attn_run(plan, b["q"], b["k_pool"], b["v_pool"], b["block_table_dev"], b["out"])
    with pytest.raises(ValueError, match=name):
        api.RunCall(plan, b["q"], b["k_pool"], b["v_pool"], b["block_table_dev"], b["out"])


def test_binding_shape_checks_pass_for_the_plans_shapes():
    """With every shape right, the first complaint is that the tensors are not on a GPU."""
    w = W.build("sh", [5, 1], [40, 70], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=32, seed=1)
    plan = api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    b = _cpu_buffers(w, plan)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.varlen_attn_run(plan, b["q"], b["k_pool"], b["v_pool"], b["block_table_dev"], b["out"])


def test_binding_rejects_wrong_scale_and_append_pool_shapes():
    import torch
    w = W.build("sh8", [5, 1], [40, 70], num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=32, seed=1,
                dtype="fp8")
    plan = api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    p = plan.params
    b = _cpu_buffers(w, plan)
    k8 = torch.zeros(tuple(b["k_pool"].shape), dtype=torch.uint8)
    v8 = torch.zeros(tuple(b["v_pool"].shape), dtype=torch.uint8)
    ks = torch.zeros(p.num_pages, p.num_kv_heads, p.page_size)
    short = torch.zeros(p.num_pages - 1, p.num_kv_heads, p.page_size)
    with pytest.raises(ValueError, match="v_scale"):
        api.varlen_attn_run_fp8(plan, b["q"], k8, v8, ks, short, b["block_table_dev"], b["out"])
    T = 3
    new = torch.zeros(T, p.num_kv_heads, p.head_dim, dtype=torch.bfloat16)
    loc = torch.zeros(T, dtype=torch.int64)
    with pytest.raises(ValueError, match="v_pool"):
        api.varlen_attn_append_kv(num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, page_size=p.page_size,
                                  num_pages=p.num_pages, k_new=new, v_new=new, out_cache_loc=loc,
                                  k_pool=b["k_pool"], v_pool=b["k_pool"])
    with pytest.raises(ValueError, match="k_scale"):
        api.varlen_attn_append_kv_fp8(num_kv_heads=p.num_kv_heads, head_dim=p.head_dim, page_size=p.page_size,
                                      num_pages=p.num_pages, k_new=new, v_new=new, out_cache_loc=loc, k_pool=k8,
                                      v_pool=v8, k_scale=short, v_scale=ks)


def test_launch_order_pairs_heavy_with_light_tiles_on_each_cu():
    # ORCA's 4096-row prefill: 1024 tiles of 2..64 steps of 64 keys plus 64 decode tiles, 136
    # per XCD.  XCD positions c and c + 32 start together on one CU, so each XCD's first 64
    # positions pair its heaviest tile with the lightest of those 64: every CU's first two
    # tiles sum to the same work, and the remaining tiles follow heaviest first.
    w = W.config(2)
    tiles = api.varlen_attn_plan_export(_plan(w), 3)
    work = tiles[:, 6] - tiles[:, 7]
    for x in range(8):
        wx = work[x::8]
        assert len(wx) == 136
        pair_sums = wx[:32] + wx[32:64]
        assert pair_sums.max() - pair_sums.min() <= 128          # one 64-key step each way
        assert np.all(np.diff(wx[:32]) <= 0) and np.all(np.diff(wx[32:64]) >= 0)
        assert np.all(np.diff(wx[64:]) <= 0) and wx[64:].max() <= wx[:64].min()

