"""GPU parity of the fp8 KV path (e4m3fn codes with per-position float32 scales) through
the C ABI, against the oracle on the dequantised pools.

Tolerance: max |gpu - oracle| <= 1e-2: the codes widen to bf16 exactly, the scales are
applied in fp32, and the row sum adds the same rounded weights that the P.V product
applies, so the remaining roundings are those of the bf16 path (P rounded to bf16 for the
P.V product, bf16 output).  The code widening is
compared bit for bit on all 256 codes, and the page gather of the codes bit for bit."""
import sys

import numpy as np
import pytest

import oracle
from varlen_paged_attention_amd import api, workloads as W

pytestmark = pytest.mark.gpu

TOL = 1e-2


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
    K, V = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
    return oracle.varlen_paged_attention(w.q, K, V, w.block_table, w.q_start, w.q_end, w.kv_len, w.page_size,
                                         w.softmax_scale or None)


def _oracle_rows(w, r, rows):
    """Oracle rows of request r from its own pages only (dequantising the whole pool of a
    full-size workload would not fit in memory)."""
    npg = -(-int(w.kv_len[r]) // w.page_size)
    pages = np.asarray(w.block_table[r][:npg], np.int64)
    K, V = oracle.dequantize_pools(w.k_pool[pages], w.k_scale[pages], w.v_pool[pages], w.v_scale[pages])
    bt = np.arange(npg, dtype=np.int32)[None, :]
    qs = np.array([w.q_start[r]], np.int32)
    return oracle.attention_rows(w.q, K, V, bt, qs, np.array([w.q_end[r]], np.int32),
                                 np.array([w.kv_len[r]], np.int32), w.page_size, 0, rows)


def _run(w, flags=0, out_fill=None, **kw):
    import torch
    plan = api.plan_for(w, flags=flags, **kw)
    q, k, v, bt = api.to_device(w)
    ks, vs = api.scales_to_device(w)
    out = torch.zeros_like(q) if out_fill is None else torch.full_like(q, out_fill)
    ws = api.new_workspace(plan)
    api.varlen_attn_run_fp8(plan, q, k, v, ks, vs, bt, out, ws)
    torch.cuda.synchronize()
    return out, plan


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
    _say(f"[parity] {label}: max|gpu-oracle| = {e:.3e} (tol {TOL})")
    assert np.isfinite(got[rows]).all(), f"{label}: non-finite output"
    assert e <= TOL, f"{label}: max error {e}"


def test_fp8_widening_all_codes_bit_exact():
    """Every code at every byte position of an 8-code group widens to the bf16 value the
    format defines (NaN codes to a NaN)."""
    import torch
    codes = np.concatenate([np.roll(np.arange(256, dtype=np.uint8), s) for s in range(8)])
    _say("[gpu] fp8 widening of all codes")
    dev = torch.from_numpy(codes).cuda()
    out = torch.empty(codes.size, dtype=torch.int16, device="cuda")
    api.varlen_attn_debug_fp8_to_bf16(dev, out)
    torch.cuda.synchronize()
    got_bits = out.cpu().numpy().view(np.uint16)
    got = oracle.bf16_bits_to_f64(got_bits)
    want = oracle.e4m3fn_to_f64(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))     # -0 stays -0


SMALL = [
    ("tiny-d64", 1, 1, 0),
    ("orca-mixed/4", 2, 4, 0),
    ("decode-heavy/8", 3, 8, 0),
    ("chunk-mix/8", 4, 8, 0),
    ("shared-6", 5, 1, api.VA_FLAG_SHARED_PREFIX),
    ("shared-6 plain", 5, 1, 0),
    ("spec-decode-mtp7/8", 7, 8, 0),
    ("shared-6 split items", 5, 1, api.VA_FLAG_SHARED_PREFIX | api.VA_FLAG_NO_PREFILL_KERNEL),
    # the decodes of a plan with prefill tiles ride in that launch as tiles when their KV is
    # small (the cases above); with decode tiles off they run as split-KV items beside them
    ("orca-mixed/4 decodes on items", 2, 4, api.VA_FLAG_NO_DECODE_TILES),
    ("chunk-mix/8 decodes on items", 4, 8, api.VA_FLAG_NO_DECODE_TILES),
]


@pytest.mark.parametrize("label,cid,scale,flags", SMALL, ids=[s[0] for s in SMALL])
def test_fp8_parity_small_elementwise(label, cid, scale, flags):
    w = W.config(cid, scale=scale, poison_tail=True, dtype="fp8")
    _say(f"[gpu] fp8 run {label} rows={w.total_q_rows} kv={list(w.kv_len[:4])}...")
    out, plan = _run(w, flags)
    _check_full(w, out, "fp8 " + label)


def test_fp8_parity_split_len_64():
    """Many parts per output (every 64-key step its own item) through the combine pass."""
    w = W.config(4, scale=16, poison_tail=True, dtype="fp8")
    _say("[gpu] fp8 split_len=64")
    out, plan = _run(w, api.VA_FLAG_NO_DECODE_TILES, split_len=64)
    st = api.varlen_attn_plan_stats(plan)
    assert st["combine_rows"] > 0 and st["split_items"] > 0
    _check_full(w, out, "fp8 chunk-mix/16 split 64")


FULL = [("decode-heavy", 3, 0), ("orca-mixed", 2, 0), ("shared-64", 51, api.VA_FLAG_SHARED_PREFIX)]


@pytest.mark.parametrize("label,cid,flags", FULL, ids=[f[0] for f in FULL])
def test_fp8_parity_full_size_sampled(label, cid, flags):
    w = W.config(cid, dtype="fp8")
    _say(f"[gpu] fp8 run full {label}: reqs={w.num_reqs} rows={w.total_q_rows} pages={w.num_pages}")
    out, plan = _run(w, flags)
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(200 + cid)
    R = w.num_reqs
    reqs = sorted({0, R - 1, int(np.argmax(w.kv_len))} | set(int(x) for x in rng.choice(R, min(R, 6), False)))
    worst = 0.0
    for r in reqs:
        m = int(w.q_end[r] - w.q_start[r])
        rows = sorted({0, m - 1} | set(int(x) for x in rng.choice(m, min(m, 8), False)))
        for h, o in _oracle_rows(w, r, rows).items():
            g = got[int(w.q_start[r]) + np.asarray(rows), h, :]
            assert np.isfinite(g).all()
            worst = max(worst, float(np.abs(g - o).max()))
    _say(f"[parity] fp8 full {label}: sampled max|gpu-oracle| = {worst:.3e}")
    assert worst <= TOL


FOCUSED = [("decode-heavy", 3, 0), ("chunk-mix", 4, 0), ("shared-64", 51, api.VA_FLAG_SHARED_PREFIX)]


@pytest.mark.parametrize("label,cid,flags", FOCUSED, ids=[f[0] for f in FOCUSED])
def test_fp8_parity_full_size_focused(label, cid, flags):
    """fp8 pools of the full-size workloads on the focused companion inputs (outputs O(1)):
    sampled rows against the oracle on the dequantised pools, with negative controls."""
    import sampled
    w = W.focus(W.config(cid, dtype="fp8"))
    _say(f"[gpu] fp8 run full focused {label}: reqs={w.num_reqs} rows={w.total_q_rows}")
    out, plan = _run(w, flags)
    got = out.float().cpu().numpy()
    rng = np.random.default_rng(400 + cid)
    R, Hq = w.num_reqs, w.num_q_heads
    reqs = sorted({0, R - 1, int(np.argmax(w.kv_len))} | set(int(x) for x in rng.choice(R, min(R, 4), False)))
    worst, margin = 0.0, np.inf
    for r in reqs:
        m = int(w.q_end[r] - w.q_start[r])
        rows = sorted({0, m - 1} | set(int(x) for x in rng.choice(m, min(m, 6), False)))
        heads = sorted({0, Hq - 1} | set(int(x) for x in rng.choice(Hq, min(Hq, 6), False)))
        got_rows = {h: got[int(w.q_start[r]) + np.asarray(rows), h, :] for h in heads}
        e, mg = sampled.check_request(w, r, rows, heads, got_rows, TOL)
        worst, margin = max(worst, e), min(margin, mg)
    _say(f"[parity] fp8 focused full {label}: sampled max|gpu-oracle| = {worst:.3e}; "
         f"smallest negative-control error {margin:.3e}")
    assert worst <= TOL and margin > TOL


EDGE = [
    ("gap+zero-row+kv1", dict(q_rows=[3, 0, 1, 1, 5], kv=[3, 9, 1, 2, 40], hq=4, hkv=4, d=64, ps=16)),
    ("g16-multi-row-ps256", dict(q_rows=[3, 1], kv=[700, 257], hq=32, hkv=2, d=128, ps=256)),
    ("mtp-g8-ps32", dict(q_rows=[5, 4, 1], kv=[300, 64, 31], hq=16, hkv=2, d=128, ps=32)),
    ("long-decode", dict(q_rows=[1, 1], kv=[40000, 77], hq=8, hkv=1, d=128, ps=64)),
    ("prefill-rows-d64", dict(q_rows=[130, 2], kv=[200, 2], hq=6, hkv=3, d=64, ps=16)),
]


@pytest.mark.parametrize("label,spec", EDGE, ids=[e[0] for e in EDGE])
def test_fp8_edge_cases(label, spec):
    w = W.build(label, spec["q_rows"], spec["kv"], num_q_heads=spec["hq"], num_kv_heads=spec["hkv"],
                head_dim=spec["d"], page_size=spec["ps"], dtype="fp8", seed=19, poison_tail=True, extra_pages=2)
    w.q_start = w.q_start.copy()
    w.q_end = w.q_end.copy()
    w.q_start[1:] += 2
    w.q_end[1:] += 2
    w.q = np.concatenate([w.q[:w.q_end[0]], np.zeros((2,) + w.q.shape[1:], w.q.dtype), w.q[w.q_end[0]:]])
    _say(f"[gpu] fp8 edge {label}")
    out, plan = _run(w, out_fill=7.0)
    _check_full(w, out, "fp8 " + label)
    gap = out[w.q_end[0]:w.q_start[1]].float().cpu().numpy()
    assert (gap == 7.0).all(), "rows outside every request were written"


@pytest.mark.parametrize("d,ps", [(128, 16), (64, 64)])
def test_fp8_unusual_scales(d, ps):
    """Scales outside what the append writes: V scales below the normal float range (1e-40),
    zero and negative, and negative K scales, on prefill tiles and split-KV decode items.
    The dequantised values are code * scale whatever the scale; the kernels count a V
    scale below the normal range as a zero V row (|V| < 5e-36), which the tolerance covers."""
    w = W.build(f"fp8-scales-d{d}-ps{ps}", [130, 1, 1, 3], [300, 900, 77, 64], num_q_heads=8, num_kv_heads=2,
                head_dim=d, page_size=ps, dtype="fp8", seed=23, poison_tail=True)
    rng = np.random.default_rng(5)
    vs, ks = w.v_scale.copy(), w.k_scale.copy()
    u = rng.random(vs.shape)
    vs[u < 0.1] = np.float32(1e-40)
    vs[(u >= 0.1) & (u < 0.15)] = 0.0
    vs[(u >= 0.15) & (u < 0.25)] *= -1
    ks[rng.random(ks.shape) < 0.1] *= -1
    w.v_scale, w.k_scale = vs.astype(np.float32), ks.astype(np.float32)
    # the decodes ride in the prefill launch as tiles (their KV is small), and, with decode
    # tiles off, run as split-KV items: both paths see the unusual scales
    for flags, on_items in ((0, False), (api.VA_FLAG_NO_DECODE_TILES, True)):
        _say(f"[gpu] fp8 unusual scales d{d} ps{ps} decodes on {'items' if on_items else 'tiles'}")
        out, plan = _run(w, flags)
        st = api.varlen_attn_plan_stats(plan)
        assert st["prefill_tiles"] > 0 and (st["split_items"] > 0) == on_items, st
        _check_full(w, out, f"fp8 unusual scales d{d} ps{ps} decodes on {'items' if on_items else 'tiles'}")


def test_fp8_deterministic_and_gather():
    import torch
    w = W.config(3, scale=8, dtype="fp8")
    _say("[gpu] fp8 determinism + gather")
    a, plan = _run(w)
    b, _ = _run(w)
    assert np.array_equal(a.view(torch.int16).cpu().numpy(), b.view(torch.int16).cpu().numpy())
    q, k, v, bt = api.to_device(w)
    tot = int(w.kv_len.sum())
    ko = torch.empty((tot, w.num_kv_heads, w.head_dim), dtype=torch.uint8, device="cuda")
    vo = torch.empty_like(ko)
    api.varlen_attn_debug_gather(plan, k, v, bt, ko, vo)
    torch.cuda.synchronize()
    ks, vs = [], []
    for r in range(w.num_reqs):
        j = np.arange(int(w.kv_len[r]))
        pages, slots = w.block_table[r][j // w.page_size], j % w.page_size
        ks.append(w.k_pool[pages, :, slots, :])
        vs.append(w.v_pool[pages, :, :, slots])
    assert np.array_equal(ko.cpu().numpy(), np.concatenate(ks))
    assert np.array_equal(vo.cpu().numpy(), np.concatenate(vs))


def test_fp8_run_errors():
    import torch
    w = W.config(3, scale=64, dtype="fp8")
    plan = api.plan_for(w)
    q, k, v, bt = api.to_device(w)
    ks, vs = api.scales_to_device(w)
    out = torch.zeros_like(q)
    ws = api.new_workspace(plan)
    L = api.lib()
    P = lambda t: None if t is None else t.data_ptr()          # noqa: E731
    base = [plan.handle, P(q), P(k), P(v), P(ks), P(vs), P(bt), P(out), P(ws), ws.numel(), None, None]
    no_scale = list(base)
    no_scale[4] = None
    assert L.varlen_attn_run_fp8(*no_scale) == api.VA_ERR_INVALID_ARG
    misaligned = list(base)
    misaligned[5] = P(vs) + 4
    assert L.varlen_attn_run_fp8(*misaligned) == api.VA_ERR_INVALID_ARG
    assert "aligned" in L.varlen_attn_last_error().decode()
    assert L.varlen_attn_run_fp8(*base) == api.VA_OK
    torch.cuda.synchronize()


# ------------------------------------------------------------------ fp8 append --

def _bf16_rows(rng, shape, special=True):
    """bf16 bit patterns of test rows: N(0,1) draws, plus (``special``) rows that reach the
    subnormal codes (magnitudes spread over 2^-20 .. 4) and rows whose maximum is 448 so
    that the scale is 1 and every other element sits exactly halfway between two codes."""
    x = rng.standard_normal(shape).astype(np.float32)
    T, H, D = shape
    if not special:
        bits = np.empty(shape, np.uint16)
        W.f32_to_bf16_bits(x, bits)
        return bits
    x[0, 0] = np.ldexp(1.0, rng.integers(-20, 3, D)) * rng.choice([-1, 1], D)
    mids = (oracle.e4m3fn_to_f64(np.arange(0, 0x7E, dtype=np.uint8)) +
            oracle.e4m3fn_to_f64(np.arange(1, 0x7F, dtype=np.uint8))) / 2
    row = rng.choice(mids, D) * rng.choice([-1, 1], D)
    row[0] = 448.0
    x[1 % T, H - 1] = row
    x[min(2, T - 1), 0] = 0.0                        # all-zero vector: scale 1, zero codes
    bits = np.empty(shape, np.uint16)
    W.f32_to_bf16_bits(x, bits)
    assert np.array_equal((bits[1 % T, H - 1].astype(np.uint32) << 16).view(np.float32), row.astype(np.float32))
    return bits


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


APPEND_LAYOUTS = {
    # new rows starting mid-page: every V column written byte by byte
    "mid-page": ([37, 1, 5, 0, 200], [90, 300, 5, 10, 200]),
    # an uncached prefill first: its tokens fill whole pages from slot 0 (16-byte V stores)
    "page-aligned": ([200, 37, 1, 5, 0], [200, 90, 300, 5, 10]),
}


@pytest.mark.parametrize("layout", list(APPEND_LAYOUTS))
@pytest.mark.parametrize("d,ps", [(128, 16), (64, 64), (128, 256)])
def test_fp8_append_bit_exact(d, ps, layout):
    """GPU quantise-and-append == the oracle's, bit for bit (codes and scales), with
    padding, an out-of-range entry (skipped and counted) and untouched slots kept."""
    import torch
    q_rows, kv = APPEND_LAYOUTS[layout]
    w = W.build("ap8", q_rows, kv, num_q_heads=8, num_kv_heads=4, head_dim=d,
                page_size=ps, dtype="fp8", seed=29, extra_pages=3)
    _say(f"[gpu] fp8 append d={d} ps={ps} {layout}")
    plan = api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    loc = api.varlen_attn_plan_slots(plan)
    loc[3] = -1
    loc[7] = w.num_pages * ps + 5                       # out of range: skipped, counted
    rng = np.random.default_rng(7)
    shape = (w.total_q_rows, w.num_kv_heads, d)
    k_new, v_new = _bf16_rows(rng, shape), _bf16_rows(rng, shape)
    ok = np.where(loc < w.num_pages * ps, loc, -1)
    want = oracle.append_kv_fp8(w.k_pool, w.v_pool, w.k_scale, w.v_scale, _f32(k_new), _f32(v_new), ok, ps)
    kp, vp = torch.from_numpy(w.k_pool.copy()).cuda(), torch.from_numpy(w.v_pool.copy()).cuda()
    ks, vs = api.scales_to_device(w)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.varlen_attn_append_kv_fp8(num_kv_heads=w.num_kv_heads, head_dim=d, page_size=ps, num_pages=w.num_pages,
                                  k_new=torch.from_numpy(k_new).view(torch.bfloat16).cuda(),
                                  v_new=torch.from_numpy(v_new).view(torch.bfloat16).cuda(),
                                  out_cache_loc=torch.from_numpy(loc).cuda(), k_pool=kp, v_pool=vp, k_scale=ks,
                                  v_scale=vs, bad_loc_count=bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1
    for got, exp, name in zip((kp, vp, ks, vs), want, ("k codes", "v codes", "k scales", "v scales")):
        g = got.cpu().numpy()
        assert np.array_equal(g.view(np.uint8), np.ascontiguousarray(exp).view(np.uint8)), name


def _bf16_exact(a):
    """float32 values rounded to bf16 (nearest even), as float32."""
    bits = np.empty(a.shape, np.uint16)
    W.f32_to_bf16_bits(np.ascontiguousarray(a, np.float32), bits)
    return _f32(bits)


def test_fp8_append_every_bf16_magnitude_bit_exact():
    """Every finite bf16 magnitude (random signs) quantised in rows whose maximum is one of
    sixteen values from a bf16 subnormal to 3e38: the appended codes and scales equal the
    oracle's bit for bit (the kernel's quotient through the reciprocal, with its exact
    fallback near e4m3fn rounding midpoints, against the float32 division)."""
    import torch
    rng = np.random.default_rng(41)
    vals = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    amaxes = _bf16_exact(np.array([448.0, 1.0, 3.0, 0.1, 100.0, 1e-3, 7.875, 6e4, 3e38, 1e-30, 2e-38, 1e-39,
                                   0.3333, 12345.0, 5e-5, 1.5e10], np.float32))
    rows = []
    for a in amaxes:
        xs = vals[vals <= a] * rng.choice(np.float32([-1, 1]), int((vals <= a).sum()))
        rng.shuffle(xs)
        n = -(-len(xs) // 127)
        xs = np.concatenate([xs, np.zeros(n * 127 - len(xs), np.float32)]).reshape(n, 127)
        rows.append(np.concatenate([np.full((n, 1), a, np.float32), xs], 1))
    K = np.concatenate(rows)
    V = K[rng.permutation(len(K))][:, rng.permutation(128)]
    T, ps, D = len(K), 16, 128
    P = -(-T // ps)
    _say(f"[gpu] fp8 append of every bf16 magnitude: {T} rows x {D}")
    want = oracle.append_kv_fp8(np.zeros((P, 1, ps, D), np.uint8), np.zeros((P, 1, D, ps), np.uint8),
                                np.zeros((P, 1, ps), np.float32), np.zeros((P, 1, ps), np.float32),
                                K[:, None, :], V[:, None, :], np.arange(T), ps)
    kb, vb = np.empty(K.shape, np.uint16), np.empty(V.shape, np.uint16)
    W.f32_to_bf16_bits(K, kb)
    W.f32_to_bf16_bits(V, vb)
    kp = torch.zeros((P, 1, ps, D), dtype=torch.uint8, device="cuda")
    vp = torch.zeros((P, 1, D, ps), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((P, 1, ps), dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    api.varlen_attn_append_kv_fp8(num_kv_heads=1, head_dim=D, page_size=ps, num_pages=P,
                                  k_new=torch.from_numpy(kb[:, None, :].copy()).view(torch.bfloat16).cuda(),
                                  v_new=torch.from_numpy(vb[:, None, :].copy()).view(torch.bfloat16).cuda(),
                                  out_cache_loc=torch.arange(T, dtype=torch.int64, device="cuda"), k_pool=kp,
                                  v_pool=vp, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    for got, exp, name in zip((kp, vp, ks, vs), want, ("k codes", "v codes", "k scales", "v scales")):
        g = got.cpu().numpy()
        assert np.array_equal(g.view(np.uint8), np.ascontiguousarray(exp).view(np.uint8)), name


@pytest.mark.parametrize("cid,scale", [(3, 16), (4, 16)])
def test_fp8_append_then_attend(cid, scale):
    """Quantise and append the iteration's new rows on the GPU into pools whose new-row
    slots hold NaN codes, then attend: the output matches the oracle on the pools the
    oracle's own append produces."""
    import torch
    w = W.config(cid, scale=scale, dtype="fp8")
    _say(f"[gpu] fp8 append then attend config {cid}/{scale}")
    plan = api.plan_for(w)
    loc = api.varlen_attn_plan_slots(plan)
    rng = np.random.default_rng(31)
    shape = (w.total_q_rows, w.num_kv_heads, w.head_dim)
    # N(0,1) rows: outputs of order 1, where the bf16 tolerance applies
    k_new, v_new = _bf16_rows(rng, shape, special=False), _bf16_rows(rng, shape, special=False)
    kb, vb = w.k_pool.copy(), w.v_pool.copy()
    ksb, vsb = w.k_scale.copy(), w.v_scale.copy()
    for l in loc[loc >= 0]:
        kb[l // w.page_size, :, l % w.page_size, :] = W.FP8_NAN
        vb[l // w.page_size, :, :, l % w.page_size] = W.FP8_NAN
        ksb[l // w.page_size, :, l % w.page_size] = np.nan
        vsb[l // w.page_size, :, l % w.page_size] = np.nan
    w.k_pool, w.v_pool, w.k_scale, w.v_scale = oracle.append_kv_fp8(kb, vb, ksb, vsb, _f32(k_new), _f32(v_new), loc,
                                                                     w.page_size)
    q, _, _, bt = api.to_device(w)
    kp, vp = torch.from_numpy(kb).cuda(), torch.from_numpy(vb).cuda()
    ks, vs = torch.from_numpy(ksb).cuda(), torch.from_numpy(vsb).cuda()
    api.varlen_attn_append_kv_fp8(num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size,
                                  num_pages=w.num_pages, k_new=torch.from_numpy(k_new).view(torch.bfloat16).cuda(),
                                  v_new=torch.from_numpy(v_new).view(torch.bfloat16).cuda(),
                                  out_cache_loc=torch.from_numpy(loc).cuda(), k_pool=kp, v_pool=vp, k_scale=ks, v_scale=vs)
    out = torch.zeros_like(q)
    api.varlen_attn_run_fp8(plan, q, kp, vp, ks, vs, bt, out, api.new_workspace(plan))
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(), w.k_pool) and np.array_equal(vs.cpu().numpy().view(np.uint32),
                                                                          w.v_scale.view(np.uint32))
    _check_full(w, out, f"fp8 append+attend {cid}/{scale}")
