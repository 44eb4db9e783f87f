"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test cites the passage (page title, section) it checks.  None of them runs the
HIP library.  ``test_mutants_are_caught`` plants plausible mistakes in the oracle and
checks that at least one pin fails for each.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as OA
from varlen_paged_attention_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(w, **kw):
    return oracle.varlen_paged_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start,
                                         w.q_end, w.kv_len, w.page_size, w.softmax_scale or None, **kw)


def _f32(q_rows, kv, hq=2, hkv=1, d=8, ps=4, seed=0, **kw):
    return W.build("t", q_rows, kv, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                   dtype="f32", seed=seed, **kw)


def _request_kv(w, r, kvh):
    return OA.gather_kv(w.k_pool, w.v_pool, w.block_table[r], int(w.kv_len[r]), kvh, w.page_size)


# ---------------------------------------------------------------- mask ----------

def _load_mask_fixture():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "abc_xefg_mask.txt"))
            if l.strip() and not l.startswith("#")]
    return np.array([[c == "1" for c in r] for r in rows])


def check_mask_worked_example():
    """abc cached + xefg new -> [4, 7] pattern ("How To Scale Your Model 笔记(7-8)", §2)."""
    want = _load_mask_fixture()
    got = oracle.visibility_mask(3, 4)
    assert got.shape == (4, 7)
    assert np.array_equal(got, want)
    assert int(got.sum()) == 22


def test_mask_worked_example():
    check_mask_worked_example()


def test_decode_is_m1_special_case():
    """Decode is the m = 1 case: one row that sees every position (same page, §2;
    "ORCA 和 chunked prefill", §4: decode is chunked prefill with C = 1)."""
    for S0 in (0, 1, 7, 100):
        m = oracle.visibility_mask(S0, 1)
        assert m.shape == (1, S0 + 1) and m.all()


def test_uncached_prefill_is_causal_s0_0():
    """S0 = 0 is the ordinary causal mask; equals torch SDPA(is_causal=True) in fp64."""
    for n in (1, 5, 17):
        m = oracle.visibility_mask(0, n)
        assert np.array_equal(m, np.tril(np.ones((n, n), bool)))
    w = _f32([13], [13], hq=2, hkv=2, d=8, ps=4, seed=3)
    out = _run(w)
    q = torch.from_numpy(w.q.astype(np.float64)).permute(1, 0, 2)          # [H, n, D]
    K = np.stack([_request_kv(w, 0, h)[0] for h in range(2)])
    V = np.stack([_request_kv(w, 0, h)[1] for h in range(2)])
    ref = torch.nn.functional.scaled_dot_product_attention(q, torch.from_numpy(K), torch.from_numpy(V),
                                                           is_causal=True)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref.numpy(), rtol=0, atol=1e-12)


def test_chunk_with_prefix_matches_sdpa_explicit_mask():
    """S0 > 0: SDPA with an explicit boolean mask j <= S0 + i, built here independently."""
    S0, m = 9, 6
    w = _f32([m], [S0 + m], hq=4, hkv=2, d=16, ps=4, seed=5)
    out = _run(w)
    allowed = torch.ones(m, S0 + m, dtype=torch.bool).tril(diagonal=S0)
    for h in range(4):
        K, V = _request_kv(w, 0, h // 2)
        q = torch.from_numpy(w.q[:, h, :].astype(np.float64))
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], torch.from_numpy(K)[None],
                                                               torch.from_numpy(V)[None], attn_mask=allowed)
        np.testing.assert_allclose(out[:, h, :], ref[0].numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------- chunked prefill --------

def test_chunked_mask_is_slice_of_unchunked():
    """Chunk k of size C on prefix S = kC has the mask of rows [kC, (k+1)C) of the
    unchunked N-row prefill, restricted to columns [0, (k+1)C); the columns after that
    are all masked ("ORCA 和 chunked prefill", §4)."""
    N, C = 40, 8
    full = oracle.visibility_mask(0, N)
    for k in range(N // C):
        chunk = oracle.visibility_mask(k * C, C)
        rows = full[k * C:(k + 1) * C]
        assert np.array_equal(chunk, rows[:, :(k + 1) * C])
        assert not rows[:, (k + 1) * C:].any()


def test_chunked_outputs_equal_unchunked():
    """Running the chunks as separate requests gives the unchunked rows (fp64 1e-13);
    chunking moves work between iterations and changes no result (§4, §6)."""
    N, C = 24, 8
    whole = _f32([N], [N], hq=2, hkv=1, d=8, ps=4, seed=9)
    ref = _run(whole)
    for k in range(N // C):
        w = W.Workload(**{**whole.__dict__})
        w.q = whole.q[k * C:(k + 1) * C]
        w.q_start = np.array([0], np.int32)
        w.q_end = np.array([C], np.int32)
        w.kv_len = np.array([(k + 1) * C], np.int32)
        out = _run(w)
        np.testing.assert_allclose(out, ref[k * C:(k + 1) * C], rtol=0, atol=1e-13)


def test_chunk_pair_sum():
    """Σ_k visible pairs over the chunks = N(N+1)/2 = the unchunked count; the page's
    "Σ C·(k+1)C ≈ N²/2" counts whole rectangles ("ORCA 和 chunked prefill", §6)."""
    for N, C in ((100, 10), (2048 * 4, 2048), (37, 5)):
        total = sum(oracle.visible_pairs([min(C, N - s)], [min(s + C, N)]) for s in range(0, N, C))
        assert total == N * (N + 1) // 2
        if N < 200:
            assert total == int(oracle.visibility_mask(0, N).sum())
    rng = np.random.default_rng(0)
    for _ in range(50):
        m, S0 = int(rng.integers(1, 30)), int(rng.integers(0, 30))
        assert oracle.visible_pairs([m], [S0 + m]) == int(oracle.visibility_mask(S0, m).sum())


# ------------------------------------------------------------ closed forms ------

def test_zero_query_gives_prefix_means():
    """q = 0: all visible scores are equal, so row i is the mean of V[0..S0+i]."""
    S0, m = 5, 4
    w = _f32([m], [S0 + m], hq=2, hkv=1, d=8, ps=4, seed=11)
    w.q[:] = 0
    out = _run(w)
    _, V = _request_kv(w, 0, 0)
    for i in range(m):
        np.testing.assert_allclose(out[i, 0], V[:S0 + i + 1].mean(axis=0), rtol=0, atol=1e-14)


def test_single_position_and_first_row():
    """kv_len = 1 gives V[0]; row 0 of an uncached prefill sees only position 0 -> V[0]
    exactly (the softmax of one element is 1)."""
    w = _f32([1, 6], [1, 6], hq=2, hkv=2, d=8, ps=4, seed=13)
    out = _run(w)
    for r, t in ((0, 0), (1, int(w.q_start[1]))):
        for h in range(2):
            _, V = _request_kv(w, r, h)
            assert np.array_equal(out[t, h], V[0])


def test_weights_sum_to_one():
    w = _f32([7], [20], hq=2, hkv=1, d=8, ps=4, seed=15)
    K, V = _request_kv(w, 0, 0)
    # V = identity rows turns the output into the weights themselves
    eye = np.eye(20)
    out = OA.attend(w.q[:, 0, :].astype(np.float64), K, eye, 13, 1 / math.sqrt(8))
    np.testing.assert_allclose(out.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (out >= 0).all()


def check_scale_hand_computed():
    """softmax(q·Kᵀ/√d_head) ("LLM 从头到尾走一遍", attention; "一次 forward 怎么塞下很多个
    request", §6): d_head = 4, q = (2,0,0,0), keys (1,0,0,0) and 0 -> scores 1 and 0,
    weights e/(1+e) and 1/(1+e); V rows are one-hot so the output is the weights."""
    w = _f32([1], [2], hq=1, hkv=1, d=4, ps=2, seed=0)
    w.q[:] = 0
    w.q[0, 0, 0] = 2.0
    w.k_pool[:] = 0
    w.v_pool[:] = 0
    p = int(w.block_table[0, 0])
    w.k_pool[p, 0, 0, 0] = 1.0
    w.v_pool[p, 0, 0, 0] = 1.0      # V[0] = e0 (V page is [D, page_size])
    w.v_pool[p, 0, 1, 1] = 1.0      # V[1] = e1
    out = _run(w)[0, 0]
    e = math.e
    np.testing.assert_allclose(out, [e / (1 + e), 1 / (1 + e), 0, 0], rtol=0, atol=1e-15)


def test_scale_hand_computed():
    check_scale_hand_computed()


# ------------------------------------------------------------- invariants -------

def check_gqa_replication():
    """g query heads per KV head ("How To Scale Your Model 笔记(7-8)", §3 KV 容量与 GQA):
    copying each KV head g times into an MHA pool gives the same result."""
    w = _f32([5, 1, 3], [9, 12, 3], hq=6, hkv=2, d=8, ps=4, seed=21)
    ref = _run(w)
    g = 3
    mha = W.Workload(**{**w.__dict__})
    mha.num_kv_heads = 6
    mha.k_pool = np.repeat(w.k_pool, g, axis=1)
    mha.v_pool = np.repeat(w.v_pool, g, axis=1)
    np.testing.assert_array_equal(_run(mha), ref)


def test_gqa_replication():
    check_gqa_replication()


def test_request_isolation():
    """Requests never read each other ("ORCA 和 chunked prefill", §2; "一次 forward 怎么塞下
    很多个 request", §6.2): changing request B's Q and pages leaves A bit-identical."""
    w = _f32([4, 3], [10, 7], hq=4, hkv=2, d=8, ps=4, seed=23)
    ref = _run(w)
    w2 = W.Workload(**{**w.__dict__})
    w2.q = w.q.copy()
    w2.k_pool = w.k_pool.copy()
    w2.v_pool = w.v_pool.copy()
    w2.q[int(w.q_start[1]):] += 1.0
    pages_b = w.block_table[1, :2]
    w2.k_pool[pages_b] *= -3.0
    w2.v_pool[pages_b] += 5.0
    out = _run(w2)
    np.testing.assert_array_equal(out[:4], ref[:4])
    assert not np.allclose(out[4:], ref[4:])


def check_page_permutation():
    """Paging changes placement, not results ("How To Scale Your Model 笔记(7-8)", §3):
    permuting physical pages and rewriting the block table changes no output bit."""
    w = _f32([3, 1, 6], [11, 9, 6], hq=2, hkv=1, d=8, ps=4, seed=25, permute_pages=False)
    ref = _run(w)
    perm = np.random.default_rng(7).permutation(w.num_pages)
    w2 = W.Workload(**{**w.__dict__})
    w2.k_pool = np.empty_like(w.k_pool)
    w2.v_pool = np.empty_like(w.v_pool)
    w2.k_pool[perm] = w.k_pool
    w2.v_pool[perm] = w.v_pool
    bt = w.block_table.copy()
    bt[bt >= 0] = perm[bt[bt >= 0]]
    w2.block_table = bt
    np.testing.assert_array_equal(_run(w2), ref)


def test_page_permutation_invariance():
    check_page_permutation()


# ------------------------------------------------------------ brute force -------

def check_brute_force(ncases=200, seed=31):
    rng = np.random.default_rng(seed)
    for c in range(ncases):
        R = int(rng.integers(1, 5))
        hkv = int(rng.integers(1, 3))
        g = int(rng.integers(1, 3))
        d = int(rng.integers(1, 9))
        ps = int(rng.choice([1, 2, 4]))
        kv = rng.integers(1, 13, size=R)
        qr = np.array([int(rng.integers(1, k + 1)) for k in kv])
        dtype = "bf16" if c % 2 else "f32"
        w = W.build("b", qr, kv, num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d, page_size=ps,
                    dtype=dtype, seed=1000 + c)
        got = _run(w, threads=1)
        want = np.array(oracle.brute_force_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start,
                                                     w.q_end, w.kv_len, w.page_size))
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12, err_msg=f"case {c}")


def test_bruteforce_tiny():
    check_brute_force()


def test_bf16_decoding_is_exact():
    """bf16 bit patterns decode to the float32 values they round from (within bf16)."""
    x = np.array([1.0, -2.5, 3.140625, 65504.0, 1e-3], np.float32)
    bits = np.empty(x.shape, np.uint16)
    W.f32_to_bf16_bits(x.copy(), bits)
    back = oracle.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(back[:4], [1.0, -2.5, 3.140625, 65536.0])
    assert abs(back[4] - 1e-3) < 1e-3 * 2 ** -8


# ---------------------------------------------------------- byte / FLOP counters -

def test_kv_bytes_closed_forms():
    """c_KV: 32 layers x 8 KV heads x H=128 in bf16 = 128 KiB per position
    ("How To Scale Your Model 笔记(7-8)", §3); 80 layers x 8 x 128 in int8 = 160 KiB and
    8192 positions -> 1.25 GiB = 1.342 GB (same page, §5); Llama-2-7B (32 layers,
    32 heads x 128, fp16) = 2·32·32·128·2 B ~ 512 KB per token ("Prefill/Decode 拆机", §3)."""
    assert oracle.kv_bytes_per_position(32, 8, 128, 2) == 128 * 1024
    assert oracle.kv_bytes_per_position(80, 8, 128, 1) == 160 * 1024
    assert 8192 * oracle.kv_bytes_per_position(80, 8, 128, 1) == int(1.25 * 2 ** 30)
    assert round(8192 * oracle.kv_bytes_per_position(80, 8, 128, 1) / 1e9, 3) == 1.342
    assert oracle.kv_bytes_per_position(32, 32, 128, 2) == 512 * 1024


def test_fp8_scale_bytes_closed_forms():
    """An fp8 vector of 128 elements with its float32 scale is 132 bytes, and 21 layers of
    such one-vector-per-token entries over 1M positions are about 2.9 GB ("GLM-5.3
    推理全链路(八)", the indexer-cache figures)."""
    per_token_layer = oracle.kv_bytes_per_position(1, 1, 128, 1, 4) // 2     # K only
    assert per_token_layer == 132
    assert round(21 * per_token_layer * 1048576 / 1e9, 1) == 2.9
    # K and V of 8 KV heads x 128 in fp8 with scales: 2 * 8 * 132 bytes per position
    assert oracle.kv_bytes_per_position(1, 8, 128, 1, 4) == 2112


def test_shared_prefix_bytes():
    """Six requests sharing 4096 positions + 1024 private each, 32 layers x 8 KV heads x
    H=128 bf16: 3.75 GiB read naively vs 1.25 GiB stored ("How To Scale Your Model
    笔记(7-8)", §3 物理存一份...).  Counted on the shared-prefix workload's own block
    tables."""
    w = W.config(5)
    logical = oracle.logical_kv_bytes(w.kv_len, 8, 128, 2, layers=32)
    physical = oracle.physical_kv_bytes(w.block_table, w.kv_len, 64, 8, 128, 2, layers=32)
    assert logical == int(3.75 * 2 ** 30)
    assert physical == int(1.25 * 2 ** 30)
    assert oracle.logical_kv_bytes(w.kv_len, 8, 128, 2) == 120 * 2 ** 20
    assert oracle.physical_kv_bytes(w.block_table, w.kv_len, 64, 8, 128, 2) == 40 * 2 ** 20


def _printed(value, printed, sig):
    """value rounds to the printed figure at the printed precision (sig = place value)."""
    return abs(value - printed) <= 0.5 * sig


def test_flop_counter_matches_cost_table():
    """Llama-2-7B (32 layers, 32 heads, d_head 128): 4·128·32·32 ≈ 0.52 MFLOP per pair;
    attention of a causal prefill of 1k / 4k / 16k / 100k tokens ≈ 0.3 / 4 / 67 / 2600 TF,
    10k ≈ 26 TF, 8 decodes at ~1k ≈ 4 GF ("ORCA 和 chunked prefill", §3 tables)."""
    per_pair = 4 * 128 * 32 * 32
    assert _printed(per_pair / 1e6, 0.52, 0.01)

    def net(q, kv):       # whole network = 32 layers of 32 heads
        return 32 * oracle.attention_flops(q, kv, 32, 128)

    assert _printed(net([1000], [1000]) / 1e12, 0.3, 0.1)
    assert _printed(net([4000], [4000]) / 1e12, 4, 1)
    assert _printed(net([16000], [16000]) / 1e12, 67, 1)
    assert _printed(net([100000], [100000]) / 1e15, 2.6, 0.1)
    assert _printed(net([10000], [10000]) / 1e12, 26, 1)
    assert _printed(net([1] * 8, [1000] * 8) / 1e9, 4, 1)


def test_varlen_block_arithmetic():
    """cu_seqlens [0, 10, 40]: the diagonal blocks hold 10² + 30² = 1000 scores against
    1600 for the whole 40 x 40, 600 wasted; 1 request of 1000 tokens costs 10⁶ against
    10⁵ for 10 of 100 ("一次 forward 怎么塞下很多个 request", §6.1, §8)."""
    blocks = [oracle.visibility_mask(0, n).size for n in (10, 30)]
    assert sum(blocks) == 1000 and 40 * 40 - sum(blocks) == 600
    assert oracle.visibility_mask(0, 1000).size == 10 ** 6
    assert 10 * oracle.visibility_mask(0, 100).size == 10 ** 5


# ----------------------------------------------------------------- mutants ------

def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    return False


ALL_CHECKS = [check_mask_worked_example, check_scale_hand_computed, check_gqa_replication,
              check_page_permutation, lambda: check_brute_force(ncases=40, seed=77)]


def test_mutants_are_caught(monkeypatch):
    """Plant plausible mistakes in the oracle; at least one pin must fail for each."""
    real_mask, real_gather, real_attend = OA.visibility_mask, OA.gather_kv, OA.attend

    def mask_off_by_one(S0, m):
        mk = real_mask(S0, m)
        mk[:, S0:] = np.tril(np.ones((m, m), bool), k=-1)
        mk[:, S0] = True            # keep each row non-empty
        return mk

    def mask_upper(S0, m):
        mk = real_mask(S0, m)
        mk[:, S0:] = np.triu(np.ones((m, m), bool))
        return mk

    def gather_v_untransposed(k_pool, v_pool, row, L, kvh, ps):
        K, _ = real_gather(k_pool, v_pool, row, L, kvh, ps)
        j = np.arange(L)
        pages = np.asarray(row)[j // ps].astype(np.int64)
        as_rows = v_pool.reshape(v_pool.shape[0], v_pool.shape[1], ps, -1)     # read as [ps, D]
        return K, OA.to_f64(as_rows[pages, kvh, j % ps, :])

    def gather_wrong_slot(k_pool, v_pool, row, L, kvh, ps):
        j = np.arange(L)
        pages = np.asarray(row)[j // ps].astype(np.int64)
        slots = (ps - 1 - j % ps)
        return OA.to_f64(k_pool[pages, kvh, slots, :]), OA.to_f64(v_pool[pages, kvh, :, slots])

    def attend_no_scale(q, K, V, S0, scale, row_ids=None):
        return real_attend(q, K, V, S0, 1.0, row_ids)

    def attend_no_norm(q, K, V, S0, scale, row_ids=None):
        m = K.shape[0] - S0
        row_ids = np.arange(m) if row_ids is None else row_ids
        S = np.where(OA.visibility_mask(S0, m)[row_ids], (q @ K.T) * scale, -np.inf)
        return np.exp(S - S.max(axis=1, keepdims=True)) @ V

    mutants = {
        "mask off by one": ("visibility_mask", mask_off_by_one),
        "mask transposed": ("visibility_mask", mask_upper),
        "V page not transposed": ("gather_kv", gather_v_untransposed),
        "slot index reversed": ("gather_kv", gather_wrong_slot),
        "scale dropped": ("attend", attend_no_scale),
        "softmax not normalised": ("attend", attend_no_norm),
    }
    for name, (attr, fn) in mutants.items():
        with monkeypatch.context() as mp:
            mp.setattr(OA, attr, fn)
            mp.setattr(oracle, attr, fn, raising=False)
            assert any(_fails(c) for c in ALL_CHECKS), f"no pin catches mutant: {name}"

    # wrong GQA mapping (h % Hkv instead of h // g): caught by the replication pin
    real_rows = OA.attention_rows

    def rows_mod(q, k_pool, v_pool, bt, qs, qe, kv, ps, req, rows=None, heads=None, softmax_scale=None):
        Hq, Hkv = q.shape[1], k_pool.shape[1]
        heads = range(Hq) if heads is None else list(heads)
        out = {}
        for h in heads:
            # route head h through KV head h % Hkv by presenting a pool whose head h//g is that
            kvh_wrong = h % Hkv
            g = Hq // Hkv
            kp = k_pool.copy(); vp = v_pool.copy()
            kp[:, h // g] = k_pool[:, kvh_wrong]; vp[:, h // g] = v_pool[:, kvh_wrong]
            out.update(real_rows(q, kp, vp, bt, qs, qe, kv, ps, req, rows, [h], softmax_scale))
        return out

    with monkeypatch.context() as mp:
        mp.setattr(OA, "attention_rows", rows_mod)
        assert _fails(check_gqa_replication)


# ------------------------------------------------------------ KV append ----------

def test_append_slots_worked_example():
    """Hand-derived slot mapping ("GLM-5.3 推理全链路(八)", stage 4; tests/golden)."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "kv_append_slots.txt"))
            if l.strip() and not l.startswith("#")]
    want = np.array([int(r[1]) for r in rows], np.int64)
    bt = np.array([[5, 2], [7, -1], [1, 0]], np.int32)
    got = oracle.slots_for_new_rows([0, 2, 3], [2, 3, 5], [5, 1, 8], bt, 4, 6)
    assert np.array_equal(got, want)


def _bits_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_then_gather_round_trip(dtype):
    """Writing the new rows' K/V back through the slot mapping restores the pools bit for
    bit, and the request's gather reads them at positions S0 .. kv_len-1 ("ORCA 和 chunked
    prefill", section 3: append, then attention reads the whole prefix)."""
    w = W.build("a", [5, 1, 3], [9, 40, 3], num_q_heads=4, num_kv_heads=2, head_dim=8, page_size=4,
                dtype=dtype, seed=11)
    loc = oracle.slots_for_new_rows(w.q_start, w.q_end, w.kv_len, w.block_table, w.page_size, w.total_q_rows)
    Hkv, D = w.num_kv_heads, w.head_dim
    k_new = np.zeros((w.total_q_rows, Hkv, D), w.k_pool.dtype)
    v_new = np.zeros_like(k_new)
    for r in range(w.num_reqs):
        m = int(w.q_end[r] - w.q_start[r])
        S0 = int(w.kv_len[r]) - m
        for i in range(m):
            pos = S0 + i
            page, slot = w.block_table[r][pos // w.page_size], pos % w.page_size
            k_new[w.q_start[r] + i] = w.k_pool[page, :, slot, :]
            v_new[w.q_start[r] + i] = w.v_pool[page, :, :, slot]
    # blank the new slots, then append: the original pools come back
    kb, vb = w.k_pool.copy(), w.v_pool.copy()
    for t, l in enumerate(loc):
        if l >= 0:
            kb[l // w.page_size, :, l % w.page_size, :] = 0
            vb[l // w.page_size, :, :, l % w.page_size] = 0
    assert not _bits_equal(kb, w.k_pool)
    k2, v2 = oracle.append_kv(kb, vb, k_new, v_new, loc, w.page_size)
    assert _bits_equal(k2, w.k_pool) and _bits_equal(v2, w.v_pool)
    # and the gather of request r reads token t's rows at position S0 + i
    for r in range(w.num_reqs):
        m = int(w.q_end[r] - w.q_start[r])
        for kvh in range(Hkv):
            K, V = OA.gather_kv(k2, v2, w.block_table[r], int(w.kv_len[r]), kvh, w.page_size)
            assert np.array_equal(K[-m:], OA.to_f64(k_new[w.q_start[r]:w.q_end[r], kvh, :]))
            assert np.array_equal(V[-m:], OA.to_f64(v_new[w.q_start[r]:w.q_end[r], kvh, :]))


def test_append_padding_writes_nothing():
    w = W.build("p", [2], [6], num_q_heads=2, num_kv_heads=1, head_dim=8, page_size=4, dtype="f32", seed=2)
    k_new = np.full((3, 1, 8), 9.0, np.float32)
    v_new = np.full((3, 1, 8), 9.0, np.float32)
    k2, v2 = oracle.append_kv(w.k_pool, w.v_pool, k_new, v_new, np.array([-1, -1, -1]), 4)
    assert _bits_equal(k2, w.k_pool) and _bits_equal(v2, w.v_pool)
    # one real entry changes exactly D values in each pool
    k3, v3 = oracle.append_kv(w.k_pool, w.v_pool, k_new, v_new, np.array([-1, 5, -1]), 4)
    assert int((k3 != w.k_pool).sum()) <= 8 and np.all(k3[1, 0, 1, :] == 9.0) and np.all(v3[1, 0, :, 1] == 9.0)
