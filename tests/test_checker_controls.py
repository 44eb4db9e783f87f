"""CPU checks of the sampled parity check itself (no GPU).

* The oracle's row-subset path (``attention_rows(rows=..., heads=...)``, which every
  full-size sampled test uses) equals the same rows of the full oracle and of the scalar
  brute force.
* ``workloads.focus`` changes only the elements it documents, and keeps outputs O(1)
  where N(0,1) inputs make them vanish (at 131,072 keys an all-zero output would pass the
  2e-2 check on N(0,1) inputs: shown here).
* Negative controls at the full context lengths of the long workloads: on focused inputs
  the sampled comparison rejects an all-zero output and the oracle with one hot 64-key
  step dropped or doubled, each by more than 0.1 (five times the tolerance).
"""
import numpy as np
import pytest

import oracle
from varlen_paged_attention_amd import workloads as W

import sampled

TOL = 2e-2


@pytest.mark.parametrize("cid,scale,flags", [(1, 1, None), (2, 16, None), (4, 32, None), (51, 16, None), (9, 64, None),
                                             (7, 32, None)])
def test_attention_rows_subset_equals_full_oracle(cid, scale, flags):
    w = W.config(cid, scale=scale)
    full = oracle.varlen_paged_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                         w.page_size, threads=1)
    rng = np.random.default_rng(cid)
    for r in sorted({0, w.num_reqs - 1, int(rng.integers(w.num_reqs))}):
        m = int(w.q_end[r] - w.q_start[r])
        rows = sorted(set(int(x) for x in rng.choice(m, size=min(m, 5), replace=False)) | {m - 1})
        heads = sorted(set(int(x) for x in rng.choice(w.num_q_heads, size=min(3, w.num_q_heads), replace=False)))
        sub = oracle.attention_rows(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                    w.page_size, r, rows, heads)
        assert sorted(sub) == heads
        for h in heads:
            want = full[int(w.q_start[r]) + np.asarray(rows), h, :]
            assert sub[h].shape == want.shape
            assert np.abs(sub[h] - want).max() <= 1e-12


def test_attention_rows_subset_equals_brute_force():
    """Row and head subsets of tiny random cases against the scalar triple loop."""
    rng = np.random.default_rng(11)
    for case in range(40):
        R = int(rng.integers(1, 4))
        hkv = int(rng.integers(1, 3))
        g = int(rng.integers(1, 3))
        ps = int(rng.choice([1, 2, 4]))
        kv = [int(rng.integers(1, 12)) for _ in range(R)]
        m = [int(rng.integers(1, k + 1)) for k in kv]
        w = W.build(f"b{case}", m, kv, num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=4, page_size=ps,
                    dtype="f32", seed=case)
        brute = oracle.brute_force_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                             w.page_size)
        for r in range(R):
            rows = sorted(set(int(x) for x in rng.choice(m[r], size=min(m[r], 2), replace=False)))
            heads = [int(rng.integers(hkv * g))]
            sub = oracle.attention_rows(w.q, w.k_pool, w.v_pool, w.block_table, w.q_start, w.q_end, w.kv_len,
                                        w.page_size, r, rows, heads)
            for h in heads:
                want = np.asarray(brute)[int(w.q_start[r]) + np.asarray(rows), h, :]
                assert np.abs(sub[h] - want).max() <= 1e-12


def _bf16(bits):
    return oracle.to_f64(bits)


def test_focus_changes_only_documented_elements():
    w = W.config(3, scale=16)
    f = W.focus(w)
    g = w.num_q_heads // w.num_kv_heads
    info = f.notes["focus"]
    # Q: every element scaled by q_rest exactly, the marker element of each head = peak
    q0, q1 = _bf16(w.q), _bf16(f.q)
    mark = np.zeros(q1.shape, bool)
    for h in range(w.num_q_heads):
        mark[:, h, info["dcol"][h % g]] = True
    assert np.array_equal(q1[~mark], q0[~mark] * info["q_rest"])
    assert (q1[mark] == info["peak"]).all()
    # K/V: only the hot keys' marker elements differ
    k0, k1, v0, v1 = _bf16(w.k_pool), _bf16(f.k_pool), _bf16(w.v_pool), _bf16(f.v_pool)
    km = np.zeros(k1.shape, bool)
    vm = np.zeros(v1.shape, bool)
    n = 0
    for (r, kvh, c), pos in f.notes["hot"].items():
        d = info["dcol"][c]
        for k, j in enumerate(pos):
            p, s = w.block_table[r, j // w.page_size], j % w.page_size
            km[p, kvh, s, d] = True
            vm[p, kvh, d, s] = True
            assert k1[p, kvh, s, d] == info["peak"]
            assert abs(v1[p, kvh, d, s]) == info["v_mark"]
            n += 1
        # one hot key per segment of colour c
        L, nseg = int(w.kv_len[r]), info["hot"] * g
        bounds = np.arange(nseg + 1) * L // nseg                 # segment s is [bounds[s], bounds[s+1])
        segs = np.searchsorted(bounds, pos, side="right") - 1
        assert list(segs % g) == [c] * len(pos) and len(set(segs)) == len(pos)
    assert n > 0
    assert np.array_equal(k0[~km], k1[~km]) and np.array_equal(v0[~vm], v1[~vm])


def test_focus_shared_prefix_marks_shared_pages_once():
    """Members of a shared prefix get the same hot keys inside the shared pages, so each
    member still sees `hot` keys of each colour."""
    f = W.focus(W.config(51, scale=16))
    sl = f.shared_prefix_pages * f.page_size
    for kvh in range(f.num_kv_heads):
        for c in range(f.num_q_heads // f.num_kv_heads):
            shared = {tuple(int(j) for j in f.notes["hot"][(r, kvh, c)] if j < sl) for r in range(f.num_reqs)}
            assert len(shared) == 1
            assert len(f.notes["hot"][(0, kvh, c)]) == f.notes["focus"]["hot"]


def test_focus_fp8_requantises_marked_vectors():
    w = W.config(3, scale=32, dtype="fp8")
    f = W.focus(w)
    K0, V0 = oracle.dequantize_pools(w.k_pool, w.k_scale, w.v_pool, w.v_scale)
    K1, V1 = oracle.dequantize_pools(f.k_pool, f.k_scale, f.v_pool, f.v_scale)
    info = f.notes["focus"]
    g = w.num_q_heads // w.num_kv_heads
    changed = 0
    for (r, kvh, c), pos in f.notes["hot"].items():
        d = info["dcol"][c]
        for j in pos:
            p, s = w.block_table[r, j // w.page_size], j % w.page_size
            # the largest element of its vector: code 448 times the float32 scale max / 448
            assert abs(K1[p, kvh, s, d] - info["peak"]) <= 1e-6 * info["peak"]
            # V marks are the largest element of their column unless a drawn value is larger:
            # then they round to within half an e4m3 step (2^-4 relative)
            assert abs(abs(V1[p, kvh, d, s]) - info["v_mark"]) <= 2 ** -4 * info["v_mark"]
            # the rest of the vector moves by at most one step of its new scale
            others = np.arange(w.head_dim) != d
            assert np.abs(K1[p, kvh, s, others] - K0[p, kvh, s, others]).max() <= 16 / 448 * 16 + 1e-12
            changed += 1
    assert changed > 0


def test_hashed_marks_on_host_pages():
    w = W.config(8, scale=1024)                   # 1 request x 128 positions, hashed pools
    f = W.focus(w)
    pages = np.arange(f.num_pages)
    k0, v0 = W.host_kv_pages(w, pages)
    k1, v1 = W.host_kv_pages(f, pages)
    kd = np.argwhere(k0 != k1)
    vd = np.argwhere(v0 != v1)
    n = sum(len(p) for p in f.notes["hot"].values())
    assert len(kd) == n and len(vd) == n
    # hashing a subset of KV heads gives the same values for those heads
    ks, vs = W.host_kv_pages(f, pages[:2], kv_heads=[1])
    assert np.array_equal(ks[:, 1], k1[:2, 1]) and np.array_equal(vs[:, 1], v1[:2, 1])
    assert not ks[:, 0].any()


def test_plain_inputs_are_blind_at_128k_and_focus_is_not():
    """At 131,072 keys the N(0,1)-like hashed inputs give outputs below the tolerance (an
    all-zero output would pass); on focused inputs the same rows are O(1)."""
    w = W.build("lc1", [1], [131072], num_q_heads=4, num_kv_heads=1, head_dim=128, page_size=64, seed=8,
                hashed_kv=True)
    plain = sampled.oracle_rows(w, 0, [0], [0, 3])
    assert max(float(np.abs(o).max()) for o in plain.values()) < TOL
    f = W.focus(w)
    foc = sampled.oracle_rows(f, 0, [0], [0, 3])
    assert min(float(np.abs(o).max()) for o in foc.values()) > 0.5


# Long-context shapes at their full lengths (few requests, so the CPU suite stays short).
LONG = [
    ("decode kv 8192 (g=4, page 64)", lambda: W.build("d", [1, 1, 1], [8192, 1024, 5000], num_q_heads=32,
                                                      num_kv_heads=8, head_dim=128, page_size=64, seed=3), [0]),
    ("chunk 2048 rows on S0=30720 (g=8)", lambda: W.build("c", [2048], [32768], num_q_heads=64, num_kv_heads=8,
                                                          head_dim=128, page_size=64, seed=4), [0, 777, 2047]),
    ("chunk 256 rows on S0=65536 (g=4)", lambda: W.build("l", [256], [65792], num_q_heads=32, num_kv_heads=8,
                                                         head_dim=128, page_size=64, seed=9), [0, 255]),
    ("shared prefix 16384 + 1024 (g=4)", lambda: W.build("s", [1, 1], [17408, 17408], num_q_heads=32,
                                                         num_kv_heads=8, head_dim=128, page_size=64, seed=51,
                                                         shared_prefix_pages=256), [0]),
    ("decode 131072, hashed pages (g=4)", lambda: W.build("h", [1], [131072], num_q_heads=8, num_kv_heads=2,
                                                          head_dim=128, page_size=64, seed=8, hashed_kv=True), [0]),
    ("fp8 decode kv 8192", lambda: W.build("f", [1], [8192], num_q_heads=8, num_kv_heads=2, head_dim=128,
                                           page_size=64, seed=3, dtype="fp8"), [0]),
]


@pytest.mark.parametrize("label,make,rows", LONG, ids=[x[0] for x in LONG])
def test_controls_reject_planted_mistakes_at_full_length(label, make, rows):
    f = W.focus(make())
    g = f.num_q_heads // f.num_kv_heads
    heads = [0, g - 1, f.num_q_heads - 1]
    for r in range(f.num_reqs):
        ref = sampled.oracle_rows(f, r, rows if r == 0 else [0], heads)
        margin = sampled.controls(f, r, rows if r == 0 else [0], heads, ref, TOL)
        assert margin > 5 * TOL, f"{label}: request {r}: a planted mistake moves the output by only {margin:.3e}"
