"""Seeded synthetic inputs for varlen paged attention.

This module only builds inputs: request metadata, block tables, and the Q / K / V
values.  It holds none of the attention arithmetic, and it is the one module that
both the HIP path (tests, bench) and the CPU oracle's tests read inputs from.

Shapes follow the worked workloads of the pages:

* the ORCA iteration of one 4096-token prefill plus decodes at 1500 and 1700
  cached positions ("ORCA 和 chunked prefill", section 2 table);
* decode-heavy and chunked-prefill mixes ("ORCA 和 chunked prefill", sections 4-5);
* six requests sharing a 4096-position prefix with 1024 private positions each
  ("How To Scale Your Model 笔记(7-8)", section 3, "物理存一份，不保证从 HBM 只读一次").

Memory layout (the library's own layout, described in include/varlen_attn.h):

* ``q``      : ``[total_q_rows, num_q_heads, head_dim]``
* ``k_pool`` : ``[num_pages, num_kv_heads, page_size, head_dim]``
* ``v_pool`` : ``[num_pages, num_kv_heads, head_dim, page_size]``  (transposed page)

bf16 tensors are carried as ``uint16`` bit patterns (numpy has no bf16); fp32 as
``float32``.  Draw recipe (deterministic, independent of thread count): every
stream ``s`` (0 lengths, 1 page permutation, 2 Q, 3 K pool, 4 V pool) draws from
``numpy.random.default_rng(SeedSequence([seed, s, chunk]))``; values are float32
N(0,1) drawn in memory order in chunks of ``CHUNK`` elements and rounded to bf16
with round-to-nearest-even.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

CHUNK = 1 << 22
STREAM_LENGTHS, STREAM_PERM, STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2, 3, 4
BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
FP8_MAX = 448.0             # largest finite e4m3fn value


def quantize_fp8(x: np.ndarray, axis: int):
    """Per-vector fp8 e4m3fn storage of float32 ``x``: one float32 scale per vector along
    ``axis`` (its absolute maximum / 448, 1 for an all-zero vector) and the codes of
    x / scale rounded to nearest even by torch's float8_e4m3fn conversion.  Returns
    (uint8 codes shaped like x, float32 scales with ``axis`` removed)."""
    import torch
    amax = np.abs(x).max(axis=axis)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / np.expand_dims(scale, axis)).astype(np.float32)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, stream, chunk]))


def f32_to_bf16_bits(x: np.ndarray, out: np.ndarray) -> None:
    """Round float32 to bf16 (nearest, ties to even) into ``out`` (uint16 bits)."""
    u = x.view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    out[...] = r


def _normal_fill(seed: int, stream: int, n: int, bf16: bool, fp8_vec: Optional[tuple] = None):
    """n standard normal float32 draws (chunk c from its own seeded stream), stored as
    float32, as bf16 bits, or -- with ``fp8_vec`` = (D, stride) -- as e4m3fn codes with
    one scale per vector of D elements spaced ``stride`` apart inside blocks of D*stride
    elements (stride 1: K rows, stride page_size: V columns of a transposed page); then
    returns (codes, scales).  Chunks hold whole blocks, so the draws do not depend on the
    storage type."""
    if fp8_vec is not None:
        D, stride = fp8_vec
        assert CHUNK % (D * stride) == 0 and n % (D * stride) == 0
        out = np.empty(n, np.uint8)
        scales = np.empty(n // D, np.float32)
    else:
        out = np.empty(n, np.uint16 if bf16 else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def job(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = _rng(seed, stream, c)
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if fp8_vec is not None:
            codes, sc = quantize_fp8(x.reshape(-1, D, stride), axis=1)
            out[lo:hi] = codes.reshape(-1)
            scales[lo // D:hi // D] = sc.reshape(-1)
        elif bf16:
            f32_to_bf16_bits(x, out[lo:hi])
        else:
            out[lo:hi] = x

    if nchunks <= 1:
        for c in range(nchunks):
            job(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, range(nchunks)))
    return out if fp8_vec is None else (out, scales)


@dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    dtype: str                      # "bf16", "f32" or "fp8" (bf16 Q/out, fp8 e4m3fn K/V + scales)
    q_start: np.ndarray             # int32 [R]
    q_end: np.ndarray               # int32 [R]
    kv_len: np.ndarray              # int32 [R]
    block_table: np.ndarray         # int32 [R, max_pages]; unused entries are -1
    num_pages: int
    q: np.ndarray                   # [T, Hq, D]
    k_pool: np.ndarray              # [P, Hkv, ps, D]
    v_pool: np.ndarray              # [P, Hkv, D, ps]
    softmax_scale: float = 0.0      # <= 0 means 1/sqrt(head_dim)
    shared_prefix_pages: int = 0    # leading pages shared by every request (0: none)
    hashed_kv: bool = False         # K/V not held on the host: made page by page by hashed_pages*
    seed: int = 0
    k_scale: Optional[np.ndarray] = None   # fp8 only: float32 [P, Hkv, ps], one per K row
    v_scale: Optional[np.ndarray] = None   # fp8 only: float32 [P, Hkv, ps], one per V column
    notes: dict = field(default_factory=dict)
    # hashed pools only: elements overwritten after the hash (see ``focus``): int64 rows
    # (pool, page, kv_head, slot, d) with pool STREAM_K or STREAM_V, and their float values
    marks: Optional[np.ndarray] = None
    mark_values: Optional[np.ndarray] = None

    @property
    def num_reqs(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def total_q_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_pages_per_req(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def elem_bytes(self) -> int:
        """Bytes of one stored K or V element."""
        return {"bf16": 2, "f32": 4, "fp8": 1}[self.dtype]

    @property
    def scale_bytes(self) -> int:
        """Bytes of the scale stored with each K or V vector (fp8: one float32)."""
        return 4 if self.dtype == "fp8" else 0


def build(name: str, q_rows: Sequence[int], kv_lens: Sequence[int], *, num_q_heads: int,
          num_kv_heads: int, head_dim: int, page_size: int, dtype: str = "bf16", seed: int = 0,
          permute_pages: bool = True, shared_prefix_pages: int = 0, poison_tail: bool = False,
          extra_pages: int = 0, softmax_scale: float = 0.0, hashed_kv: bool = False) -> Workload:
    """Build a workload from per-request (q_rows, kv_length) pairs.

    Requests' Q rows are laid out back to back in request order.  Each request owns
    ``ceil(kv_len / page_size)`` logical pages, except that with ``shared_prefix_pages``
    > 0 the first that many logical pages of every request are one set of pages held
    once in the pool.  The pool holds exactly the pages in use (+ ``extra_pages``
    never referenced), permuted by a seeded permutation when ``permute_pages``.
    With ``poison_tail`` the slots past kv_len in each tail page (and the extra pages)
    hold NaN, so any read beyond a request's length shows in its output.
    With ``hashed_kv`` (bf16 only) the K/V pools are not built on the host: every page's
    values come from a counter-based hash of (seed, pool, page, element), made on the
    device by ``hashed_pools_device`` and for any pages on the host by
    ``hashed_pages_host`` (pools too large for host memory).
    """
    q_rows = np.asarray(q_rows, np.int64)
    kv = np.asarray(kv_lens, np.int64)
    R = len(kv)
    assert q_rows.shape == (R,)
    fp8 = dtype == "fp8"
    bf16 = dtype == "bf16" or fp8
    ps = page_size
    npg = (kv + ps - 1) // ps
    sp = shared_prefix_pages
    if sp:
        assert np.all(npg >= sp), "every request must cover the shared prefix"
    # logical page ids: the shared prefix first, then each request's own pages
    owned = npg - sp if sp else npg
    P = int(sp + owned.sum()) + extra_pages
    perm = _rng(seed, STREAM_PERM).permutation(P) if permute_pages else np.arange(P)
    maxp = int(npg.max()) if R else 1
    bt = np.full((R, max(1, maxp)), -1, np.int32)
    nxt = sp
    for r in range(R):
        logical = list(range(sp)) + list(range(nxt, nxt + int(owned[r])))
        nxt += int(owned[r])
        bt[r, : len(logical)] = perm[np.asarray(logical, np.int64)] if logical else []
    qs = np.concatenate([[0], np.cumsum(q_rows)[:-1]]).astype(np.int32) if R else np.zeros(0, np.int32)
    qe = (qs + q_rows).astype(np.int32)
    T = int(q_rows.sum())
    D = head_dim
    q = _normal_fill(seed, STREAM_Q, T * num_q_heads * D, bf16).reshape(T, num_q_heads, D)
    k_scale = v_scale = None
    if hashed_kv:
        assert dtype == "bf16" and not poison_tail and not extra_pages
        k = v = None
    elif fp8:
        k, k_scale = _normal_fill(seed, STREAM_K, P * num_kv_heads * ps * D, False, fp8_vec=(D, 1))
        v, v_scale = _normal_fill(seed, STREAM_V, P * num_kv_heads * D * ps, False, fp8_vec=(D, ps))
        k, k_scale = k.reshape(P, num_kv_heads, ps, D), k_scale.reshape(P, num_kv_heads, ps)
        v, v_scale = v.reshape(P, num_kv_heads, D, ps), v_scale.reshape(P, num_kv_heads, ps)
    else:
        k = _normal_fill(seed, STREAM_K, P * num_kv_heads * ps * D, bf16).reshape(P, num_kv_heads, ps, D)
        v = _normal_fill(seed, STREAM_V, P * num_kv_heads * D * ps, bf16).reshape(P, num_kv_heads, D, ps)
    if poison_tail and not hashed_kv:
        nanv = FP8_NAN if fp8 else (BF16_NAN if bf16 else np.float32(np.nan))
        for r in range(R):
            valid = int(kv[r]) - (int(npg[r]) - 1) * ps
            if int(npg[r]) > 0 and valid < ps:
                p = bt[r, int(npg[r]) - 1]
                k[p, :, valid:, :] = nanv
                v[p, :, :, valid:] = nanv
                if fp8:
                    k_scale[p, :, valid:] = np.nan
                    v_scale[p, :, valid:] = np.nan
        for u in range(P - extra_pages, P):
            k[perm[u]] = nanv
            v[perm[u]] = nanv
            if fp8:
                k_scale[perm[u]] = np.nan
                v_scale[perm[u]] = np.nan
    return Workload(name=name, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=D,
                    page_size=ps, dtype=dtype, q_start=qs, q_end=qe, kv_len=kv.astype(np.int32),
                    block_table=bt, num_pages=P, q=q, k_pool=k, v_pool=v, softmax_scale=softmax_scale,
                    shared_prefix_pages=sp, k_scale=k_scale, v_scale=v_scale, hashed_kv=hashed_kv, seed=seed)


# ---- counter-based page values (pools too large to build on the host) ----------------
# Element e of physical page p of pool s (3 = K, 4 = V) is a function of (seed, s, p, e)
# only: key = h(h(seed) ^ s), page key = h(p ^ key), u = h(e ^ page key), where h is the
# 32-bit "lowbias32" integer hash (xor-shift 16, multiply 0x7feb352d, xor-shift 15,
# multiply 0x846ca68b, xor-shift 16, all modulo 2^32; C. Wellons, "Prospecting for hash
# functions").  The value is (byte0(u) + byte1(u) - 255) / 128: a triangular
# distribution on [-1.99, 1.99] (std 0.82) whose every value is exact in bf16.  The same
# integer steps run in NumPy (host) and in torch (device), with products split so that no
# intermediate exceeds 2^48, so both give identical bits.
_M32 = 0xFFFFFFFF
_H1, _H2 = 0x7FEB352D, 0x846CA68B


def _mul32(x, c: int):
    """(x * c) mod 2^32 for 0 <= x < 2^32 without intermediates above 2^48 (x: int64
    array or tensor)."""
    lo, hi = c & 0xFFFF, c >> 16
    return ((((x * hi) & 0xFFFF) << 16) + x * lo) & _M32


def _lowbias32(x):
    x = x ^ (x >> 16)
    x = _mul32(x, _H1)
    x = x ^ (x >> 15)
    x = _mul32(x, _H2)
    return x ^ (x >> 16)


def _pool_key(seed: int, stream: int) -> int:
    k = int(_lowbias32(np.array([seed & _M32], np.int64))[0])
    return int(_lowbias32(np.array([k ^ stream], np.int64))[0])


def _page_elems(w: "Workload") -> int:
    return w.num_kv_heads * w.page_size * w.head_dim


def hashed_pages_host(w: "Workload", pages, stream: int, kv_heads=None) -> np.ndarray:
    """bf16 bits (uint16) of the given physical pages of pool ``stream`` (STREAM_K or
    STREAM_V) of a hashed workload: [len(pages), Hkv, ps, D] for K, [len(pages), Hkv, D, ps]
    for V, with the workload's marks applied.  ``kv_heads``: hash only these KV heads (the
    others are left 0)."""
    H, ps, D = w.num_kv_heads, w.page_size, w.head_dim
    pages = np.asarray(pages, np.int64)
    per_head = ps * D
    heads = range(H) if kv_heads is None else sorted(set(int(x) for x in kv_heads))
    key = _pool_key(w.seed, stream)
    pk = _lowbias32(pages[:, None] ^ key)
    bits = np.zeros((len(pages), H * per_head), np.uint16)
    for h in heads:
        e = np.arange(h * per_head, (h + 1) * per_head, dtype=np.int64)[None, :]
        u = _lowbias32(e ^ pk)
        vals = ((u & 0xFF) + ((u >> 8) & 0xFF) - 255).astype(np.float32) / np.float32(128.0)
        f32_to_bf16_bits(np.ascontiguousarray(vals), bits[:, h * per_head:(h + 1) * per_head])
    out = bits.reshape((len(pages), H, ps, D) if stream == STREAM_K else (len(pages), H, D, ps))
    if w.marks is not None and len(w.marks):
        sel = w.marks[:, 0] == stream
        mk, mv = w.marks[sel], w.mark_values[sel]
        where = {int(p): i for i, p in enumerate(pages)}
        vb = np.empty(len(mv), np.uint16)
        f32_to_bf16_bits(np.ascontiguousarray(mv, np.float32), vb)
        hs = set(heads)
        for (_, page, kvh, slot, d), b in zip(mk, vb):
            i = where.get(int(page))
            if i is None or int(kvh) not in hs:
                continue
            if stream == STREAM_K:
                out[i, kvh, slot, d] = b
            else:
                out[i, kvh, d, slot] = b
    return out


def hashed_pools_device(w: "Workload", device="cuda", pages_per_chunk: Optional[int] = None):
    """The K and V pools of a hashed workload, made on the device (bf16 torch tensors), in
    chunks of about 2^28 elements (2 GiB int64 intermediates) unless pages_per_chunk says."""
    import torch
    E = _page_elems(w)
    if pages_per_chunk is None:
        pages_per_chunk = max(1, (1 << 28) // E)
    H, ps, D = w.num_kv_heads, w.page_size, w.head_dim
    elems = torch.arange(E, dtype=torch.int64, device=device)[None, :]
    out = []
    for stream, shape in ((STREAM_K, (w.num_pages, H, ps, D)), (STREAM_V, (w.num_pages, H, D, ps))):
        pool = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = pool.view(w.num_pages, E)
        key = _pool_key(w.seed, stream)
        for p0 in range(0, w.num_pages, pages_per_chunk):
            p1 = min(w.num_pages, p0 + pages_per_chunk)
            pk = _lowbias32(torch.arange(p0, p1, dtype=torch.int64, device=device)[:, None] ^ key)
            u = _lowbias32(elems ^ pk)
            flat[p0:p1] = (((u & 0xFF) + ((u >> 8) & 0xFF) - 255).to(torch.float32) / 128.0).to(torch.bfloat16)
            del pk, u
        if w.marks is not None and len(w.marks):
            sel = w.marks[:, 0] == stream
            if sel.any():
                mk = torch.from_numpy(w.marks[sel]).to(device)
                mv = torch.from_numpy(np.ascontiguousarray(w.mark_values[sel], np.float32)).to(device)
                idx = (mk[:, 1], mk[:, 2], mk[:, 3], mk[:, 4]) if stream == STREAM_K else \
                      (mk[:, 1], mk[:, 2], mk[:, 4], mk[:, 3])
                pool.index_put_(idx, mv.to(torch.bfloat16))
        out.append(pool)
    return out[0], out[1]


def host_kv_pages(w: "Workload", pages, kv_heads=None):
    """(K, V) host values of the given physical pages, for any workload (hashed pools: only
    the KV heads in ``kv_heads`` are filled when it is given)."""
    pages = np.asarray(pages, np.int64)
    if w.hashed_kv:
        return (hashed_pages_host(w, pages, STREAM_K, kv_heads), hashed_pages_host(w, pages, STREAM_V, kv_heads))
    return w.k_pool[pages], w.v_pool[pages]


def subset(w: Workload, reqs: Sequence[int], name: Optional[str] = None) -> Workload:
    """The iteration made of requests ``reqs`` of ``w`` only: their Q rows laid back to back,
    their block-table rows and lengths, the same pools (shared, not copied)."""
    import copy
    reqs = [int(r) for r in reqs]
    out = copy.copy(w)
    out.name = name or f"{w.name}[{len(reqs)} requests]"
    rows = [np.arange(int(w.q_start[r]), int(w.q_end[r])) for r in reqs]
    m = np.array([len(x) for x in rows], np.int64)
    out.q = w.q[np.concatenate(rows)] if rows else w.q[:0]
    out.q_start = np.concatenate([[0], np.cumsum(m)[:-1]]).astype(np.int32)
    out.q_end = (out.q_start + m).astype(np.int32)
    out.kv_len = w.kv_len[reqs].copy()
    out.block_table = w.block_table[reqs].copy()
    out.notes = dict(w.notes)
    out.notes.pop("hot", None)
    return out


def share_runs(w: Workload, runs: Sequence[tuple], name: Optional[str] = None) -> Workload:
    """A copy of ``w`` whose block tables share more pages: for each (src, dsts, p0, p1),
    requests ``dsts`` read request ``src``'s physical pages at logical pages [p0, p1).  Those
    must be full pages of every request involved (no tail page, whose slots past kv_len may
    be poisoned).  Only the tables change; the pools keep every page (pages no table names
    any more stay in them, unread)."""
    import copy
    out = copy.copy(w)
    out.name = name or f"{w.name}/shared-runs"
    bt = w.block_table.copy()
    ps = w.page_size
    for src, dsts, p0, p1 in runs:
        for r in [src] + list(dsts):
            assert p1 * ps <= int(w.kv_len[r]) and (p1 < -(-int(w.kv_len[r]) // ps) or int(w.kv_len[r]) % ps == 0), \
                f"request {r}: pages [{p0}, {p1}) are not all full pages"
        for r in dsts:
            bt[r, p0:p1] = bt[src, p0:p1]
    out.block_table = bt
    out.notes = dict(w.notes)
    out.notes.pop("hot", None)
    return out


STREAM_FOCUS = 5


def _dequant_fp8(codes: np.ndarray, scale: np.ndarray, axis: int) -> np.ndarray:
    """float32 values of e4m3fn codes times their per-vector scales (torch's decoding)."""
    import torch
    x = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    return x * np.expand_dims(scale, axis)


def focus(w: Workload, hot: int = 8, peak: float = 16.0, q_rest: float = 0.25, v_mark: float = 4.0) -> Workload:
    """A companion input to ``w`` on which every (request, query head) attends mostly to a
    few keys spread over its whole context, so that outputs stay O(1) at any kv length and
    a lost, doubled or misplaced key range changes them by much more than the bf16
    tolerance (with N(0,1) inputs an output row averages thousands of keys and shrinks
    like 1/sqrt(kv_len)).

    Query head h = kvh * g + c has colour c and marker dimension d_c = (c * D // g) % D.
    Each request's context [0, kv_len) is cut into hot * g equal segments; segment
    k * g + c holds one hot key of colour c at a seeded position.  A hot key's K element
    d_c becomes ``peak`` and its V element d_c becomes +v_mark or -v_mark (alternating
    with k); every Q row of head h is scaled by ``q_rest`` (a power of two: exact) and its
    element d_c set to ``peak``.  A hot key then scores about peak^2 / sqrt(D) above the
    others, so the softmax weight of the context sits on the visible hot keys.  Keys in
    pages shared by every request (``shared_prefix_pages``) are chosen the same for all of
    them.  Only element values change: shapes, pages, tables and lengths are ``w``'s.
    fp8 workloads re-quantise the vectors that hold a marked element; hashed pools keep the
    marks in ``marks`` / ``mark_values`` (applied on the device and by host_kv_pages).
    The hot positions are in ``notes["hot"][(r, kvh, c)]``.
    """
    import copy
    R, Hq, Hkv, D, ps = w.num_reqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size
    g = Hq // Hkv
    out = copy.copy(w)
    out.notes = dict(w.notes)
    out.name = w.name + "/focus"
    shared_len = w.shared_prefix_pages * ps
    if shared_len:
        assert len(set(int(x) for x in w.kv_len)) == 1, "shared prefix with unequal lengths"
    dcol = [(c * D // g) % D for c in range(g)]
    hot_pos = {}
    k_marks, v_marks, v_vals = [], [], []
    for r in range(R):
        if int(w.q_end[r]) == int(w.q_start[r]):
            continue
        L = int(w.kv_len[r])
        nseg = hot * g
        for kvh in range(Hkv):
            for c in range(g):
                pos = []
                for k in range(hot):
                    seg = k * g + c
                    lo, hi = seg * L // nseg, (seg + 1) * L // nseg
                    if hi <= lo:
                        continue
                    if lo < shared_len:
                        hi = min(hi, shared_len)
                        rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_FOCUS, kvh, c, seg]))
                    else:
                        rng = np.random.default_rng(np.random.SeedSequence([w.seed, STREAM_FOCUS, kvh, c, seg, r + 1]))
                    j = int(rng.integers(lo, hi))
                    pos.append(j)
                    page, slot = int(w.block_table[r, j // ps]), j % ps
                    k_marks.append((page, kvh, slot, dcol[c]))
                    v_marks.append((page, kvh, slot, dcol[c]))
                    v_vals.append(v_mark if k % 2 == 0 else -v_mark)
                hot_pos[(r, kvh, c)] = np.asarray(pos, np.int64)
    out.notes["hot"] = hot_pos
    out.notes["focus"] = dict(hot=hot, peak=peak, q_rest=q_rest, v_mark=v_mark, dcol=dcol)
    km = np.asarray(k_marks, np.int64).reshape(-1, 4)
    vm = np.asarray(v_marks, np.int64).reshape(-1, 4)
    vv = np.asarray(v_vals, np.float32)
    # Q: every row scaled by q_rest, the marker element of each head set to peak
    if w.q.dtype == np.uint16:
        qf = (w.q.astype(np.uint32) << 16).view(np.float32) * np.float32(q_rest)
    else:
        qf = w.q.astype(np.float32) * np.float32(q_rest)
    for h in range(Hq):
        qf[:, h, dcol[h % g]] = peak
    if w.q.dtype == np.uint16:
        out.q = np.empty(w.q.shape, np.uint16)
        f32_to_bf16_bits(np.ascontiguousarray(qf), out.q)
    else:
        out.q = qf.astype(w.q.dtype)
    if w.hashed_kv:
        rows = [np.column_stack([np.full(len(km), STREAM_K), km]), np.column_stack([np.full(len(vm), STREAM_V), vm])]
        vals = [np.full(len(km), peak, np.float32), vv]
        if w.marks is not None:
            rows.insert(0, w.marks)
            vals.insert(0, w.mark_values)
        out.marks = np.concatenate(rows).astype(np.int64)
        out.mark_values = np.concatenate(vals).astype(np.float32)
        return out
    if w.dtype == "fp8":
        k_codes, v_codes = w.k_pool.copy(), w.v_pool.copy()
        k_scale, v_scale = w.k_scale.copy(), w.v_scale.copy()
        # K rows (page, kvh, slot, :) and V columns (page, kvh, :, slot) holding a mark
        for marks, vals, is_k in ((km, np.full(len(km), peak, np.float32), True), (vm, vv, False)):
            if not len(marks):
                continue
            vec = {}
            for (page, kvh, slot, d), val in zip(marks, vals):
                vec.setdefault((int(page), int(kvh), int(slot)), []).append((int(d), float(val)))
            keys = list(vec)
            p_, h_, s_ = (np.asarray(x, np.int64) for x in zip(*keys))
            if is_k:
                x = _dequant_fp8(k_codes[p_, h_, s_, :], k_scale[p_, h_, s_], 1)
            else:
                x = _dequant_fp8(v_codes[p_, h_, :, s_], v_scale[p_, h_, s_], 1)
            for i, key in enumerate(keys):
                for d, val in vec[key]:
                    x[i, d] = val
            codes, sc = quantize_fp8(x.astype(np.float32), axis=1)
            if is_k:
                k_codes[p_, h_, s_, :] = codes
                k_scale[p_, h_, s_] = sc
            else:
                v_codes[p_, h_, :, s_] = codes
                v_scale[p_, h_, s_] = sc
        out.k_pool, out.v_pool, out.k_scale, out.v_scale = k_codes, v_codes, k_scale, v_scale
        return out
    k, v = w.k_pool.copy(), w.v_pool.copy()
    if w.dtype == "bf16":
        kb = np.empty(1, np.uint16)
        f32_to_bf16_bits(np.array([peak], np.float32), kb)
        vb = np.empty(len(vv), np.uint16)
        f32_to_bf16_bits(np.ascontiguousarray(vv), vb)
        kval, vval = kb[0], vb
    else:
        kval, vval = np.float32(peak), vv
    if len(km):
        k[km[:, 0], km[:, 1], km[:, 2], km[:, 3]] = kval
        v[vm[:, 0], vm[:, 1], vm[:, 3], vm[:, 2]] = vval
    out.k_pool, out.v_pool = k, v
    return out


def uniform_lengths(seed: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi] inclusive (stream 0 of the seed)."""
    return _rng(seed, STREAM_LENGTHS).integers(lo, hi, size=n, endpoint=True)


CONFIG_NAMES = {
    1: "tiny-mixed-f32",
    2: "orca-mixed-llama7b",
    3: "decode-heavy-gqa",
    4: "chunked-prefill-mix-gqa8",
    5: "shared-prefix-6",
    51: "shared-prefix-64",
    6: "spec-decode-mtp3",
    7: "spec-decode-mtp7",
    8: "long-context-decode-128k",
    9: "long-prefix-chunk",
}


def config(cid: int, seed: Optional[int] = None, poison_tail: bool = False,
           scale: int = 1, dtype: Optional[str] = None, tp: int = 1, dp: int = 1) -> Workload:
    """The five workloads of the pages (plus 51: the scaled shared-prefix variant; 6 and 7:
    multi-row speculative-decode verify steps with 4 and 8 rows per request).

    ``scale`` > 1 shrinks the lengths (integer division, min 1) and keeps the head
    layout, for parity runs the oracle finishes quickly.  ``dtype`` replaces the
    configuration's element type (e.g. "fp8" for the same shapes in fp8 storage).

    ``tp`` / ``dp`` > 1 give one GPU's share of the iteration when it is split over that
    many GPUs: by head (tensor parallel: num_q_heads / tp query heads and num_kv_heads / tp
    KV heads, at least one KV head, replicated when there are fewer KV heads than GPUs) or
    by request (data parallel: requests r with r % dp == 0).
    """
    s = cid if seed is None else seed

    def mk(name, q_rows, kv_lens, **kw):
        if dtype is not None:
            kw["dtype"] = dtype
        if tp > 1:
            assert kw["num_q_heads"] % tp == 0, "query heads must split evenly"
            kw["num_q_heads"] //= tp
            kw["num_kv_heads"] = max(1, kw["num_kv_heads"] // tp)
            name += f"/tp{tp}"
        if dp > 1:
            q_rows, kv_lens = list(q_rows)[::dp], list(kv_lens)[::dp]
            name += f"/dp{dp}"
        return build(name, q_rows, kv_lens, **kw)

    def sh(x):
        return np.maximum(1, np.asarray(x, np.int64) // scale)

    if cid == 1:
        # A uncached prefill 64/64, B decode 1/100, C chunk 16 rows on S0=32
        return mk(CONFIG_NAMES[1], [64, 1, 16], [64, 100, 48], num_q_heads=4, num_kv_heads=2,
                     head_dim=64, page_size=16, dtype="f32", seed=s, permute_pages=False,
                     poison_tail=poison_tail)
    if cid == 2:
        a = int(sh(4096))
        return mk(CONFIG_NAMES[2], [a, 1, 1], [a, int(sh(1500)), int(sh(1700))], num_q_heads=32,
                     num_kv_heads=32, head_dim=128, page_size=16, seed=s, poison_tail=poison_tail)
    if cid == 3:
        n = max(1, 256 // scale)
        kv = sh(uniform_lengths(s, n, 1024, 8192))
        return mk(CONFIG_NAMES[3], [1] * n, kv, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     page_size=64, seed=s, poison_tail=poison_tail)
    if cid == 4:
        n = max(1, 64 // scale)
        kv = sh(uniform_lengths(s, n, 512, 16384))
        chunk, total = int(sh(2048)), int(sh(32768))
        return mk(CONFIG_NAMES[4], [chunk] + [1] * n, [total] + list(kv), num_q_heads=64,
                     num_kv_heads=8, head_dim=128, page_size=64, seed=s, poison_tail=poison_tail)
    if cid in (5, 51):
        nreq, shared = (6, 4096) if cid == 5 else (64, 16384)
        shared = max(64, (shared // scale) // 64 * 64)
        priv = int(sh(1024))
        return mk(CONFIG_NAMES[cid], [1] * nreq, [shared + priv] * nreq, num_q_heads=32,
                     num_kv_heads=8, head_dim=128, page_size=64, seed=s,
                     shared_prefix_pages=shared // 64, poison_tail=poison_tail)
    if cid in (6, 7):
        # speculative / MTP verify: each request checks k draft tokens plus one, so it has
        # k+1 new rows, causal among themselves (k = 3 or 7); otherwise the decode-heavy shape
        n = max(1, 256 // scale)
        kv = sh(uniform_lengths(s, n, 1024, 8192))
        rows = 4 if cid == 6 else 8
        kv = np.maximum(kv, rows)
        return mk(CONFIG_NAMES[cid], [rows] * n, kv, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  page_size=64, seed=s, poison_tail=poison_tail)
    if cid == 8:
        # 256 decodes at 128K context each, page 64: 256 x 2048 = 524,288 block-table entries
        # ("GLM-5.3 推理全链路(八)", stage 4); the decode-heavy head layout.  K/V (137 GB in
        # bf16) are hashed page values made on the device.
        n = max(1, 256 // scale)
        L = max(64, 131072 // scale)
        return mk(CONFIG_NAMES[8], [1] * n, [L] * n, num_q_heads=32, num_kv_heads=8, head_dim=128,
                  page_size=64, seed=s, hashed_kv=True)
    if cid == 9:
        # chunked prefill of a long prompt with a small chunk budget: a 256-row chunk whose
        # cached prefix is 65,536 positions ("ORCA 和 chunked prefill", section 4: a chunk
        # reads everything before it), batched with 64 decodes as in the chunk mix; the
        # decode-heavy head layout (g = 4)
        n = max(1, 64 // scale)
        kv = sh(uniform_lengths(s, n, 512, 16384))
        chunk, S0 = int(sh(256)), int(sh(65536))
        return mk(CONFIG_NAMES[9], [chunk] + [1] * n, [S0 + chunk] + list(kv), num_q_heads=32, num_kv_heads=8,
                  head_dim=128, page_size=64, seed=s, poison_tail=poison_tail)
    raise ValueError(f"unknown config {cid}")
