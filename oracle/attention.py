"""The oracle's definition of varlen paged attention (fp64, materialised scores).

Test infrastructure only (see the package docstring).

Sources, cited by page title and section:

* "一次 forward 怎么塞下很多个 request", section 6 (Attention) and 6.2: a request's
  output row is softmax(q·Kᵀ/√d_head + mask)·V over that request's own keys only;
  requests are walked one at a time over a flat Q tensor.
* "ORCA 和 chunked prefill", section 2: each request gives (q_start, q_end, kv_length);
  q_rows = q_end − q_start new rows, kv_length = the whole context after this
  iteration's K/V were appended.  Section 4: the chunk's rows see the cached prefix
  in full and their own block lower-triangularly.
* "How To Scale Your Model 笔记(7-8)", section 2: with S0 cached and m new positions the
  mask is 0 or −inf; the first S0 columns are visible to every new row; in the last m
  columns only the strict upper triangle is masked.  Section 3 ("KV 容量与 GQA"): a
  group of g query heads shares one KV head, each query head computing its own
  weights.  Section 3 (paging): a block table maps logical positions to physical
  blocks; paging changes placement, not the result.

Readings where the pages are silent:
  scale = 1/sqrt(head_dim) unless given; query head h uses KV head h // g;
  the new rows' own K/V are the last q_rows logical positions (S0 = kv_len − q_rows);
  logical position j lives in page block_table[r][j // page_size], slot j % page_size;
  V pages are stored transposed ([head_dim, page_size]).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterable, Optional, Sequence

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Decode an input array: uint16 = bf16 bit patterns, otherwise a float array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def visibility_mask(S0: int, m: int) -> np.ndarray:
    """Boolean [m, S0+m]: True where new row i may read source column j.

    The first S0 columns (the cache) are visible to every new row; among the last m
    columns (the new block) only the strict upper triangle is hidden, i.e. row i sees
    column S0 + t exactly when t <= i ("How To Scale Your Model 笔记(7-8)", section 2;
    "ORCA 和 chunked prefill", section 4).
    """
    mask = np.zeros((m, S0 + m), dtype=bool)
    mask[:, :S0] = True
    mask[:, S0:] = np.tril(np.ones((m, m), dtype=bool))
    return mask


def gather_kv(k_pool: np.ndarray, v_pool: np.ndarray, block_table_row: np.ndarray,
              kv_len: int, kv_head: int, page_size: int):
    """K, V of one request and one KV head in logical order, as float64 [kv_len, D].

    Logical position j sits in physical page block_table_row[j // page_size] at slot
    j % page_size ("How To Scale Your Model 笔记(7-8)", section 3, paging).  K pages are
    [page_size, D]; V pages are stored transposed, [D, page_size].
    """
    j = np.arange(kv_len)
    pages = np.asarray(block_table_row)[j // page_size].astype(np.int64)
    slots = j % page_size
    K = to_f64(k_pool[pages, kv_head, slots, :])
    V = to_f64(v_pool[pages, kv_head, :, slots])      # fancy index on axes 0,1,3 -> [kv_len, D]
    return K, V


def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, S0: int, scale: float,
           row_ids: Optional[np.ndarray] = None) -> np.ndarray:
    """Masked softmax attention for one request and one query head, fp64.

    q_rows: [n, D] (the new rows, or the subset ``row_ids`` of them);
    K, V: [S0+m, D].  Materialises the [n, S0+m] score matrix, adds the 0/−inf mask,
    takes the row softmax (subtract row max, exponentiate, divide by the row sum) and
    multiplies by V.
    """
    kv_len = K.shape[0]
    m = kv_len - S0
    if row_ids is None:
        row_ids = np.arange(m)
    S = (q_rows @ K.T) * scale
    full = visibility_mask(S0, m)[row_ids]
    S = np.where(full, S, -np.inf)
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=1, keepdims=True)
    return P @ V


def _default_scale(head_dim: int, softmax_scale: Optional[float]) -> float:
    if softmax_scale is None or softmax_scale <= 0:
        return 1.0 / math.sqrt(head_dim)
    return float(softmax_scale)


def attention_rows(q, k_pool, v_pool, block_table, q_start, q_end, kv_len, page_size: int,
                   req: int, rows: Optional[Sequence[int]] = None,
                   heads: Optional[Iterable[int]] = None, softmax_scale: Optional[float] = None):
    """Oracle output of request ``req`` for the given local rows and query heads.

    Returns {head: [len(rows), D] float64}.  Rows are indices within the request
    (0..q_rows-1).
    """
    Hq = q.shape[1]
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    D = q.shape[2]
    scale = _default_scale(D, softmax_scale)
    qs, qe, L = int(q_start[req]), int(q_end[req]), int(kv_len[req])
    m = qe - qs
    S0 = L - m
    rows = np.arange(m) if rows is None else np.asarray(rows, np.int64)
    heads = range(Hq) if heads is None else list(heads)
    out = {}
    cache = {}
    for h in heads:
        kvh = h // g
        if kvh not in cache:
            cache[kvh] = gather_kv(k_pool, v_pool, block_table[req], L, kvh, page_size)
        K, V = cache[kvh]
        Q = to_f64(q[qs + rows, h, :])
        out[h] = attend(Q, K, V, S0, scale, rows)
    return out


def varlen_paged_attention(q, k_pool, v_pool, block_table, q_start, q_end, kv_len, page_size: int,
                           softmax_scale: Optional[float] = None, threads: Optional[int] = None):
    """Full oracle: float64 [total_q_rows, Hq, D]; rows outside every request stay 0.

    Works request by request ("一次 forward 怎么塞下很多个 request", section 6.2), one
    query head at a time; the (request, KV head) pairs run on a thread pool (NumPy
    releases the GIL inside BLAS and ufuncs).
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    g = Hq // Hkv
    out = np.zeros((T, Hq, D), np.float64)
    jobs = [(r, kvh) for r in range(len(kv_len)) for kvh in range(Hkv)
            if int(q_end[r]) > int(q_start[r])]

    def job(rk):
        r, kvh = rk
        res = attention_rows(q, k_pool, v_pool, block_table, q_start, q_end, kv_len, page_size,
                             r, None, range(kvh * g, (kvh + 1) * g), softmax_scale)
        qs, qe = int(q_start[r]), int(q_end[r])
        for h, o in res.items():
            out[qs:qe, h, :] = o

    nthreads = threads or max(1, min(16, os.cpu_count() or 1))
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1 if nthreads > 1 else None):
        if nthreads == 1 or len(jobs) <= 1:
            for jb in jobs:
                job(jb)
        else:
            with ThreadPoolExecutor(nthreads) as ex:
                list(ex.map(job, jobs))
    return out
