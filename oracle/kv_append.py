"""The oracle's definition of writing one iteration's new K/V into the paged pools.

Test infrastructure only (see the package docstring).

Sources, cited by page title and section:

* "ORCA 和 chunked prefill", section 3 (the walk of one block over a chunk): after the
  QKV projection, the layer's K and V of the chunk are appended to the request's cache,
  and attention then reads the whole prefix including them.
* "GLM-5.3 推理全链路(八)", stage 4 (freezing the scheduler's result into GPU inputs):
  out_cache_loc tells, for every new token, the page and the slot it is written to.

Readings where the pages are silent: an out_cache_loc entry is the
flat slot index page * page_size + slot, and a negative entry is padding that writes
nothing; the new token of flat row t of request r is logical position
S0 + (t - q_start[r]) with S0 = kv_len - q_rows (the new rows are the last positions).
Pool layouts are the library's: K pages [page][kv_head][slot][d], V pages transposed
[page][kv_head][d][slot].
"""
from __future__ import annotations

import numpy as np


def slots_for_new_rows(q_start, q_end, kv_len, block_table, page_size: int, total_rows: int) -> np.ndarray:
    """out_cache_loc for the flat rows of one iteration: int64 [total_rows], -1 for rows
    outside every request.  Row q_start[r] + i is position S0 + i of request r, which
    lives in page block_table[r][(S0 + i) // page_size] at slot (S0 + i) % page_size."""
    loc = np.full(total_rows, -1, np.int64)
    for r in range(len(kv_len)):
        qs, qe, L = int(q_start[r]), int(q_end[r]), int(kv_len[r])
        S0 = L - (qe - qs)
        for i in range(qe - qs):
            pos = S0 + i
            page = int(block_table[r][pos // page_size])
            loc[qs + i] = page * page_size + pos % page_size
    return loc


def append_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              out_cache_loc: np.ndarray, page_size: int):
    """Copies of the pools with token t's K and V ([kv_heads, D] each) written at slot
    out_cache_loc[t]; negative entries are skipped.  Values are copied bit for bit."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for t, loc in enumerate(np.asarray(out_cache_loc, np.int64)):
        if loc < 0:
            continue
        page, slot = divmod(int(loc), page_size)
        k_out[page, :, slot, :] = k_new[t]
        v_out[page, :, :, slot] = v_new[t]
    return k_out, v_out
