"""Closed-form work and traffic counters (test infrastructure only).

* KV bytes per position: each of L layers stores a K and a V vector of H elements for
  each of its N_KV KV heads, p_kv bytes per element: c_KV = 2·L·N_KV·H·p_kv
  ("How To Scale Your Model 笔记(7-8)", section 3, "KV 容量与 GQA"; the printed formula
  is lost in extraction, this is the reading that reproduces all three figures the
  pages print: 128 KiB, 160 KiB and 512 KB).
* Visible pairs of a request with S0 cached and m new rows: every row sees the S0
  cached positions plus its own block up to the diagonal, m·S0 + m(m+1)/2
  ("How To Scale Your Model 笔记(7-8)", section 2, cumulative-work paragraph).
* FLOPs: 2·H for q·k plus 2·H for the weighted sum of V, per visible pair and query
  head, i.e. 4·H per pair ("ORCA 和 chunked prefill", section 3 cost model;
  "How To Scale Your Model 笔记(7-8)", section 2: about 4·S·H per query head reading S
  sources).
* Quantised storage: with p_kv = 1 byte (fp8) every stored vector also carries its
  float32 scale, so each of the 2·L·N_KV vectors of a position takes H·p_kv + s bytes
  ("GLM-5.3 推理全链路(八)": the indexer cache holds 128 FP8 bytes plus a 4-byte
  scale per token and layer, 132 bytes; and the scales of the main KV are read along
  with its data).
* Logical vs physical KV bytes: logical counts every request's positions; physical
  counts each distinct (page, slot) once ("How To Scale Your Model 笔记(7-8)",
  section 3, shared-prefix example).
"""
from __future__ import annotations

import numpy as np


def kv_bytes_per_position(layers: int, kv_heads: int, head_dim: int, elem_bytes: int,
                          scale_bytes: int = 0) -> int:
    return 2 * layers * kv_heads * (head_dim * elem_bytes + scale_bytes)


def visible_pairs(q_rows, kv_len) -> int:
    """Σ over requests of m·S0 + m(m+1)/2 with S0 = kv_len − m."""
    m = np.asarray(q_rows, np.int64)
    L = np.asarray(kv_len, np.int64)
    S0 = L - m
    return int(np.sum(m * S0 + m * (m + 1) // 2))


def attention_flops(q_rows, kv_len, num_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * num_q_heads * visible_pairs(q_rows, kv_len)


def logical_kv_bytes(kv_len, kv_heads: int, head_dim: int, elem_bytes: int, layers: int = 1,
                     scale_bytes: int = 0) -> int:
    return int(np.sum(np.asarray(kv_len, np.int64))) * kv_bytes_per_position(layers, kv_heads, head_dim,
                                                                              elem_bytes, scale_bytes)


def physical_kv_bytes(block_table, kv_len, page_size: int, kv_heads: int, head_dim: int,
                      elem_bytes: int, layers: int = 1, scale_bytes: int = 0) -> int:
    """Bytes of the distinct (physical page, slot) positions the requests read."""
    seen = set()
    for r, L in enumerate(np.asarray(kv_len, np.int64)):
        L = int(L)
        full, tail = divmod(L, page_size)
        row = np.asarray(block_table[r])
        for p in range(full):
            seen.update((int(row[p]), s) for s in range(page_size))
        if tail:
            seen.update((int(row[full]), s) for s in range(tail))
    return len(seen) * kv_bytes_per_position(layers, kv_heads, head_dim, elem_bytes, scale_bytes)
