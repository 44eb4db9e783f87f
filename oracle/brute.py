"""Scalar brute-force varlen paged attention (pure Python, tiny inputs only).

Test infrastructure only.  An independent second writing of the same definition
("一次 forward 怎么塞下很多个 request", section 6.2 loop over requests;
"How To Scale Your Model 笔记(7-8)", section 2 mask) with no NumPy arithmetic: every
score, exponential and sum is a Python float operation, so it shares no vectorised
code path with ``oracle.attention``.
"""
from __future__ import annotations

import math
import struct


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _val(x) -> float:
    # uint16 inputs are bf16 bit patterns; anything else is a number
    if hasattr(x, "dtype") and str(x.dtype) == "uint16":
        return _bf16(int(x))
    return float(x)


def brute_force_attention(q, k_pool, v_pool, block_table, q_start, q_end, kv_len, page_size,
                          softmax_scale=None):
    """Returns nested lists out[t][h][d] (rows not in any request stay 0.0)."""
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    scale = (1.0 / math.sqrt(D)) if (softmax_scale is None or softmax_scale <= 0) else softmax_scale
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for r in range(len(kv_len)):
        qs, qe, L = int(q_start[r]), int(q_end[r]), int(kv_len[r])
        m = qe - qs
        S0 = L - m
        for h in range(Hq):
            kvh = h // g
            for i in range(m):
                t = qs + i
                last = S0 + i                    # highest visible source position
                scores = []
                for j in range(last + 1):
                    page = int(block_table[r][j // page_size])
                    slot = j % page_size
                    s = 0.0
                    for d in range(D):
                        s += _val(q[t, h, d]) * _val(k_pool[page, kvh, slot, d])
                    scores.append(s * scale)
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for d in range(D):
                    acc = 0.0
                    for j in range(last + 1):
                        page = int(block_table[r][j // page_size])
                        slot = j % page_size
                        acc += w[j] * _val(v_pool[page, kvh, d, slot])
                    out[t][h][d] = acc / tot
    return out
