"""The oracle's reading of fp8 KV storage with per-token scales.

Test infrastructure only (see the package docstring).

Sources, cited by page title and section:

* "How To Scale Your Model 笔记(7-8)", section 4 (storage format vs compute format):
  compressed values are widened on chip and the arithmetic still runs in the wider
  format; compression cuts the bytes read, not the multiply-add work.
* "GLM-5.3 推理全链路(八)", the section on the two costs outside the 656-byte ledger:
  every token carries FP32 scales stored next to its FP8 data, and a kernel reading
  the cache needs both to dequantise.

Readings where the pages are silent (listed in the design doc): the FP8 format is OCP
e4m3fn (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, the
all-ones exponent-and-mantissa codes are NaN, exponent 0 is subnormal); there is one
float32 scale per (page, KV head, slot) for K and one for V, i.e. one per token and
head covering its head_dim values; the stored value of element d of that token is
decode(code) * scale.  Pools keep the library's layouts: K [page][kv_head][slot][d],
V transposed [page][kv_head][d][slot]; scale pools are [page][kv_head][slot].
"""
from __future__ import annotations

import math

import numpy as np


def _decode_code(c: int) -> float:
    """Value of one e4m3fn code from the format's definition:
    (-1)^s * 2^(e-7) * (1 + m/8) for exponent field e in 1..15,
    (-1)^s * 2^-6 * (m/8) for e = 0, NaN for e = 15 with m = 7."""
    s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -mag if s else mag


_TABLE = np.array([_decode_code(c) for c in range(256)], np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact float64 value of each uint8 e4m3fn code (the 256 values decoded one by one,
    then looked up)."""
    return _TABLE[np.asarray(codes, np.uint8)]


def dequantize_pools(k_codes: np.ndarray, k_scale: np.ndarray, v_codes: np.ndarray,
                     v_scale: np.ndarray):
    """float64 K and V pools (same layouts as the code pools) from fp8 codes and their
    per-token scales: K[p,h,s,d] = decode(k)[p,h,s,d] * k_scale[p,h,s] and
    V[p,h,d,s] = decode(v)[p,h,d,s] * v_scale[p,h,s]."""
    K = e4m3fn_to_f64(k_codes) * np.asarray(k_scale, np.float64)[:, :, :, None]
    V = e4m3fn_to_f64(v_codes) * np.asarray(v_scale, np.float64)[:, :, None, :]
    return K, V
