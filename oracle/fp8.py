"""The oracle's reading of fp8 KV storage with per-token scales.

Test infrastructure only (see the package docstring).

Sources, cited by page title and section:

* "How To Scale Your Model 笔记(7-8)", section 4 (storage format vs compute format):
  compressed values are widened on chip and the arithmetic still runs in the wider
  format; compression cuts the bytes read, not the multiply-add work.
* "GLM-5.3 推理全链路(八)", the section on the two costs outside the 656-byte ledger:
  every token carries FP32 scales stored next to its FP8 data, and a kernel reading
  the cache needs both to dequantise.

Readings where the pages are silent: the FP8 format is OCP
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


# ---- storing new rows in fp8 ----------------------------------------------------------
# Readings where the pages are silent: a new K or V vector of one token and KV head is stored
# with scale = max|x| / 448 (the largest finite e4m3fn magnitude), computed in float32, or 1
# for an all-zero vector; each element's code is x / scale (float32 division) rounded to
# the nearest e4m3fn value, ties to the even code; magnitudes above 448 (reachable only by
# a rounding of the scale) take the largest finite code.

_POS = _TABLE[1:0x7F]                       # the 126 positive finite values, increasing


def e4m3fn_round(y: np.ndarray) -> np.ndarray:
    """uint8 code of the e4m3fn value nearest to each float32 y (ties to the code with an
    even mantissa, i.e. an even code), saturating at +-448; NaN is not accepted."""
    y = np.asarray(y, np.float32)
    assert not np.isnan(y).any()
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    vals = np.concatenate([[0.0], _POS])            # code c has value vals[c], c = 0..126
    hi = np.searchsorted(vals, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """(codes, scales) for float32 vectors along the last axis of x: scale = max|x| / 448
    in float32 (1 for an all-zero vector), code = e4m3fn_round(x / scale)."""
    x = np.asarray(x, np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return e4m3fn_round(x / scale[..., None]), scale


def append_kv_fp8(k_pool, v_pool, k_scale, v_scale, k_new, v_new, out_cache_loc, page_size: int):
    """Copies of the fp8 pools and scale pools with token t's K and V ([kv_heads, D] float32
    values each, e.g. bf16 inputs decoded) quantised per (token, KV head) and written at
    slot out_cache_loc[t] (K row / transposed V column, and the two scales); negative
    entries are skipped."""
    k_out, v_out = k_pool.copy(), v_pool.copy()
    ks_out, vs_out = k_scale.copy(), v_scale.copy()
    kc, ks = quantize_rows(k_new)
    vc, vs = quantize_rows(v_new)
    for t, loc in enumerate(np.asarray(out_cache_loc, np.int64)):
        if loc < 0:
            continue
        page, slot = divmod(int(loc), page_size)
        k_out[page, :, slot, :] = kc[t]
        v_out[page, :, :, slot] = vc[t]
        ks_out[page, :, slot] = ks[t]
        vs_out[page, :, slot] = vs[t]
    return k_out, v_out, ks_out, vs_out
