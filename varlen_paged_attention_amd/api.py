"""ctypes binding over the C ABI in include/varlen_attn.h (argument marshalling only).

Every function here has the name of the C entry point it calls.  Tensors are PyTorch
tensors on the GPU (only their data pointers cross the boundary); metadata arrays are
host numpy int32 arrays.  There is no fallback: if ``libvarlen_attn.so`` has not been
built the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

VA_OK, VA_ERR_INVALID_ARG, VA_ERR_UNSUPPORTED, VA_ERR_OUT_OF_MEMORY, VA_ERR_HIP, VA_ERR_WORKSPACE_TOO_SMALL = \
    0, -1, -2, -3, -4, -5
VA_DTYPE_BF16, VA_DTYPE_F32, VA_DTYPE_FP8_E4M3 = 0, 1, 2
DTYPE_CODES = {"bf16": VA_DTYPE_BF16, "f32": VA_DTYPE_F32, "fp8": VA_DTYPE_FP8_E4M3}
VA_FLAG_SHARED_PREFIX, VA_FLAG_NO_PREFILL_KERNEL, VA_FLAG_HOST_ONLY = 1, 2, 4
VA_FLAG_NO_DECODE_TILES = 1 << 3

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvarlen_attn.so")
EXPORTED = ["varlen_attn_plan", "varlen_attn_run", "varlen_attn_run_events", "varlen_attn_plan_stats", "varlen_attn_plan_export",
            "varlen_attn_debug_gather", "varlen_attn_plan_destroy", "varlen_attn_status_string",
            "varlen_attn_last_error", "varlen_attn_append_kv", "varlen_attn_plan_slots", "varlen_attn_run_fp8",
            "varlen_attn_debug_fp8_to_bf16", "varlen_attn_append_kv_fp8", "varlen_attn_debug_stream_read",
            "varlen_attn_run_noalloc", "varlen_attn_debug_stage_gather"]
VA_STATIC_SCRATCH_BYTES = 64 << 20


class VaParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_req", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("prefill_min_rows", ctypes.c_int32), ("split_len", ctypes.c_int32),
                ("prefill_split_len", ctypes.c_int32)]


class VaPlanStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("num_reqs", "total_q_rows", "prefill_tiles", "split_items",
                                              "shared_items", "shared_groups", "partial_slots",
                                              "combine_rows", "visible_pairs")] + \
               [("flops", ctypes.c_double)] + \
               [(n, ctypes.c_int64) for n in ("logical_kv_bytes", "physical_kv_bytes", "q_bytes", "o_bytes",
                                              "table_bytes", "workspace_bytes")] + \
               [("plan_host_us", ctypes.c_double), ("prefill_flops", ctypes.c_double),
                ("split_flops", ctypes.c_double)] + \
               [(n, ctypes.c_int64) for n in ("prefill_kv_bytes", "split_kv_bytes", "split_q_bytes",
                                              "direct_items", "shared_tiles")] + \
               [("shared_tile_flops", ctypes.c_double), ("split_item_kv_bytes", ctypes.c_int64),
                ("prefill_split_tiles", ctypes.c_int64), ("split_item_flops", ctypes.c_double)]


class VarlenAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libvarlen_attn.so (after torch, so both use the one HIP runtime in the process)."""
    global _lib
    if _lib is None:
        try:
            import torch  # noqa: F401  (loads torch's libamdhip64 first; ours binds to it by soname)
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(python -m varlen_paged_attention_amd.build_lib)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.varlen_attn_plan.argtypes = [ctypes.POINTER(VaParams), ctypes.c_int32, i32p, i32p, i32p, i32p,
                                       ctypes.POINTER(P), ctypes.POINTER(ctypes.c_size_t)]
        L.varlen_attn_plan.restype = ctypes.c_int
        L.varlen_attn_run.argtypes = [P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.varlen_attn_run.restype = ctypes.c_int
        L.varlen_attn_run_noalloc.argtypes = [P, P, P, P, P, P, P]
        L.varlen_attn_run_noalloc.restype = ctypes.c_int
        L.varlen_attn_run_events.argtypes = [P, P, P, P, P, P, P, ctypes.c_size_t, P, ctypes.POINTER(P)]
        L.varlen_attn_run_events.restype = ctypes.c_int
        L.varlen_attn_run_fp8.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, ctypes.POINTER(P)]
        L.varlen_attn_run_fp8.restype = ctypes.c_int
        L.varlen_attn_debug_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
        L.varlen_attn_debug_stream_read.restype = ctypes.c_int
        L.varlen_attn_debug_fp8_to_bf16.argtypes = [P, P, ctypes.c_int64, P]
        L.varlen_attn_debug_fp8_to_bf16.restype = ctypes.c_int
        L.varlen_attn_append_kv_fp8.argtypes = [ctypes.POINTER(VaParams), ctypes.c_int64, P, P, P, P, P, P, P, P, P]
        L.varlen_attn_append_kv_fp8.restype = ctypes.c_int
        L.varlen_attn_plan_stats.argtypes = [P, ctypes.POINTER(VaPlanStats)]
        L.varlen_attn_plan_stats.restype = ctypes.c_int
        L.varlen_attn_plan_export.argtypes = [P, ctypes.c_int32, ctypes.POINTER(i32p),
                                              ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
        L.varlen_attn_plan_export.restype = ctypes.c_int
        L.varlen_attn_debug_gather.argtypes = [P, P, P, P, P, P, P]
        L.varlen_attn_debug_gather.restype = ctypes.c_int
        L.varlen_attn_debug_stage_gather.argtypes = [P, P, P, P, P, P, P]
        L.varlen_attn_debug_stage_gather.restype = ctypes.c_int
        L.varlen_attn_append_kv.argtypes = [ctypes.POINTER(VaParams), ctypes.c_int64, P, P, P, P, P, P, P]
        L.varlen_attn_append_kv.restype = ctypes.c_int
        L.varlen_attn_plan_slots.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
        L.varlen_attn_plan_slots.restype = ctypes.c_int
        L.varlen_attn_plan_destroy.argtypes = [P]
        L.varlen_attn_plan_destroy.restype = None
        L.varlen_attn_status_string.argtypes = [ctypes.c_int]
        L.varlen_attn_status_string.restype = ctypes.c_char_p
        L.varlen_attn_last_error.argtypes = []
        L.varlen_attn_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != VA_OK:
        L = lib()
        raise VarlenAttnError(status, f"{L.varlen_attn_status_string(status).decode()}: "
                                      f"{L.varlen_attn_last_error().decode()}")


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr32(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class Plan:
    """Owns a va_plan handle (destroyed with the object), with the sizes its buffers must
    have: num_reqs, total_q_rows (rows q and out must hold) and kv_total (sum of kv_len)."""

    def __init__(self, handle: ctypes.c_void_p, workspace_bytes: int, params: VaParams, num_reqs: int = 0,
                 total_q_rows: int = 0, kv_total: int = 0):
        self.handle = handle
        self.workspace_bytes = int(workspace_bytes)
        self.params = params
        self.num_reqs = int(num_reqs)
        self.total_q_rows = int(total_q_rows)
        self.kv_total = int(kv_total)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.varlen_attn_plan_destroy(h)
            self.handle = None


def varlen_attn_plan(*, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int,
                     q_start, q_end, kv_len, block_table, dtype: str = "bf16", softmax_scale: float = 0.0,
                     flags: int = 0, prefill_min_rows: int = 0, split_len: int = 0,
                     prefill_split_len: int = 0) -> Plan:
    qs, qe, kv = _i32(q_start), _i32(q_end), _i32(kv_len)
    bt = _i32(block_table)
    if bt.ndim != 2 or not (len(qs) == len(qe) == len(kv) == bt.shape[0]):
        raise ValueError("q_start/q_end/kv_len must be [R] and block_table [R, max_pages]")
    p = VaParams(num_q_heads, num_kv_heads, head_dim, page_size, num_pages, bt.shape[1],
                 DTYPE_CODES[dtype], softmax_scale, flags, prefill_min_rows, split_len, prefill_split_len)
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check(lib().varlen_attn_plan(ctypes.byref(p), len(kv), _ptr32(qs), _ptr32(qe), _ptr32(kv), _ptr32(bt),
                                  ctypes.byref(h), ctypes.byref(ws)))
    live = qe > qs
    return Plan(h, ws.value, p, num_reqs=len(kv), total_q_rows=int(qe[live].max()) if live.any() else 0,
                kv_total=int(kv.astype(np.int64).sum()))


def plan_for(w, flags: int = 0, **kw) -> Plan:
    """Plan for a ``workloads.Workload``."""
    return varlen_attn_plan(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                            page_size=w.page_size, num_pages=w.num_pages, q_start=w.q_start, q_end=w.q_end,
                            kv_len=w.kv_len, block_table=w.block_table, dtype=w.dtype,
                            softmax_scale=w.softmax_scale, flags=flags, **kw)


def varlen_attn_plan_stats(plan: Plan) -> dict:
    st = VaPlanStats()
    _check(lib().varlen_attn_plan_stats(plan.handle, ctypes.byref(st)))
    return {n: getattr(st, n) for n, _ in VaPlanStats._fields_}


def varlen_attn_plan_export(plan: Plan, which: int) -> np.ndarray:
    data = ctypes.POINTER(ctypes.c_int32)()
    count = ctypes.c_int64()
    width = ctypes.c_int32()
    _check(lib().varlen_attn_plan_export(plan.handle, which, ctypes.byref(data), ctypes.byref(count),
                                         ctypes.byref(width)))
    n = count.value * width.value
    if n == 0:
        return np.zeros((0, width.value), np.int32)
    return np.ctypeslib.as_array(data, shape=(n,)).reshape(count.value, width.value).copy()


def _dev_ptr(t, name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name: str, shape):
    """Raise unless tensor t has exactly ``shape`` (a dimension given as (n, None) needs at
    least n)."""
    got = tuple(t.shape)
    ok = len(got) == len(shape)
    if ok:
        for g, want in zip(got, shape):
            ok = ok and (g >= want[0] if isinstance(want, tuple) else g == want)
    if not ok:
        desc = ", ".join(f">={x[0]}" if isinstance(x, tuple) else str(x) for x in shape)
        raise ValueError(f"{name} has shape {list(got)}, the plan needs [{desc}]")


def _check_run_buffers(plan: "Plan", q, k_pool, v_pool, block_table_dev, out, workspace, k_scale=None,
                       v_scale=None):
    """Shapes of a run's buffers against the plan, checked on the host before any kernel
    reads or writes them (the library itself checks pointers and the workspace size,
    returning VA_ERR_WORKSPACE_TOO_SMALL)."""
    p = plan.params
    Hq, Hkv, D, ps, P = p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size, p.num_pages
    for name, t in (("q", q), ("out", out)):
        if t is not None:
            _need(t, name, ((plan.total_q_rows, None), Hq, D))
    if k_pool is not None:
        _need(k_pool, "k_pool", (P, Hkv, ps, D))
    if v_pool is not None:
        _need(v_pool, "v_pool", (P, Hkv, D, ps))
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        if t is not None:
            _need(t, name, (P, Hkv, ps))
    if block_table_dev is not None and block_table_dev.numel() < plan.num_reqs * p.max_pages_per_req:
        raise ValueError(f"block_table_dev has {block_table_dev.numel()} entries, the plan needs "
                         f"{plan.num_reqs} x {p.max_pages_per_req}")


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _elem_dtype(plan: Plan):
    """torch dtype of q and out."""
    import torch
    return torch.float32 if plan.params.dtype == VA_DTYPE_F32 else torch.bfloat16


def _pool_dtype(plan: Plan):
    """torch dtype of the K/V pools (fp8 codes travel as uint8)."""
    import torch
    return torch.uint8 if plan.params.dtype == VA_DTYPE_FP8_E4M3 else _elem_dtype(plan)


def varlen_attn_run(plan: Plan, q, k_pool, v_pool, block_table_dev, out, workspace=None, stream=None) -> None:
    import torch
    dt = _elem_dtype(plan)
    _check_run_buffers(plan, q, k_pool, v_pool, block_table_dev, out, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().varlen_attn_run(plan.handle, _dev_ptr(q, "q", dt), _dev_ptr(k_pool, "k_pool", dt),
                                 _dev_ptr(v_pool, "v_pool", dt), _dev_ptr(block_table_dev, "block_table", torch.int32),
                                 _dev_ptr(out, "out", dt), _dev_ptr(workspace, "workspace"), ws_bytes,
                                 _stream_ptr(stream)))


def varlen_attn_run_noalloc(plan: Plan, q, k_pool, v_pool, block_table_dev, out, stream=None) -> None:
    """varlen_attn_run with the library's static device scratch as the workspace (nothing is
    allocated; plans needing more than VA_STATIC_SCRATCH_BYTES are refused; calls that
    overlap on one device race on the scratch)."""
    import torch
    dt = _elem_dtype(plan)
    _check_run_buffers(plan, q, k_pool, v_pool, block_table_dev, out, None)
    _check(lib().varlen_attn_run_noalloc(plan.handle, _dev_ptr(q, "q", dt), _dev_ptr(k_pool, "k_pool", dt),
                                         _dev_ptr(v_pool, "v_pool", dt),
                                         _dev_ptr(block_table_dev, "block_table", torch.int32),
                                         _dev_ptr(out, "out", dt), _stream_ptr(stream)))


VA_RUN_EVENTS = 4


def varlen_attn_run_events(plan: Plan, q, k_pool, v_pool, block_table_dev, out, workspace, events,
                           stream=None) -> None:
    """``events``: VA_RUN_EVENTS torch.cuda.Event(enable_timing=True) objects."""
    import torch
    if len(events) != VA_RUN_EVENTS:
        raise ValueError(f"need {VA_RUN_EVENTS} events")
    _check_run_buffers(plan, q, k_pool, v_pool, block_table_dev, out, workspace)
    s = torch.cuda.current_stream() if stream is None else stream
    handles = []
    for ev in events:
        if ev.cuda_event == 0:        # torch creates the event on its first record
            ev.record(s)
        handles.append(ev.cuda_event)
    arr = (ctypes.c_void_p * VA_RUN_EVENTS)(*handles)
    dt = _elem_dtype(plan)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().varlen_attn_run_events(plan.handle, _dev_ptr(q, "q", dt), _dev_ptr(k_pool, "k_pool", dt),
                                        _dev_ptr(v_pool, "v_pool", dt),
                                        _dev_ptr(block_table_dev, "block_table", torch.int32),
                                        _dev_ptr(out, "out", dt), _dev_ptr(workspace, "workspace"), ws_bytes,
                                        ctypes.c_void_p(s.cuda_stream), arr))


def varlen_attn_run_fp8(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table_dev, out, workspace=None,
                        stream=None, events=None) -> None:
    """Run an fp8 plan: k_pool/v_pool uint8 e4m3fn codes, k_scale/v_scale float32
    [num_pages, Hkv, page_size], q/out bf16.  ``events``: None or VA_RUN_EVENTS
    torch.cuda.Event(enable_timing=True) objects."""
    import torch
    _check_run_buffers(plan, q, k_pool, v_pool, block_table_dev, out, workspace, k_scale, v_scale)
    s = torch.cuda.current_stream() if stream is None else stream
    arr = None
    if events is not None:
        if len(events) != VA_RUN_EVENTS:
            raise ValueError(f"need {VA_RUN_EVENTS} events")
        for ev in events:
            if ev.cuda_event == 0:
                ev.record(s)
        arr = (ctypes.c_void_p * VA_RUN_EVENTS)(*[ev.cuda_event for ev in events])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().varlen_attn_run_fp8(plan.handle, _dev_ptr(q, "q", torch.bfloat16),
                                     _dev_ptr(k_pool, "k_pool", torch.uint8), _dev_ptr(v_pool, "v_pool", torch.uint8),
                                     _dev_ptr(k_scale, "k_scale", torch.float32),
                                     _dev_ptr(v_scale, "v_scale", torch.float32),
                                     _dev_ptr(block_table_dev, "block_table", torch.int32),
                                     _dev_ptr(out, "out", torch.bfloat16), _dev_ptr(workspace, "workspace"), ws_bytes,
                                     ctypes.c_void_p(s.cuda_stream), arr))


def varlen_attn_debug_fp8_to_bf16(codes, out, stream=None) -> None:
    """Widen uint8 e4m3fn codes (GPU tensor, numel % 8 == 0) into ``out`` (bf16 or int16
    GPU tensor of the same numel) with the attention kernel's converter."""
    import torch
    if out.numel() != codes.numel():
        raise ValueError("out must have as many elements as codes")
    if out.element_size() != 2:
        raise ValueError("out must hold 2-byte elements")
    _check(lib().varlen_attn_debug_fp8_to_bf16(_dev_ptr(codes, "codes", torch.uint8), _dev_ptr(out, "out"),
                                               codes.numel(), _stream_ptr(stream)))


def varlen_attn_debug_stream_read(buf, sink, stream=None) -> None:
    """Read every byte of the GPU tensor ``buf`` once (HBM read-rate measurement); ``sink``
    is a GPU int32 tensor of at least one element."""
    _check(lib().varlen_attn_debug_stream_read(_dev_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                               _dev_ptr(sink, "sink"), _stream_ptr(stream)))


def varlen_attn_debug_gather(plan: Plan, k_pool, v_pool, block_table_dev, k_out, v_out, stream=None) -> None:
    import torch
    dt = _pool_dtype(plan)
    _check_run_buffers(plan, None, k_pool, v_pool, block_table_dev, None, None)
    p = plan.params
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        _need(t, name, (plan.kv_total, p.num_kv_heads, p.head_dim))
    _check(lib().varlen_attn_debug_gather(plan.handle, _dev_ptr(k_pool, "k_pool", dt), _dev_ptr(v_pool, "v_pool", dt),
                                          _dev_ptr(block_table_dev, "block_table", torch.int32),
                                          _dev_ptr(k_out, "k_out", dt), _dev_ptr(v_out, "v_out", dt),
                                          _stream_ptr(stream)))


def varlen_attn_debug_stage_gather(plan: Plan, k_pool, v_pool, block_table_dev, k_out, v_out, stream=None) -> None:
    """varlen_attn_debug_gather made by the attention kernel's own LDS staging (bf16 plans)."""
    import torch
    dt = _pool_dtype(plan)
    _check_run_buffers(plan, None, k_pool, v_pool, block_table_dev, None, None)
    p = plan.params
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        _need(t, name, (plan.kv_total, p.num_kv_heads, p.head_dim))
    _check(lib().varlen_attn_debug_stage_gather(plan.handle, _dev_ptr(k_pool, "k_pool", dt),
                                                _dev_ptr(v_pool, "v_pool", dt),
                                                _dev_ptr(block_table_dev, "block_table", torch.int32),
                                                _dev_ptr(k_out, "k_out", dt), _dev_ptr(v_out, "v_out", dt),
                                                _stream_ptr(stream)))


def varlen_attn_plan_slots(plan: Plan) -> np.ndarray:
    """out_cache_loc of the planned iteration: int64 [total_q_rows], -1 outside requests."""
    n = int(varlen_attn_plan_stats(plan)["total_q_rows"])
    out = np.empty(n, np.int64)
    _check(lib().varlen_attn_plan_slots(plan.handle, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
    return out


def varlen_attn_append_kv(*, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int, k_new, v_new,
                          out_cache_loc, k_pool, v_pool, bad_loc_count=None, dtype: str = "bf16", stream=None) -> None:
    """Write k_new/v_new ([T, Hkv, D] GPU tensors) into the pools at out_cache_loc (int64 [T] GPU
    tensor); bad_loc_count: optional int32 [1] GPU tensor counting out-of-range entries."""
    import torch
    dt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[dtype]
    p = VaParams(0, num_kv_heads, head_dim, page_size, num_pages, 0, DTYPE_CODES[dtype], 0.0, 0, 0, 0)
    T = int(out_cache_loc.numel())
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (T, num_kv_heads, head_dim):
            raise ValueError(f"{name} must be [{T}, {num_kv_heads}, {head_dim}]")
    _need(k_pool, "k_pool", (num_pages, num_kv_heads, page_size, head_dim))
    _need(v_pool, "v_pool", (num_pages, num_kv_heads, head_dim, page_size))
    _check(lib().varlen_attn_append_kv(ctypes.byref(p), T, _dev_ptr(k_new, "k_new", dt), _dev_ptr(v_new, "v_new", dt),
                                       _dev_ptr(out_cache_loc, "out_cache_loc", torch.int64),
                                       _dev_ptr(k_pool, "k_pool", dt), _dev_ptr(v_pool, "v_pool", dt),
                                       _dev_ptr(bad_loc_count, "bad_loc_count", torch.int32), _stream_ptr(stream)))


def varlen_attn_append_kv_fp8(*, num_kv_heads: int, head_dim: int, page_size: int, num_pages: int, k_new, v_new,
                              out_cache_loc, k_pool, v_pool, k_scale, v_scale, bad_loc_count=None,
                              stream=None) -> None:
    """Quantise k_new/v_new (bf16 [T, Hkv, D] GPU tensors) per (token, KV head) and write codes
    into the uint8 pools and scales into the float32 scale pools at out_cache_loc."""
    import torch
    p = VaParams(0, num_kv_heads, head_dim, page_size, num_pages, 0, VA_DTYPE_FP8_E4M3, 0.0, 0, 0, 0)
    T = int(out_cache_loc.numel())
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (T, num_kv_heads, head_dim):
            raise ValueError(f"{name} must be [{T}, {num_kv_heads}, {head_dim}]")
    _need(k_pool, "k_pool", (num_pages, num_kv_heads, page_size, head_dim))
    _need(v_pool, "v_pool", (num_pages, num_kv_heads, head_dim, page_size))
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, (num_pages, num_kv_heads, page_size))
    _check(lib().varlen_attn_append_kv_fp8(
        ctypes.byref(p), T, _dev_ptr(k_new, "k_new", torch.bfloat16), _dev_ptr(v_new, "v_new", torch.bfloat16),
        _dev_ptr(out_cache_loc, "out_cache_loc", torch.int64), _dev_ptr(k_pool, "k_pool", torch.uint8),
        _dev_ptr(v_pool, "v_pool", torch.uint8), _dev_ptr(k_scale, "k_scale", torch.float32),
        _dev_ptr(v_scale, "v_scale", torch.float32), _dev_ptr(bad_loc_count, "bad_loc_count", torch.int32),
        _stream_ptr(stream)))


def new_workspace(plan: Plan, device="cuda"):
    import torch
    return torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device=device)


def to_device(w, device="cuda"):
    """Move a workload's arrays to the GPU: (q, k_pool, v_pool, block_table) torch tensors."""
    import torch

    def conv(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        return t.to(device)

    bt = torch.from_numpy(_i32(w.block_table)).to(device)
    if getattr(w, "hashed_kv", False):          # pools made on the device from the page hash
        from .workloads import hashed_pools_device
        k, v = hashed_pools_device(w, device)
        return conv(w.q), k, v, bt
    return conv(w.q), conv(w.k_pool), conv(w.v_pool), bt


def scales_to_device(w, device="cuda"):
    """An fp8 workload's (k_scale, v_scale) as float32 GPU tensors."""
    import torch
    return (torch.from_numpy(np.ascontiguousarray(w.k_scale, np.float32)).to(device),
            torch.from_numpy(np.ascontiguousarray(w.v_scale, np.float32)).to(device))


def run_workload(w, flags: int = 0, plan: Optional[Plan] = None, device="cuda", **kw):
    """Plan + run one workload; returns (out tensor, plan)."""
    import torch
    plan = plan or plan_for(w, flags, **kw)
    q, k, v, bt = to_device(w, device)
    out = torch.zeros_like(q)
    ws = new_workspace(plan, device)
    if plan.params.dtype == VA_DTYPE_FP8_E4M3:
        ks, vs = scales_to_device(w, device)
        varlen_attn_run_fp8(plan, q, k, v, ks, vs, bt, out, ws)
    else:
        varlen_attn_run(plan, q, k, v, bt, out, ws)
    torch.cuda.synchronize()
    return out, plan


class RunCall:
    """``varlen_attn_run`` with its arguments marshalled once, for launch loops where the
    per-call ctypes conversion would cost more than the GPU work (same checks as
    ``varlen_attn_run`` at construction)."""

    def __init__(self, plan: Plan, q, k_pool, v_pool, block_table_dev, out, workspace=None, stream=None,
                 k_scale=None, v_scale=None):
        import torch
        dt, pdt = _elem_dtype(plan), _pool_dtype(plan)
        self._fp8 = plan.params.dtype == VA_DTYPE_FP8_E4M3
        _check_run_buffers(plan, q, k_pool, v_pool, block_table_dev, out, workspace,
                           k_scale if self._fp8 else None, v_scale if self._fp8 else None)
        self._s = torch.cuda.current_stream() if stream is None else stream
        scales = ()
        if self._fp8:
            scales = (_dev_ptr(k_scale, "k_scale", torch.float32), _dev_ptr(v_scale, "v_scale", torch.float32))
        self._args = (plan.handle, _dev_ptr(q, "q", dt), _dev_ptr(k_pool, "k_pool", pdt),
                      _dev_ptr(v_pool, "v_pool", pdt)) + scales + (
                      _dev_ptr(block_table_dev, "block_table", torch.int32),
                      _dev_ptr(out, "out", dt), _dev_ptr(workspace, "workspace"),
                      0 if workspace is None else workspace.numel() * workspace.element_size(),
                      ctypes.c_void_p(self._s.cuda_stream))
        self._keep = (plan, q, k_pool, v_pool, block_table_dev, out, workspace, k_scale, v_scale)

    def __call__(self) -> None:
        if self._fp8:
            _check(lib().varlen_attn_run_fp8(*self._args, None))
        else:
            _check(lib().varlen_attn_run(*self._args))

    def with_events(self, events):
        """A callable that runs with ``varlen_attn_run_events`` and these VA_RUN_EVENTS
        torch.cuda.Event(enable_timing=True) objects."""
        if len(events) != VA_RUN_EVENTS:
            raise ValueError(f"need {VA_RUN_EVENTS} events")
        for ev in events:
            if ev.cuda_event == 0:
                ev.record(self._s)
        arr = (ctypes.c_void_p * VA_RUN_EVENTS)(*[ev.cuda_event for ev in events])
        args = self._args + (arr,)
        L = lib()
        fn = L.varlen_attn_run_fp8 if self._fp8 else L.varlen_attn_run_events

        def call():
            _check(fn(*args))
        call._keep = (events, arr)
        return call
