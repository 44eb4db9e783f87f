"""varlen_attn_run_noalloc (the library's static device scratch as the workspace) against
varlen_attn_run with a caller-allocated workspace, through the C ABI: two calls in a row,
the second on a smaller iteration (the scratch then holds the first call's partials)."""
import sys

import numpy as np
import pytest

from varlen_paged_attention_amd import api, workloads as W

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.int32)


def _both(w, **kw):
    import torch
    plan = api.plan_for(w, **kw)
    assert 0 < plan.workspace_bytes <= api.VA_STATIC_SCRATCH_BYTES
    q, k, v, bt = api.to_device(w)
    ref = torch.full_like(q, 3.0)
    api.varlen_attn_run(plan, q, k, v, bt, ref, api.new_workspace(plan))
    got = torch.full_like(q, 5.0)
    api.varlen_attn_run_noalloc(plan, q, k, v, bt, got)
    torch.cuda.synchronize()
    return plan, ref, got


def test_noalloc_matches_run_two_calls_second_smaller():
    cases = [
        # split-KV items and the combine pass: 17.6 MiB of partials
        ("decode-heavy on split-KV items", W.config(3), dict(flags=api.VA_FLAG_NO_DECODE_TILES)),
        # a smaller iteration next (17.7 MiB of partials): a 32-row chunk on an 8192-position
        # prefix cut into key-chunk tiles, with 8 decodes
        ("long-prefix-chunk/8 (key-chunk tiles)", W.config(9, scale=8, poison_tail=True), {}),
        # and a smaller one again (5.1 MiB): 64 decodes on split-KV items
        ("decode-heavy/4 on split-KV items", W.config(3, scale=4, poison_tail=True),
         dict(flags=api.VA_FLAG_NO_DECODE_TILES)),
    ]
    sizes = []
    for label, w, kw in cases:
        _say(f"[gpu] noalloc {label}")
        plan, ref, got = _both(w, **kw)
        sizes.append(plan.workspace_bytes)
        rows = np.zeros(w.total_q_rows, bool)
        for r in range(w.num_reqs):
            rows[w.q_start[r]:w.q_end[r]] = True
        a, b = _bits(ref), _bits(got)
        assert np.array_equal(a[rows], b[rows]), f"{label}: noalloc output differs from run"
        assert (got.float().cpu().numpy()[~rows] == 5.0).all(), f"{label}: rows outside every request written"
        diff = float((ref.float() - got.float()).abs().max())
        _say(f"[parity] noalloc {label}: workspace {plan.workspace_bytes} bytes, max |noalloc - run| = {diff:.3e}")
        assert diff <= TOL
    assert sizes[2] < sizes[1] < sizes[0]


def test_noalloc_refuses_plans_beyond_the_scratch():
    import torch
    w = W.config(7, scale=1)                     # 8-row verify steps on split items: 143 MiB of partials
    plan = api.plan_for(w, flags=api.VA_FLAG_NO_DECODE_TILES)
    assert plan.workspace_bytes > api.VA_STATIC_SCRATCH_BYTES
    q, k, v, bt = api.to_device(w)
    out = torch.zeros_like(q)
    with pytest.raises(api.VarlenAttnError) as ei:
        api.varlen_attn_run_noalloc(plan, q, k, v, bt, out)
    assert ei.value.status == api.VA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert not out.any()
