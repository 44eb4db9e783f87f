"""varlen_attn_run / varlen_attn_run_fp8 captured into a HIP graph (through torch.cuda.graph)
and replayed: every replay equals the eager run on the same inputs bit for bit, also after
the inputs change between replays (the graph reads the buffers, not a snapshot)."""
import sys

import numpy as np
import pytest

from varlen_paged_attention_amd import api, workloads as W

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    api.lib()
    yield


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("label,cid,scale,dtype,flags", [
    ("orca-mixed/4", 2, 4, None, 0),
    ("decode-heavy/8", 3, 8, None, 0),
    ("shared-6", 5, 1, None, api.VA_FLAG_SHARED_PREFIX),
    ("decode-heavy/8 fp8", 3, 8, "fp8", 0),
    # the tile kernel in its other forms: decode tiles, key-chunk tiles with decode tiles in
    # one launch, shared-prefix group tiles with members' own-key tiles
    ("decode-heavy (decode tiles)", 3, 1, None, 0),
    ("long-prefix-chunk/4 (chunk + decode tiles)", 9, 4, None, 0),
    ("shared-64/4 (column-list tiles)", 51, 4, None, api.VA_FLAG_SHARED_PREFIX),
])
def test_graph_replays_match_eager(label, cid, scale, dtype, flags):
    import torch
    w = W.config(cid, scale=scale, dtype=dtype)
    _say(f"[gpu] graph capture {label}")
    plan = api.plan_for(w, flags=flags)
    q, k, v, bt = api.to_device(w)
    scales = dict(zip(("k_scale", "v_scale"), api.scales_to_device(w))) if w.dtype == "fp8" else {}
    ws = api.new_workspace(plan)
    out_eager = torch.zeros_like(q)
    out_graph = torch.zeros_like(q)
    api.RunCall(plan, q, k, v, bt, out_eager, ws, **scales)()
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call = api.RunCall(plan, q, k, v, bt, out_graph, ws, stream=s, **scales)
        call()                                    # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()

    q0 = q.clone()
    for rep in range(3):
        if rep == 2:
            q.copy_(q0.flip(0))                   # new inputs, same buffers
            api.RunCall(plan, q, k, v, bt, out_eager, ws, **scales)()
            torch.cuda.synchronize()
        out_graph.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out_graph), _bits(out_eager)), f"{label}: replay {rep} differs from eager"
        _ = (q * 2).sum().item()                  # eager work between replays
