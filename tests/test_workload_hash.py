"""The counter-based page values of the long-context workload: the host (NumPy) and torch
versions of the generator give the same bits, pages differ from each other and from pool
to pool, and the values lie on the stated grid."""
import numpy as np
import torch

from varlen_paged_attention_amd import workloads as W


def test_lowbias32_reference_values():
    """h(0) = 0 and h is a bijection on a sample (an xor-shift-multiply chain with odd
    multipliers loses no information)."""
    x = np.arange(1 << 16, dtype=np.int64) * 65537
    h = W._lowbias32(x)
    assert int(W._lowbias32(np.array([0], np.int64))[0]) == 0
    assert len(np.unique(h)) == len(x) and h.max() <= W._M32 and h.min() >= 0


def test_host_and_torch_generators_agree():
    w = W.config(8, scale=256)
    pages = np.arange(w.num_pages)
    kd, vd = W.hashed_pools_device(w, device="cpu", pages_per_chunk=3)
    assert np.array_equal(kd.view(torch.int16).numpy().view(np.uint16), W.hashed_pages_host(w, pages, W.STREAM_K))
    assert np.array_equal(vd.view(torch.int16).numpy().view(np.uint16), W.hashed_pages_host(w, pages, W.STREAM_V))


def test_page_values_grid_and_independence():
    w = W.config(8, scale=256)
    k = W.hashed_pages_host(w, [0, 1], W.STREAM_K)
    v = W.hashed_pages_host(w, [0], W.STREAM_V)
    f = (k.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(f) <= 255 / 128) and np.all((f * 128) == np.round(f * 128))
    assert 0.75 < f.std() < 0.88 and abs(f.mean()) < 0.02
    assert not np.array_equal(k[0], k[1])
    assert not np.array_equal(k[0].reshape(-1), v[0].reshape(-1))


def test_long_context_shape():
    """256 decodes x 128K context, page 64: 524,288 block-table entries."""
    w = W.config(8)
    assert w.block_table.shape == (256, 2048) and w.num_pages == 524288
    assert np.all(w.kv_len == 131072) and w.k_pool is None
