"""Property test of the attention over caller-supplied page lists: for
randomly drawn ragged batches of lists (empty, single-page, full and
arbitrary subsets), attention grids (1 workgroup up to more workgroups than
pages, and the device default) and list bounds, the GPU's attention + merge
matches exact fp64 attention over the same pages (1e-2 max-abs), and units
with empty lists give o = 0 and lse = -inf.  Run on a GQA group of 4 and on
one of 16."""

import functools

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.step import SparseDecodeStep

from _gpu_case import ATTN_TOL, GpuLayer, feed_lists, say

pytestmark = pytest.mark.gpu

W4 = I.custom_workload("prop", 4, 8, 2, ("uniform", 17, 3000), alpha=("uniform", 1, 6),
                       index=114)
W16 = I.custom_workload("prop16", 3, 32, 2, ("uniform", 17, 70000), alpha=("uniform", 1, 6),
                        index=117)


@functools.lru_cache(maxsize=2)
def _layer(W):
    layer = GpuLayer(W)
    units = {}
    for b in range(W.batch):
        for h in range(W.kv_heads):
            un = layer.unit_oracle(b, h)
            units[(b, h)] = dict(n=un["n"], nv=un["nv"], q=O.bf16_bits_to_f64(un["q"]),
                                 k=O.bf16_bits_to_f64(un["k"]), v=O.bf16_bits_to_f64(un["v"]))
    return layer, units


SETTINGS = dict(deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


@settings(max_examples=12, **SETTINGS)
@given(data=st.data(), workers=st.sampled_from([1, 3, 8, 32, 64, 0, 5000]),
       bounded=st.booleans())
def test_attention_on_random_ragged_lists(gpu_lib, data, workers, bounded):
    _check_random_lists(W4, data, workers, bounded)


@settings(max_examples=5, **SETTINGS)
@given(data=st.data(), workers=st.sampled_from([1, 7, 0]), bounded=st.booleans())
def test_attention_on_random_ragged_lists_g16(gpu_lib, data, workers, bounded):
    _check_random_lists(W16, data, workers, bounded)


def _check_random_lists(W, data, workers, bounded):
    layer, units = _layer(W)
    lists = {}
    for (b, h), un in units.items():
        n = un["n"]
        kind = data.draw(st.sampled_from(["empty", "one", "all", "some"]))
        seed = data.draw(st.integers(0, 2**31 - 1))
        rng = np.random.default_rng(seed)
        size = {"empty": 0, "one": 1, "all": n}.get(kind, int(rng.integers(1, n + 1)))
        lists[b * W.kv_heads + h] = np.sort(rng.choice(n, size=size, replace=False))
    longest = max(len(x) for x in lists.values())
    bound = max(1, longest) if bounded else 0
    li = layer.li
    dims = lib.make_dims(W.batch, W.q_heads, W.kv_heads, li.max_pages, max_list_pages=bound)
    stp = SparseDecodeStep(dims, 0.9, workers, scale=W.scale)
    stp.buf.out.fill_(3.0)
    stp.buf.out_lse.fill_(3.0)
    feed_lists(stp, layer, lists)
    stp.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages, li.ctx_lens)
    torch.cuda.synchronize()
    G = W.group
    worst = 0.0
    for u, lst in lists.items():
        b, h = divmod(u, W.kv_heads)
        o = stp.buf.out[b, h * G:(h + 1) * G].double().cpu().numpy()
        lse = stp.buf.out_lse[b, h * G:(h + 1) * G].double().cpu().numpy()
        if len(lst) == 0:
            assert np.all(o == 0) and np.all(np.isneginf(lse)), u
            continue
        un = units[(b, h)]
        o_ref, lse_ref = O.attend_pages(un["q"], un["k"], un["v"], un["nv"], lst, W.scale)
        worst = max(worst, float(np.abs(o - o_ref).max()))
        assert np.abs(lse - lse_ref).max() < 1e-3, u
    assert worst <= ATTN_TOL
    say(f"  G {W.group} workers {workers} bound {bound}: "
        f"sizes {sorted(len(x) for x in lists.values())}, max err {worst:.1e}")
