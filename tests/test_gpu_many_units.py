"""More than 512 (request, KV head) units in one step: the attention's plan
reads the list lengths in segments of 512 units, so with U > 512 a
workgroup's first unit, and a merge workgroup's unit, can lie in a later
segment.  Checked against the fp64 oracle on every unit: the whole step
(scores, lists accepted by the coverage predicate, attention on the GPU's
own lists) and the attention + merge on random caller-supplied lists (empty,
one page, all pages, subsets) over a few workgroups, so that each one's
slice crosses many units and segment boundaries."""

import functools

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.step import SparseDecodeStep

from _gpu_case import ATTN_TOL, GpuLayer, check_unit, feed_lists, say

pytestmark = pytest.mark.gpu

# 72 requests x 8 KV heads = 576 units, short ragged contexts (2 to 44 pages)
W = I.custom_workload("many_units", 72, 32, 8, ("uniform", 17, 700), alpha=("uniform", 0.5, 6),
                      index=115)


@functools.lru_cache(maxsize=1)
def _layer():
    layer = GpuLayer(W)
    units = {}
    for b in range(W.batch):
        for h in range(W.kv_heads):
            units[(b, h)] = layer.unit_oracle(b, h)
    layer.oracle_cache = units
    return layer, units


def test_step_over_576_units(gpu_lib):
    layer, _ = _layer()
    assert W.batch * W.kv_heads > 512
    st = layer.step(0.95, 3)
    layer.run(st)
    exact = 0
    worst = 0.0
    for b in range(W.batch):
        for h in range(W.kv_heads):
            r = check_unit(layer, st, b, h, 0.95)
            exact += int(r["exact"])
            worst = max(worst, r["attn_err"])
    say(f"  576 units, 3 workers: exact lists {exact}/576, max attn err {worst:.2e}")


@pytest.mark.parametrize("workers", [1, 2, 5, 0])
def test_attention_on_random_lists_over_576_units(gpu_lib, workers):
    layer, units = _layer()
    rng = np.random.default_rng(1000 + workers)
    lists = {}
    for (b, h), un in units.items():
        n = un["n"]
        kind = rng.choice(["empty", "one", "all", "some"])
        size = {"empty": 0, "one": 1, "all": n}.get(kind, int(rng.integers(1, n + 1)))
        lists[b * W.kv_heads + h] = np.sort(rng.choice(n, size=size, replace=False))
    li = layer.li
    dims = lib.make_dims(W.batch, W.q_heads, W.kv_heads, li.max_pages)
    stp = SparseDecodeStep(dims, 0.9, workers, scale=W.scale)
    stp.buf.out.fill_(3.0)
    stp.buf.out_lse.fill_(3.0)
    feed_lists(stp, layer, lists)
    stp.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages, li.ctx_lens)
    torch.cuda.synchronize()
    counts = np.array([len(lists[u]) for u in range(len(lists))])
    G = W.group
    worst = 0.0
    out = stp.buf.out.double().cpu().numpy()
    out_lse = stp.buf.out_lse.double().cpu().numpy()
    for u, lst in lists.items():
        b, h = divmod(u, W.kv_heads)
        o = out[b, h * G:(h + 1) * G]
        lse = out_lse[b, h * G:(h + 1) * G]
        if len(lst) == 0:
            assert np.all(o == 0) and np.all(np.isneginf(lse)), u
            continue
        un = units[(b, h)]
        o_ref, lse_ref = O.attend_pages(O.bf16_bits_to_f64(un["q"]), O.bf16_bits_to_f64(un["k"]),
                                        O.bf16_bits_to_f64(un["v"]), un["nv"], lst, W.scale)
        worst = max(worst, float(np.abs(o - o_ref).max()))
        assert np.abs(lse - lse_ref).max() < 1e-3, u
    assert worst <= ATTN_TOL
    say(f"  workers {workers}: {int(counts.sum())} list entries over 576 units, "
        f"max err {worst:.1e}")
