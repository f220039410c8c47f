"""Layer-wise prefetch over the host tier, for layers that share their page
lists: the pipelined step (every layer's resolve and fetch on a second
stream, each layer's attention waiting only for its own layer) against the
same step run layer by layer on one stream, against the oracle's LRU, and
against attention over the whole KV in HBM -- bitwise at every step, eagerly
and replayed from a captured graph."""

import types

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.host_tier import LayeredHostTierStep
from adaptive_sparse_paged_amd.step import SparseDecodeStep, canonical_strides, capture

from _gpu_case import feed_lists, say

pytestmark = pytest.mark.gpu


def test_layer_prefetch_matches_sequential_oracle_and_hbm(gpu_lib):
    w = I.custom_workload("prefetch", 2, 8, 2, ("fixed", 3200), layers=3, index=123)
    nl, C, LP, steps, eager_steps = 3, 48, 20, 9, 4
    say(f"[prefetch] B=2 Hkv=2 {nl} layers, {C} slots, lists of {LP}, drift 20%, {steps} steps")
    lens = I.context_lengths(w)
    lis = [I.build_layer(w, l, "cuda", lens=lens) for l in range(nl)]
    hosts = [I.build_host_pool(w, l, lens=lens)[0] for l in range(nl)]
    MP = lis[0].max_pages
    B, H, G = w.batch, w.kv_heads, w.group
    U = B * H
    dims = lib.make_dims(B, w.q_heads, H, MP)
    seq = LayeredHostTierStep(dims, hosts, C, 0.99, 8, scale=w.scale, prefetch=False)
    pre = LayeredHostTierStep(dims, hosts, C, 0.99, 8, scale=w.scale, prefetch=True)
    lists = I.drift_lists(w, min(I.pages_of(L) for L in lens), LP, steps, 0.2)
    qs = [li.q for li in lis]
    mk = lambda: ([torch.empty((B, w.q_heads, 128), dtype=torch.float32, device="cuda")
                   for _ in range(nl)],
                  [torch.empty((B, w.q_heads), dtype=torch.float32, device="cuda")
                   for _ in range(nl)])
    o_seq, l_seq = mk()
    o_pre, l_pre = mk()
    hbm = SparseDecodeStep(dims, 0.99, 8, scale=w.scale)
    sp_, sh_ = canonical_strides(H)
    states = [O.LRUState(C, H * MP) for _ in range(B)]
    graph = None

    def feed(step, t):
        step.sel_counts.fill_(LP)
        step.sel_pages[:, :LP].copy_(torch.from_numpy(lists[t].reshape(U, LP)))

    for t in range(steps):
        feed(seq, t)
        seq.run(qs, lis[0].ctx_lens, o_seq, l_seq)
        feed(pre, t)
        if t < eager_steps:
            pre.run(qs, lis[0].ctx_lens, o_pre, l_pre)
        else:
            if graph is None:
                graph = capture(lambda: pre.run(qs, lis[0].ctx_lens, o_pre, l_pre), warmup=0)
            for o in o_pre:
                o.zero_()
            graph.replay()
        torch.cuda.synchronize()
        # the two schedules agree bitwise, layer by layer
        for l in range(nl):
            assert torch.equal(o_seq[l], o_pre[l]) and torch.equal(l_seq[l], l_pre[l]), (t, l)
            assert torch.equal(seq.caches[l].slot_tag, pre.caches[l].slot_tag), (t, l)
            assert torch.equal(seq.caches[l].stats, pre.caches[l].stats), (t, l)
        # every layer's cache follows the oracle's LRU on the shared lists
        want = []
        for b in range(B):
            units = [h * MP + int(p) for h in range(H) for p in lists[t, b, h]]
            r = O.resolve_step(states[b], units, t)
            want.append([r["hits"], r["misses"], r["evictions"], r["overflow"]])
            assert r["overflow"] == 0
        for l in range(nl):
            assert pre.caches[l].stats.cpu().numpy().tolist() == want, (t, l)
            assert np.array_equal(pre.caches[l].slot_tag.cpu().numpy(),
                                  np.stack([s.tag for s in states])), (t, l)
        # attention through the caches equals attention over the HBM pools
        for l in range(nl):
            layer = types.SimpleNamespace(w=w, dims=dims, li=lis[l])
            feed_lists(hbm, layer, {u: lists[t].reshape(U, LP)[u] for u in range(U)})
            oh, lh = hbm.attend(qs[l], lis[l].kv_pool, sp_, sh_, lis[l].pool_pages,
                                lis[l].ctx_lens)
            torch.cuda.synchronize()
            assert torch.equal(oh, o_pre[l]) and torch.equal(lh, l_pre[l]), (t, l, "vs HBM")
    misses = sum(int(c.stats[:, 1].sum()) for c in pre.caches)
    say(f"  {steps} steps bitwise equal; graph replays from step {eager_steps}; "
        f"total misses {misses}")
