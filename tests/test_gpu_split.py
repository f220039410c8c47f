"""The host tier in two halves -- attention over the hits beside the fetch of
the misses, then attention over the misses merged into the hits' result --
against the one-call resolve and one-pass attention on a second cache fed
the same lists: cache state, statistics and slot ids bitwise at every step;
hit_phys equal to the residency before the step; the miss lists equal to
their definition; outputs equal up to the order of the merge and within the
oracle's bar; eagerly and replayed from a captured graph."""

import types

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.host_tier import HbmPageCache, SplitHostTierStep
from adaptive_sparse_paged_amd.step import SparseDecodeStep, canonical_strides, capture

from _gpu_case import ATTN_TOL, feed_lists, say

pytestmark = pytest.mark.gpu


def _run(w, C, LP, steps, drift, pooled=False, shift=0, workers=8, graph_from=None,
         hit_steps=0):
    """hit_steps: that many more steps on the last lists again, where every
    access hits (the copying workgroups find nothing to copy)."""
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    host, MP = I.build_host_pool(w, 0, lens=lens)
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, MP)
    B, H, G = w.batch, w.kv_heads, w.group
    U = B * H
    ref_cache = HbmPageCache(dims, host, C, recency_shift=shift, pooled=pooled)
    spl_cache = HbmPageCache(dims, host, C, recency_shift=shift, pooled=pooled)
    ref = SparseDecodeStep(dims, 0.99, workers, scale=w.scale)
    spl = SplitHostTierStep(dims, spl_cache, 0.99, workers, scale=w.scale)
    layer = types.SimpleNamespace(w=w, dims=dims, li=li)
    lists = I.drift_lists(w, min(I.pages_of(L) for L in lens), LP, steps, drift)
    if hit_steps:
        lists = np.concatenate([lists] + [lists[-1:]] * hit_steps)
        steps += hit_steps
    out = torch.empty((B, w.q_heads, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, w.q_heads), dtype=torch.float32, device="cuda")
    graph, misses_total, worst = None, 0, 0.0
    for t in range(steps):
        feed_lists(ref, layer, {b * H + h: lists[t, b, h] for b in range(B) for h in range(H)})
        spl.sel_counts.copy_(ref.buf.sel_counts)
        spl.sel_pages.copy_(ref.buf.sel_pages)
        before = spl_cache.unit_slot.clone()
        ref_cache.resolve(ref.buf.sel_counts, ref.buf.sel_pages, ref.buf.sel_phys)
        o_ref, l_ref = ref.attend(li.q, *ref_cache.pool_args(), li.ctx_lens)
        if graph_from is not None and t >= graph_from:
            if graph is None:
                graph = capture(lambda: spl.run(li.q, li.ctx_lens, out, lse), warmup=0)
            out.zero_()
            graph.replay()
        else:
            spl.run(li.q, li.ctx_lens, out, lse)
        torch.cuda.synchronize()
        for name in ("slot_tag", "slot_stamp", "unit_slot", "stats", "step_counter"):
            assert torch.equal(getattr(ref_cache, name), getattr(spl_cache, name)), (t, name)
        assert int(spl_cache.stats[:, 3].sum()) == 0, "case sized to never overflow"
        misses_total += int(spl_cache.stats[:, 1].sum())
        if hit_steps and t >= steps - hit_steps:
            assert int(spl_cache.stats[:, 1].sum()) == 0, (t, "an all-hit step missed")
        counts = ref.buf.sel_counts.cpu().numpy()
        pages = ref.buf.sel_pages.cpu().numpy()
        phys = ref.buf.sel_phys.cpu().numpy()
        hit = spl.hit_phys.cpu().numpy()
        prev = before.cpu().numpy().reshape(-1)
        mc = spl.miss.buf.sel_counts.cpu().numpy()
        mp = spl.miss.buf.sel_pages.cpu().numpy()
        mx = spl.miss.buf.sel_phys.cpu().numpy()
        for u in range(U):
            b, h = divmod(u, H)
            k = counts[u]
            assert np.array_equal(spl.sel_phys.cpu().numpy()[u, :k], phys[u, :k]), (t, u)
            units = (b * H + h) * MP + pages[u, :k] if pooled else b * H * MP + h * MP + pages[u, :k]
            resident = prev[units] >= 0
            want_hit = np.where(resident, phys[u, :k], -1)
            assert np.array_equal(hit[u, :k], want_hit), (t, u, "hit_phys")
            is_miss = (~resident) & (phys[u, :k] >= 0)
            assert mc[u] == is_miss.sum(), (t, u, "miss count")
            assert np.array_equal(mp[u, :mc[u]], pages[u, :k][is_miss]), (t, u, "miss pages")
            assert np.array_equal(mx[u, :mc[u]], phys[u, :k][is_miss]), (t, u, "miss slots")
        # the same attention up to the order of the log-sum-exp merge
        d = float((out - o_ref).abs().max())
        assert d <= 1e-5, (t, "output", d)
        assert float((lse - l_ref).abs().max()) <= 1e-5, (t, "lse")
        worst = max(worst, d)
    # and within the oracle's bar on a few units of the last step
    for b, h in [(0, 0), (B - 1, H - 1)]:
        u = b * H + h
        k_, v_, q_, nv = I.unit_host(w, 0, b, h, int(lens[b]))
        lst = pages[u, :counts[u]]
        o_or, _ = O.attend_pages(O.bf16_bits_to_f64(q_), O.bf16_bits_to_f64(k_),
                                 O.bf16_bits_to_f64(v_), nv, lst, w.scale)
        o_gpu = out[b, h * G:(h + 1) * G].double().cpu().numpy()
        assert np.abs(o_gpu - o_or).max() <= ATTN_TOL
    return misses_total, worst


@pytest.mark.parametrize("pooled,shift", [(False, 0), (True, 0), (False, 2)],
                         ids=["exact", "pooled", "bucketed2"])
def test_split_host_tier_matches_one_pass(gpu_lib, pooled, shift):
    w = I.custom_workload("split", 2, 8, 2, ("fixed", 3200), index=124)
    say(f"[split] B=2 Hkv=2, 64 slots, lists of 24 drifting 25%, pooled={pooled} shift={shift}")
    C = 2 * 64 if pooled else 64
    misses, worst = _run(w, C, 24, 10, 0.25, pooled=pooled, shift=shift, graph_from=5)
    say(f"  10 steps (graph from step 5), {misses} misses, max |split - one pass| {worst:.1e}")
    assert misses > 0


@pytest.mark.parametrize("pooled", [False, True], ids=["exact", "pooled"])
def test_split_many_requests_then_all_hits(gpu_lib, pooled):
    """70 requests (the copying waves read the per-request miss counts 64 at
    a time: two blocks), lists of 12 pages drifting 50%, then two steps on
    the same lists where every access hits: nothing to copy, the one-pass
    resolve places nothing.  Against the one-pass step as above, eagerly and
    (from step 3) replayed from a graph."""
    w = I.custom_workload("split_many", 70, 8, 2, ("fixed", 1600), index=127)
    say(f"[split] 70 requests x 2 KV heads, 48 slots each, lists of 12, 4 drifting steps "
        f"then 2 all-hit steps, pooled={pooled}")
    C = 70 * 48 if pooled else 48
    misses, worst = _run(w, C, 12, 4, 0.5, pooled=pooled, workers=32, graph_from=3,
                         hit_steps=2)
    assert misses > 0


def test_split_cold_step_all_misses(gpu_lib):
    """The first step misses everything: the hit pass sees only empty pages
    (lse -inf), and the result is the miss pass alone."""
    w = I.custom_workload("split_cold", 3, 16, 4, ("fixed", 2000), index=125)
    say("[split] cold start, B=3 Hkv=4, 256 slots, lists of 40")
    misses, worst = _run(w, 256, 40, 2, 0.5, workers=16)
    assert misses > 0


def test_merge_pair_of_disjoint_lists(gpu_lib):
    """sparse_merge_splits_pair on lists cut in two (alternate entries; some
    units with one side empty, some with both): attention over part A and
    over part B, one merge of both sets of partials, against attention +
    merge over the whole lists (up to the order of the merge), and -- for
    units whose part A is empty -- bitwise equal to merge_splits over part B
    alone, and the reverse."""
    w = I.custom_workload("merge_pair", 3, 16, 4, ("fixed", 4000), index=126)
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, li.max_pages)
    B, H, G = w.batch, w.kv_heads, w.group
    layer = types.SimpleNamespace(w=w, dims=dims, li=li)
    rng = np.random.default_rng(126)
    n = I.pages_of(int(lens.min()))
    whole, part_a, part_b = {}, {}, {}
    for u in range(B * H):
        k = [0, 1, 2, 37, 180][u % 5]
        lst = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)
        whole[u] = lst
        if u % 3 == 1:                          # A empty: everything in B
            part_a[u], part_b[u] = lst[:0], lst
        else:                                   # B empty when the list has < 2 entries
            part_a[u], part_b[u] = lst[0::2], lst[1::2]
    sp_, sh_ = canonical_strides(H)
    workers, workers_b = 16, 5          # the two sets planned for different grids
    ref = SparseDecodeStep(dims, 0.99, workers, scale=w.scale)
    sa = SparseDecodeStep(dims, 0.99, workers, scale=w.scale)
    sb = SparseDecodeStep(dims, 0.99, workers_b, scale=w.scale)
    feed_lists(ref, layer, whole)
    feed_lists(sa, layer, part_a)
    feed_lists(sb, layer, part_b)
    args = (li.q, li.kv_pool, sp_, sh_, li.pool_pages, li.ctx_lens)
    o_ref, l_ref = ref.attend(*args)
    for st_ in (sa, sb):
        b_ = st_.buf
        lib.decode_attn(dims, *args, b_.sel_counts, b_.sel_pages, b_.sel_phys, st_.scale,
                        st_.workers, b_.part_o, b_.part_lse, st_.max_parts)
    a_, b_ = sa.buf, sb.buf
    out = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    lib.merge_splits_pair(dims, a_.part_o, a_.part_lse, a_.sel_counts, workers, b_.part_o,
                          b_.part_lse, b_.sel_counts, workers_b, out, lse)
    o_a, l_a = torch.empty_like(out), torch.empty_like(lse)
    o_b, l_b = torch.empty_like(out), torch.empty_like(lse)
    lib.merge_splits(dims, a_.part_o, a_.part_lse, a_.sel_counts, workers, o_a, l_a)
    lib.merge_splits(dims, b_.part_o, b_.part_lse, b_.sel_counts, workers_b, o_b, l_b)
    torch.cuda.synchronize()
    d = float((out - o_ref).abs().max())
    say(f"  max |pair merge - whole| {d:.1e}")
    fin = torch.isfinite(l_ref)
    assert torch.equal(fin, torch.isfinite(lse)) and bool(torch.isneginf(lse[~fin]).all())
    assert d <= 1e-5 and float((lse[fin] - l_ref[fin]).abs().max()) <= 1e-5
    for u in range(B * H):
        b, h = divmod(u, H)
        rows = slice(h * G, (h + 1) * G)
        if len(whole[u]) == 0:
            assert bool((out[b, rows] == 0).all()) and bool(torch.isinf(lse[b, rows]).all())
        elif len(part_a[u]) == 0:
            assert torch.equal(out[b, rows], o_b[b, rows]), u
            assert torch.equal(lse[b, rows], l_b[b, rows]), u
        elif len(part_b[u]) == 0:
            assert torch.equal(out[b, rows], o_a[b, rows]), u
            assert torch.equal(lse[b, rows], l_a[b, rows]), u
