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


_FETCH_ATTN_CASES = {
    # per-unit miss and hit counts; 609 plan positions: ~30 per copying wave,
    # so slices cross units
    "short": dict(kv_heads=4, pages=260, C=640, bad_u=6,
                  miss_n=[0, 1, 2, 63, 64, 65, 130, 200], hit_n=[5, 0, 40, 3, 17, 0, 64, 33]),
    # 16 units of ~1300 misses: 18816 positions, over 64 per copying wave, so
    # a wave's slice of one unit can take its ids in two batches; one pool of
    # slots shared by both requests
    # all 16 MFMA columns live (G = 16), and one (G = 1)
    "short_g16": dict(kv_heads=2, group=16, pages=260, C=640, bad_u=3,
                      miss_n=[0, 65, 130, 200], hit_n=[7, 0, 64, 33]),
    "short_g1": dict(kv_heads=4, group=1, pages=260, C=640, bad_u=6,
                     miss_n=[1, 0, 63, 64, 65, 17, 130, 2], hit_n=[5, 9, 0, 3, 17, 0, 64, 33]),
    "long": dict(kv_heads=8, pages=1400, C=20000, pooled=True, bad_u=3,
                 miss_n=[1400, 1337, 0, 1290, 1363, 1400, 64, 1301, 1400, 1299, 1342, 0, 1385,
                         1400, 1317, 1350], hit_n=[0, 3, 7, 0, 1, 0, 0, 2, 0, 0, 0, 5, 0, 0, 1, 0]),
}


def _fetch_attn_check(w, C, pooled, miss_n, hit_n, bad_u=None, workers=8, seed=128):
    """One sparse_hbm_cache_fetch_attn call on hand-made lists: per unit u,
    hit_n[u] pages already resident in the cache and miss_n[u] pages to copy
    and attend, distinct pages of the request's context and distinct slots
    (per request, or of the pool).  With bad_u, two of that unit's miss
    entries are out of range (a page of -1, a slot past the pool) and must be
    neither copied nor attended.  Checks: every valid miss's slot holds its
    host unit bitwise, the bad page's slot keeps its old bytes, the step
    advances by one, and the pair merge of both sets of partials equals
    attention + merge over the union lists on the filled cache (and the
    oracle on two units)."""
    from adaptive_sparse_paged_amd.host_tier import UNIT_ELEMS
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    host, MP = I.build_host_pool(w, 0, lens=lens)
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, MP)
    B, H, G = w.batch, w.kv_heads, w.group
    U = B * H
    S = C if pooled else B * C              # slots in all
    rng = np.random.default_rng(seed)
    cache = HbmPageCache(dims, host, C, pooled=pooled)
    poison = torch.from_numpy(rng.integers(-2**15, 2**15, size=(S, UNIT_ELEMS),
                                           dtype=np.int16)).cuda()
    cache.cache_kv.copy_(poison)
    i32 = np.int32
    hc, hp, hx = np.zeros(U, i32), np.full((U, MP), -1, i32), np.full((U, MP), -1, i32)
    mc, mp, mx = np.zeros(U, i32), np.full((U, MP), -1, i32), np.full((U, MP), -1, i32)
    shared = list(rng.permutation(C))
    free = [shared] * B if pooled else [list(rng.permutation(C)) for _ in range(B)]
    for u in range(U):
        b, h = divmod(u, H)
        n = I.pages_of(int(lens[b]))
        pages = rng.choice(n, size=hit_n[u] + miss_n[u], replace=False).astype(i32)
        slots = np.array([(0 if pooled else b * C) + free[b].pop() for _ in pages], i32)
        hc[u], mc[u] = hit_n[u], miss_n[u]
        hp[u, :hit_n[u]], hx[u, :hit_n[u]] = pages[:hit_n[u]], slots[:hit_n[u]]
        mp[u, :miss_n[u]], mx[u, :miss_n[u]] = pages[hit_n[u]:], slots[hit_n[u]:]
        for p, x in zip(hp[u, :hit_n[u]], hx[u, :hit_n[u]]):      # the hits are resident
            cache.cache_kv[x].copy_(host[b, p, h].reshape(-1).cuda())
    bad_page_slot = None
    if bad_u is not None:
        bad_page_slot = int(mx[bad_u, 70])
        mp[bad_u, 70] = -1                # a page of -1: skipped, its slot untouched
        mx[bad_u, 100] = S + 5            # a slot past the pool: skipped
    valid = (mp >= 0) & (mx >= 0) & (mx < S)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f32 = dict(dtype=torch.float32, device="cuda")
    hmax = lib.decode_max_parts(dims, workers)
    ho, hl = torch.empty((hmax, G, 128), **f32), torch.empty((hmax, G), **f32)
    mo = torch.empty((U + lib.FETCH_ATTN_COPY_WAVES, G, 128), **f32)
    ml = torch.empty((U + lib.FETCH_ATTN_COPY_WAVES, G), **f32)
    out = torch.full((B, w.q_heads, 128), float("nan"), **f32)
    lse = torch.full((B, w.q_heads), float("nan"), **f32)
    g_hc, g_mc = dev(hc), dev(mc)
    lib.hbm_cache_fetch_attn(dims, cache.policy, host, cache.cache_kv, C, cache.step_counter,
                             li.q, li.ctx_lens, g_hc, dev(hp), dev(hx), g_mc, dev(mp), dev(mx),
                             w.scale, workers, ho, hl, hmax, mo, ml)
    lib.merge_splits_pair(dims, ho, hl, g_hc, workers, mo, ml, g_mc, lib.FETCH_ATTN_COPY_WAVES,
                          out, lse)
    torch.cuda.synchronize()
    assert int(cache.step_counter) == 1
    got = cache.cache_kv.cpu()
    for u in range(U):
        b, h = divmod(u, H)
        for i in range(miss_n[u]):
            if valid[u, i]:
                assert torch.equal(got[mx[u, i]], host[b, mp[u, i], h].reshape(-1)), (u, i)
    if bad_page_slot is not None:
        assert torch.equal(got[bad_page_slot], poison[bad_page_slot].cpu()), "bad page copied"
    # the union lists on the filled cache, one pass
    uc, up, ux = np.zeros(U, i32), np.full((U, MP), -1, i32), np.full((U, MP), -1, i32)
    for u in range(U):
        keep = valid[u, :miss_n[u]]
        pg = np.concatenate([hp[u, :hit_n[u]], mp[u, :miss_n[u]][keep]])
        sl = np.concatenate([hx[u, :hit_n[u]], mx[u, :miss_n[u]][keep]])
        uc[u] = pg.size
        up[u, :pg.size], ux[u, :pg.size] = pg, sl
    po, pl = torch.empty_like(ho), torch.empty_like(hl)
    o_ref, l_ref = torch.empty_like(out), torch.empty_like(lse)
    g_uc = dev(uc)
    lib.decode_attn(dims, li.q, cache.cache_kv, UNIT_ELEMS, 0, S, li.ctx_lens, g_uc, dev(up),
                    dev(ux), w.scale, workers, po, pl, hmax)
    lib.merge_splits(dims, po, pl, g_uc, workers, o_ref, l_ref)
    torch.cuda.synchronize()
    d = float((out - o_ref).abs().max())
    fin = torch.isfinite(l_ref)
    assert torch.equal(fin, torch.isfinite(lse)) and bool(torch.isneginf(lse[~fin]).all())
    assert d <= 1e-5 and float((lse[fin] - l_ref[fin]).abs().max()) <= 1e-5
    nonempty = [u for u in range(U) if uc[u] > 0]
    for u in ([bad_u] if bad_u is not None else []) + nonempty[-1:]:
        b, h = divmod(u, H)
        k_, v_, q_, nv = I.unit_host(w, 0, b, h, int(lens[b]))
        o_or, _ = O.attend_pages(O.bf16_bits_to_f64(q_), O.bf16_bits_to_f64(k_),
                                 O.bf16_bits_to_f64(v_), nv, up[u, :uc[u]], w.scale)
        o_gpu = out[b, h * G:(h + 1) * G].double().cpu().numpy()
        assert np.abs(o_gpu - o_or).max() <= ATTN_TOL
    return d


@pytest.mark.parametrize("case", sorted(_FETCH_ATTN_CASES))
def test_fetch_attn_direct_lists(gpu_lib, case):
    """sparse_hbm_cache_fetch_attn on hand-made lists, without a resolve:
    miss lists of many lengths (0, 1, 64, 65, ... 1400) beside hit lists on
    units placed in the cache beforehand, at G = 1, 4 and 16, per-request
    and pooled slots, with two bad miss entries (see _fetch_attn_check)."""
    cf = _FETCH_ATTN_CASES[case]
    w = I.custom_workload("fetch_attn_" + case, 2, cf.get("group", 4) * cf["kv_heads"],
                          cf["kv_heads"], ("fixed", 16 * cf["pages"] - 5), index=128)
    say(f"[fetch_attn] {case}: B=2 Hkv={w.kv_heads} G={w.group}, {cf['C']} slots "
        f"{'pooled' if cf.get('pooled') else 'per request'}, miss counts {cf['miss_n']}")
    d = _fetch_attn_check(w, cf["C"], cf.get("pooled", False), cf["miss_n"], cf["hit_n"],
                          bad_u=cf["bad_u"])
    say(f"  max |fused - one pass| {d:.1e}")


def test_fetch_attn_random_lists(gpu_lib):
    """A seeded sweep of the same check: batch 1-4, 1-4 KV heads, every
    supported G, ragged contexts, per-request or pooled slots, miss and hit
    counts drawn per unit from 0 to 300 (some units empty), 1-16 attention
    workers."""
    rng = np.random.default_rng(2024)
    for case in range(8):
        B = int(rng.integers(1, 5))
        H = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        pooled = bool(rng.integers(0, 2))
        w = I.custom_workload(f"fetch_attn_rand{case}", B, G * H, H, ("uniform", 2000, 9000),
                              index=200 + case)
        lens = I.context_lengths(w)
        miss_n, hit_n = [], []
        for u in range(B * H):
            n = I.pages_of(int(lens[u // H]))
            m = int(rng.integers(0, min(300, n) + 1)) if rng.random() > 0.2 else 0
            k = int(rng.integers(0, min(300, n - m) + 1)) if rng.random() > 0.2 else 0
            miss_n.append(m)
            hit_n.append(k)
        per_req = [sum(miss_n[b * H:(b + 1) * H]) + sum(hit_n[b * H:(b + 1) * H])
                   for b in range(B)]
        C = max(sum(per_req), 1) if pooled else max(max(per_req), 1)
        workers = int(rng.integers(1, 17))
        say(f"[fetch_attn] random case {case}: B={B} Hkv={H} G={G} "
            f"{'pooled' if pooled else 'per request'} C={C} workers={workers} "
            f"misses {sum(miss_n)} hits {sum(hit_n)}")
        _fetch_attn_check(w, C, pooled, miss_n, hit_n, workers=workers, seed=300 + case)


@pytest.mark.timeout(300)
def test_split_host_tier_full(gpu_lib):
    """The split schedule at the benchmarked host-tier shape (16 requests of
    524288 tokens, 4096 slots each, 448-page lists drifting 10%, 256
    attention workers, the copying waves' plan over ~5750 misses per step):
    5 steps from cold, the last two replayed from a graph, then one step where
    every access hits, against the one-pass step as above."""
    w = I.WORKLOADS["host_tier_512k"]
    ex = w.extra
    say("[split] host_tier_512k in full: 16 x 524288 tokens, 4096 slots, 448-page lists")
    misses, worst = _run(w, ex["capacity"], ex["list_pages"], 5, ex["drift"], workers=256,
                         graph_from=3, hit_steps=1)
    say(f"  {misses} misses, max |split - one pass| {worst:.1e}")
    assert misses > 0
