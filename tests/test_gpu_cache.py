"""GPU parity of the host-tier cache resolver against the oracle's LRU model:
slot tags, stamps, unit map, statistics and slot ids exact at every step;
every resident slot holds its unit's bytes exactly; attention read through the
cache is bit-identical to attention over the HBM pool (placement only)."""

import types

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.host_tier import HbmPageCache
from adaptive_sparse_paged_amd.step import SparseDecodeStep, canonical_strides

from _gpu_case import feed_lists, say

pytestmark = pytest.mark.gpu


def _case(w, C, list_pages, steps, drift, workers=8, check_all_slots=True, lists=None,
          shift=0, pooled=False):
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    host, MP = I.build_host_pool(w, 0, lens=lens)
    assert MP == li.max_pages
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, MP)
    cache = HbmPageCache(dims, host, C, recency_shift=shift, pooled=pooled)
    n_pages = min(I.pages_of(L) for L in lens)
    if lists is None:
        lists = I.drift_lists(w, n_pages, list_pages, steps, drift)
    B, H = w.batch, w.kv_heads
    space = H * MP
    if pooled:
        pool_state = O.LRUState(C, B * space)
    else:
        states = [O.LRUState(C, space) for _ in range(B)]
    st = SparseDecodeStep(dims, 0.99, workers, scale=w.scale)
    layer = types.SimpleNamespace(w=w, dims=dims, li=li)
    sp_, sh_ = canonical_strides(H)
    out_stats = []
    for t in range(lists.shape[0]):
        feed_lists(st, layer, {b * H + h: lists[t, b, h] for b in range(B) for h in range(H)})
        phys_hbm = st.buf.sel_phys.clone()
        cache.resolve(st.buf.sel_counts, st.buf.sel_pages, st.buf.sel_phys)
        torch.cuda.synchronize()
        tags = cache.slot_tag.cpu().numpy()
        stamps = cache.slot_stamp.cpu().numpy()
        umap = cache.unit_slot.cpu().numpy()
        stats = cache.stats.cpu().numpy()
        phys = st.buf.sel_phys.cpu().numpy()
        if pooled:
            per_req = [[O.pooled_unit(b, h, int(p), H, MP) for h in range(H) for p in lists[t, b, h]]
                       for b in range(B)]
            r = O.resolve_pooled_step(pool_state, per_req, t, space, recency_shift=shift)
            assert np.array_equal(tags, pool_state.tag), (t, "tags")
            assert np.array_equal(stamps, pool_state.stamp), (t, "stamps")
            assert np.array_equal(umap.reshape(-1), pool_state.slot_of), (t, "unit map")
            assert np.array_equal(stats, r["per_request"]), (t, "stats")
            for b in range(B):
                for h in range(H):
                    u = b * H + h
                    k = len(lists[t, b, h])
                    want = [pool_state.slot_of[O.pooled_unit(b, h, int(p), H, MP)]
                            for p in lists[t, b, h]]
                    assert phys[u, :k].tolist() == [int(x) for x in want], (t, b, h, "slot ids")
                out_stats.append(dict(hits=int(r["per_request"][b, 0]),
                                      misses=int(r["per_request"][b, 1]),
                                      evictions=int(r["per_request"][b, 2]),
                                      overflow=int(r["per_request"][b, 3])))
            # resident slots hold their units' bytes
            res = np.nonzero(tags >= 0)[0]
            if not check_all_slots:
                res = res[:: max(1, len(res) // 64)]
            g = tags[res]
            b_, rest = g // space, g % space
            h_, p_ = rest // MP, rest % MP
            want = host[torch.from_numpy(b_), torch.from_numpy(p_), torch.from_numpy(h_)]
            got = cache.cache_kv[torch.from_numpy(res).cuda()].cpu()
            assert torch.equal(got, want.reshape(len(res), -1)), (t, "slot contents")
        else:
            for b in range(B):
                units = [h * MP + int(p) for h in range(H) for p in lists[t, b, h]]
                r = O.resolve_step(states[b], units, t, recency_shift=shift)
                assert np.array_equal(tags[b], states[b].tag), (t, b, "tags")
                assert np.array_equal(stamps[b], states[b].stamp), (t, b, "stamps")
                assert np.array_equal(umap[b], states[b].slot_of), (t, b, "unit map")
                assert stats[b].tolist() == [r["hits"], r["misses"], r["evictions"], r["overflow"]], (t, b)
                for h in range(H):
                    u = b * H + h
                    k = len(lists[t, b, h])
                    want = [states[b].slot_of[h * MP + int(p)] for p in lists[t, b, h]]
                    want = [b * C + s if s >= 0 else -1 for s in want]
                    assert phys[u, :k].tolist() == want, (t, b, h, "slot ids")
                out_stats.append(r)
            # resident slots hold their units' bytes
            cache_kv = cache.cache_kv.view(B, C, -1)
            for b in range(B):
                res = np.nonzero(tags[b] >= 0)[0]
                if not check_all_slots:
                    res = res[:: max(1, len(res) // 64)]
                v = tags[b][res]
                h, p = v // MP, v % MP
                want = host[b, torch.from_numpy(p), torch.from_numpy(h)].reshape(len(res), -1)
                got = cache_kv[b, torch.from_numpy(res).cuda()].cpu()
                assert torch.equal(got, want), (t, b, "slot contents")
        # attention through the cache is bit-identical to attention over HBM
        if not any(r["overflow"] for r in out_stats[-B:]):
            kv, s_page, s_head, ppages = cache.pool_args()
            oc, lc = st.attend(li.q, kv, s_page, s_head, ppages, li.ctx_lens)
            oc, lc = oc.clone(), lc.clone()
            oh, lh = st.attend(li.q, li.kv_pool, sp_, sh_, li.pool_pages, li.ctx_lens,
                               sel_phys=phys_hbm)
            torch.cuda.synchronize()
            assert torch.equal(oc, oh) and torch.equal(lc, lh), (t, "attention differs")
    return out_stats


def test_cache_resolver_repeated_lists_all_hit(gpu_lib):
    """Drifting steps, then the same lists again: every access hits, the
    resolve places nothing and copies nothing, stamps move to the new step
    and the step counter still advances once per call."""
    w = I.custom_workload("cache_rep", 3, 8, 2, ("fixed", 3200), index=128)
    base = I.drift_lists(w, I.pages_of(3200), 20, 4, 0.3)
    lists = np.concatenate([base, base[-1:], base[-1:], base[-1:]])
    say("[cache] 4 drifting steps then 3 all-hit steps, B=3 Hkv=2, 64 slots")
    stats = _case(w, C=64, list_pages=20, steps=lists.shape[0], drift=0.0, lists=lists)
    assert all(r["misses"] == 0 for r in stats[-9:])
    assert sum(r["misses"] for r in stats[:12]) > 0


def test_cache_resolver_small_drift(gpu_lib):
    w = I.custom_workload("cache_small", 2, 8, 2, ("fixed", 3200), index=120)
    say("[cache] small: B=2 Hkv=2 200 pages, 48 slots, lists of 20, drift 20%, 14 steps")
    stats = _case(w, C=48, list_pages=20, steps=14, drift=0.2)
    assert sum(r["evictions"] for r in stats) > 0
    assert sum(r["hits"] for r in stats) > 0


def test_cache_resolver_random_lists_and_ties(gpu_lib):
    """Lists of varying length that jump around, so LRU ties at equal stamps
    are broken by unit id, and some steps leave slots free."""
    w = I.custom_workload("cache_jump", 3, 12, 3, ("fixed", 1600), index=121)
    rng = np.random.default_rng(3)
    steps, H, n = 10, 3, 100
    L = 12
    lists = np.zeros((steps, 3, H, L), dtype=np.int32)
    for t in range(steps):
        for b in range(3):
            for h in range(H):
                lists[t, b, h] = np.sort(rng.choice(n if t % 3 else 30, size=L, replace=False))
    say("[cache] jumping lists, 3 requests x 3 KV heads, 40 slots")
    stats = _case(w, C=40, list_pages=L, steps=steps, drift=0.0, workers=5, lists=lists)
    assert sum(r["evictions"] for r in stats) > 0


def test_cache_overflow_flagged(gpu_lib):
    w = I.custom_workload("cache_ovf", 2, 8, 2, ("fixed", 1600), index=122)
    say("[cache] overflow: 2 heads x 20 pages into 30 slots")
    stats = _case(w, C=30, list_pages=20, steps=2, drift=0.1, workers=4)
    assert all(r["overflow"] == 1 for r in stats)


def test_cache_pool_overflow_flagged(gpu_lib):
    """A shared pool too small for the step's demand: misses rank request by
    request, so the last request's misses go unplaced and only it (and any
    request that shares the boundary) is flagged, as in the oracle."""
    w = I.custom_workload("cache_povf", 3, 8, 2, ("fixed", 1600), index=126)
    say("[cache] pooled overflow: 3 requests x 2 heads x 20 pages into 100 slots")
    stats = _case(w, C=100, list_pages=20, steps=2, drift=0.1, workers=4, pooled=True)
    flags = [r["overflow"] for r in stats]
    assert flags[:3] == [0, 0, 1]


@pytest.mark.timeout(300)
def test_cache_resolver_host_tier_shape(gpu_lib):
    """The host-tier workload's shape (524288-token contexts, 8 KV heads,
    4096 slots, lists of 448 pages drifting 10%) for 2 requests and 4 steps."""
    base = I.WORKLOADS["host_tier_512k"]
    w = I.custom_workload("host_tier_2req", 2, 32, 8, base.ctx, alpha=base.alpha, index=4)
    ex = base.extra
    say("[cache] host-tier shape: 2 x 524288 tokens, 4096 slots, 448-page lists")
    stats = _case(w, C=ex["capacity"], list_pages=ex["list_pages"], steps=4, drift=ex["drift"],
                  workers=128, check_all_slots=False)
    assert stats[-1]["misses"] > 0 and stats[-1]["hits"] > 0


@pytest.mark.timeout(300)
def test_cache_pool_host_tier_scale(gpu_lib):
    """A pool shared by 8 requests of 131072 tokens: 32768 slots (32 blocks of
    the pooled resolver), lists of 448 pages per KV head drifting 10%, 4
    steps, against the pooled oracle."""
    base = I.WORKLOADS["host_tier_512k"]
    w = I.custom_workload("pool_scale", 8, 32, 8, ("fixed", 131072), alpha=base.alpha, index=127)
    say("[cache] pooled at scale: 8 x 131072 tokens, 32768 shared slots, 448-page lists")
    stats = _case(w, C=8 * 4096, list_pages=448, steps=4, drift=0.1, workers=128,
                  check_all_slots=False, pooled=True, shift=1)
    assert sum(r["misses"] for r in stats[-8:]) > 0 and sum(r["hits"] for r in stats[-8:]) > 0


@pytest.mark.parametrize("shift,pooled", [(0, False), (2, True)],
                         ids=["exact_per_request", "bucketed_pooled"])
def test_cache_resolver_in_graph(gpu_lib, shift, pooled):
    """Resolve + attention + merge captured once and replayed per step, with
    the lists changed in place between replays: the cache state follows the
    oracle exactly (the step number lives on the device)."""
    from adaptive_sparse_paged_amd.step import capture
    w = I.custom_workload("cache_graph", 2, 8, 2, ("fixed", 3200), index=123)
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    host, MP = I.build_host_pool(w, 0, lens=lens)
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, MP)
    H, B = w.kv_heads, w.batch
    C = 80 if pooled else 40
    cache = HbmPageCache(dims, host, C, recency_shift=shift, pooled=pooled)
    lists = I.drift_lists(w, I.pages_of(lens[0]), 16, 10, 0.25)
    st = SparseDecodeStep(dims, 0.99, 4, scale=w.scale)
    layer = types.SimpleNamespace(w=w, dims=dims, li=li)
    feed_lists(st, layer, {b * H + h: lists[0, b, h] for b in range(B) for h in range(H)})
    kv, s_page, s_head, ppages = cache.pool_args()

    def step():
        cache.resolve(st.buf.sel_counts, st.buf.sel_pages, st.buf.sel_phys)
        st.attend(li.q, kv, s_page, s_head, ppages, li.ctx_lens)

    say(f"[cache] graph capture of resolve + attention, 10 replays (shift {shift}, pooled {pooled})")
    g = capture(step)
    for t_ in (cache.slot_tag, cache.slot_stamp, cache.unit_slot):
        t_.fill_(-1)
    cache.step_counter.zero_()
    cache.cache_kv.zero_()
    space = H * MP
    states = [O.LRUState(C, B * space)] if pooled else [O.LRUState(C, space) for _ in range(B)]
    for t in range(lists.shape[0]):
        feed_lists(st, layer, {b * H + h: lists[t, b, h] for b in range(B) for h in range(H)})
        g.replay()
        torch.cuda.synchronize()
        replay_out = st.buf.out.clone()
        assert cache.step_counter.item() == t + 1
        if pooled:
            per_req = [[O.pooled_unit(b, h, int(p), H, MP) for h in range(H) for p in lists[t, b, h]]
                       for b in range(B)]
            r = O.resolve_pooled_step(states[0], per_req, t, space, recency_shift=shift)
            assert np.array_equal(cache.slot_tag.cpu().numpy(), states[0].tag), t
            assert np.array_equal(cache.slot_stamp.cpu().numpy(), states[0].stamp), t
            assert np.array_equal(cache.stats.cpu().numpy(), r["per_request"]), t
        else:
            for b in range(B):
                r = O.resolve_step(states[b], [h * MP + int(p) for h in range(H)
                                               for p in lists[t, b, h]], t, recency_shift=shift)
                assert np.array_equal(cache.slot_tag[b].cpu().numpy(), states[b].tag), (t, b)
                assert np.array_equal(cache.slot_stamp[b].cpu().numpy(), states[b].stamp), (t, b)
                assert cache.stats[b].cpu().tolist() == [r["hits"], r["misses"], r["evictions"], 0]
        st.attend(li.q, kv, s_page, s_head, ppages, li.ctx_lens)   # eager, same lists
        torch.cuda.synchronize()
        assert torch.equal(replay_out, st.buf.out)


@pytest.mark.parametrize("shift", [1, 3])
def test_cache_resolver_bucketed_lru(gpu_lib, shift):
    """Bucketed recency (stamps compared in buckets of 2**shift steps, then
    unit id) against the oracle, on lists that drift fast enough to evict."""
    w = I.custom_workload("cache_bucket", 2, 8, 2, ("fixed", 3200), index=124)
    say(f"[cache] bucketed LRU shift {shift}: B=2 Hkv=2, 48 slots, lists of 20, drift 25%")
    stats = _case(w, C=48, list_pages=20, steps=16, drift=0.25, shift=shift)
    assert sum(r["evictions"] for r in stats) > 0


@pytest.mark.parametrize("shift", [0, 2])
def test_cache_pool_shared_by_requests(gpu_lib, shift):
    """One pool of slots for every request, with requests of different list
    lengths (so their slot holdings differ), against the pooled oracle."""
    w = I.custom_workload("cache_pool", 3, 8, 2, ("fixed", 3200), index=125)
    rng = np.random.default_rng(7 + shift)
    steps, H, n = 12, 2, 200
    sizes = [6, 14, 24]                     # pages per list, per request
    L = max(sizes)
    lists = np.full((steps, 3, H, L), -1, dtype=np.int32)
    cur = [[rng.choice(n, size=sizes[b], replace=False) for h in range(H)] for b in range(3)]
    for t in range(steps):
        for b in range(3):
            for h in range(H):
                lists[t, b, h, :sizes[b]] = np.sort(cur[b][h])
                keep = rng.choice(cur[b][h], size=sizes[b] - sizes[b] // 3, replace=False)
                fresh = rng.choice(np.setdiff1d(np.arange(n), keep), size=sizes[b] // 3,
                                   replace=False)
                cur[b][h] = np.concatenate([keep, fresh])
    say(f"[cache] pooled, shift {shift}: 3 requests with lists of {sizes} pages, 100 slots")
    stats = _case(w, C=100, list_pages=0, steps=steps, drift=0.0, workers=5,
                  lists=_ragged(lists, sizes), shift=shift, pooled=True)
    assert sum(r["evictions"] for r in stats) > 0


def _ragged(lists, sizes):
    """Lists of per-request length as an object array [steps][B][H] of arrays."""
    steps, B, H, _ = lists.shape
    out = np.empty((steps, B, H), dtype=object)
    for t in range(steps):
        for b in range(B):
            for h in range(H):
                out[t, b, h] = lists[t, b, h, :sizes[b]]
    return out


@pytest.mark.timeout(300)
def test_cache_resolver_host_tier_full(gpu_lib):
    """The host-tier workload itself: all 16 requests of 524288 tokens, 4096
    slots each, 448-page lists drifting 10%, 256 attention workers (the
    benchmarked shape), 6 steps from cold -- every request's LRU state,
    statistics and slot ids against the oracle at every step, every resident
    slot's bytes, and attention through the cache bit-identical to attention
    over the HBM pool."""
    w = I.WORKLOADS["host_tier_512k"]
    ex = w.extra
    say("[cache] host_tier_512k in full: 16 x 524288 tokens, 4096 slots, 448-page lists")
    stats = _case(w, C=ex["capacity"], list_pages=ex["list_pages"], steps=6, drift=ex["drift"],
                  workers=256)
    assert sum(r["evictions"] for r in stats[-16:]) > 0 and sum(r["hits"] for r in stats[-16:]) > 0


def test_plain_resolve_entry_equals_exact_policy(gpu_lib):
    """sparse_hbm_cache_resolve (no policy argument) is the exact per-request
    LRU: bitwise the same state, statistics, slot ids and slot bytes as
    sparse_hbm_cache_resolve_policy with {0, 0}, step after step."""
    w = I.custom_workload("cache_plain", 2, 8, 2, ("fixed", 1600), index=143)
    say("plain resolve entry: 2 requests, 64 slots, 8 steps")
    lens = I.context_lengths(w)
    li = I.build_layer(w, 0, "cuda", lens=lens)
    host, MP = I.build_host_pool(w, 0, lens=lens)
    dims = lib.make_dims(w.batch, w.q_heads, w.kv_heads, MP)
    C = 64
    a = HbmPageCache(dims, host, C)
    b = HbmPageCache(dims, host, C)
    lists = I.drift_lists(w, min(I.pages_of(L) for L in lens), 40, 8, 0.25)
    B, H = w.batch, w.kv_heads
    st = SparseDecodeStep(dims, 0.99, 8, scale=w.scale)
    layer = types.SimpleNamespace(w=w, dims=dims, li=li)
    for t in range(lists.shape[0]):
        feed_lists(st, layer, {q * H + h: lists[t, q, h] for q in range(B) for h in range(H)})
        phys_b = torch.empty_like(st.buf.sel_phys)
        a.resolve(st.buf.sel_counts, st.buf.sel_pages, st.buf.sel_phys)
        lib.hbm_cache_resolve(dims, st.buf.sel_counts, st.buf.sel_pages, b.host_kv, b.cache_kv,
                              b.capacity, b.slot_tag, b.slot_stamp, b.unit_slot, b.step_counter,
                              phys_b, b.stats, b.ws)
        torch.cuda.synchronize()
        for name in ("slot_tag", "slot_stamp", "unit_slot", "stats", "step_counter", "cache_kv"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (t, name)
        U = B * H
        for u in range(U):
            n = int(st.buf.sel_counts[u].item())
            assert torch.equal(st.buf.sel_phys[u, :n], phys_b[u, :n]), (t, u, "slot ids")
