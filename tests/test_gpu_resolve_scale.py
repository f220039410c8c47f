"""The resolve with its hit pass spread over several workgroups per (request,
KV head): lists longer than one 1024-entry chunk (several workgroups per
list), and enough units that each list's workgroups loop over more than one
chunk.  The resolve alone (sparse_hbm_cache_resolve_split, no pools), with
the step counter advanced between steps as the fetch would: cache state,
statistics, slot ids, hit_phys and the per-unit miss lists against the
oracle's LRU at every step, on drifting lists that overfill the cache (so
victims are chosen) and one request whose step does not fit (overflow)."""

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import lib

from _gpu_case import say

pytestmark = pytest.mark.gpu


def _lists(rng, B, H, MP, sizes, steps, drift):
    """[steps][B][H] sorted distinct page lists; each step keeps all but a
    `drift` share of the previous list and draws the rest afresh."""
    out = np.empty((steps, B, H), dtype=object)
    cur = [[rng.choice(MP, size=sizes[b][h], replace=False) for h in range(H)] for b in range(B)]
    for t in range(steps):
        for b in range(B):
            for h in range(H):
                out[t, b, h] = np.sort(cur[b][h]).astype(np.int32)
                n = sizes[b][h]
                keep = rng.choice(cur[b][h], size=n - int(n * drift), replace=False)
                fresh = rng.choice(np.setdiff1d(np.arange(MP), keep), size=n - keep.size,
                                   replace=False)
                cur[b][h] = np.concatenate([keep, fresh])
    return out


def _run(B, H, MP, C, sizes, steps, drift, seed, shift=0):
    dev = torch.device("cuda")
    dims = lib.make_dims(B, H, H, MP)
    policy = lib.CachePolicy(shift, 0)
    U = B * H
    i32 = dict(dtype=torch.int32, device=dev)
    counts = torch.zeros(U, **i32)
    pages = torch.full((U, MP), -1, **i32)
    phys = torch.full((U, MP), -7, **i32)
    hit = torch.full((U, MP), -7, **i32)
    mc = torch.full((U,), -7, **i32)
    mp = torch.full((U, MP), -7, **i32)
    mx = torch.full((U, MP), -7, **i32)
    tags = torch.full((B, C), -1, **i32)
    stamps = torch.full((B, C), -1, **i32)
    umap = torch.full((B, H * MP), -1, **i32)
    step = torch.zeros(1, **i32)
    stats = torch.zeros((B, 4), **i32)
    ws = torch.zeros(lib.cache_policy_workspace_bytes(dims, policy, C), dtype=torch.uint8,
                     device=dev)
    lists = _lists(np.random.default_rng(seed), B, H, MP, sizes, steps, drift)
    states = [O.LRUState(C, H * MP) for _ in range(B)]
    totals = dict(misses=0, evictions=0, overflow=0)
    for t in range(steps):
        cnt = np.array([len(lists[t, b, h]) for b in range(B) for h in range(H)], np.int32)
        pg = np.full((U, MP), -1, np.int32)
        for u in range(U):
            pg[u, :cnt[u]] = lists[t, u // H, u % H]
        counts.copy_(torch.from_numpy(cnt))
        pages.copy_(torch.from_numpy(pg))
        before = umap.cpu().numpy()
        lib.hbm_cache_resolve_split(dims, policy, counts, pages, C, tags, stamps, umap, step,
                                    phys, hit, stats, ws, miss_lists=(mc, mp, mx))
        step.add_(1)               # what the fetch does after the copies
        torch.cuda.synchronize()
        g_tags, g_stamps, g_umap = tags.cpu().numpy(), stamps.cpu().numpy(), umap.cpu().numpy()
        g_stats, g_phys, g_hit = stats.cpu().numpy(), phys.cpu().numpy(), hit.cpu().numpy()
        g_mc, g_mp, g_mx = mc.cpu().numpy(), mp.cpu().numpy(), mx.cpu().numpy()
        for b in range(B):
            units = [h * MP + int(p) for h in range(H) for p in lists[t, b, h]]
            r = O.resolve_step(states[b], units, t, recency_shift=shift)
            assert np.array_equal(g_tags[b], states[b].tag), (t, b, "tags")
            assert np.array_equal(g_stamps[b], states[b].stamp), (t, b, "stamps")
            assert np.array_equal(g_umap[b], states[b].slot_of), (t, b, "unit map")
            assert g_stats[b].tolist() == [r["hits"], r["misses"], r["evictions"],
                                           r["overflow"]], (t, b, "stats")
            for k in totals:
                totals[k] += r[k]
            for h in range(H):
                u = b * H + h
                lst = lists[t, b, h]
                k = len(lst)
                v = h * MP + lst.astype(np.int64)
                slot = states[b].slot_of[v]
                want = np.where(slot >= 0, b * C + slot, -1)
                assert np.array_equal(g_phys[u, :k], want), (t, u, "slot ids")
                resident = before[b][v] >= 0
                assert np.array_equal(g_hit[u, :k], np.where(resident, want, -1)), (t, u, "hit")
                is_miss = (~resident) & (want >= 0)
                assert g_mc[u] == is_miss.sum(), (t, u, "miss count")
                assert np.array_equal(g_mp[u, :g_mc[u]], lst[is_miss]), (t, u, "miss pages")
                assert np.array_equal(g_mx[u, :g_mc[u]], want[is_miss]), (t, u, "miss slots")
    assert int((ws[:8 * B].view(torch.int64) != 0).sum()) == 0, "ticket words left nonzero"
    return totals


def test_resolve_lists_over_several_chunks(gpu_lib):
    """3 requests x 2 KV heads, 4096-page rows: lists of 1100-3500 pages
    (2-4 workgroups each), 6000 slots; request 2's step holds 7000 units and
    overflows."""
    sizes = [[2500, 2400], [1100, 3000], [3500, 3500]]
    say("[resolve] lists of 1100-3500 pages, 6000 slots, 5 steps, drift 30%")
    tot = _run(3, 2, 4096, 6000, sizes, 5, 0.3, seed=31)
    say(f"  {tot}")
    assert tot["evictions"] > 0 and tot["overflow"] > 0


@pytest.mark.parametrize("shift", [0, 2])
def test_resolve_workgroups_loop_over_chunks(gpu_lib, shift):
    """65 requests x 2 KV heads (130 lists, so 3 workgroups per list) with
    lists of 2000-3500 pages (up to 4 chunks): the first workgroup of a list
    also takes its fourth chunk.  8192 slots, drift 20%."""
    rng = np.random.default_rng(77 + shift)
    sizes = rng.integers(2000, 3501, size=(65, 2)).tolist()
    say(f"[resolve] 130 lists of 2000-3500 pages, 8192 slots, 3 steps, shift {shift}")
    tot = _run(65, 2, 4096, 8192, sizes, 3, 0.2, seed=78 + shift, shift=shift)
    say(f"  {tot}")
    assert tot["misses"] > 0
