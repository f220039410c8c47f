"""The selection at the page-row lengths where its form changes (256 threads
up to 2048 pages, 512 up to 4096, 1024 above, with 8 pages per thread up to
8192, 16 up to 16384 and 32 up to 32768), on seeded fp32 logits, against the
oracle's cut of the same logits.  Each size runs ragged contexts (the full
row, a partial tail page, one page, no page) with NaN past every context (the
kernel must mask it) and a unit with exactly tied masses; coverage lists at
three gammas and fixed-budget lists at three budgets, plus the physical ids
and the whole-batch prefix sum.  And the concentrated regime: one to three
pages hold nearly all the mass of an 8192-page row, the others sit more than
100 below in logit, so their fp32 masses underflow to zero."""

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.step import SparseDecodeStep

from _gpu_case import say

pytestmark = pytest.mark.gpu

B, HQ, HKV = 4, 8, 2
G = HQ // HKV


def _inputs(max_pages, seed):
    rng = np.random.default_rng(seed)
    lens = np.array([16 * max_pages, 16 * max_pages - 5, 16, 0], dtype=np.int32)
    n = (lens + 15) // 16
    x = rng.normal(0.0, 3.0, size=(B, HKV, G, max_pages)).astype(np.float32)
    # unit (0, 1): every seventh page repeats page 0's logits, so those pages
    # share one mass exactly and the tie rule decides which are kept
    x[0, 1, :, 7::7] = x[0, 1, :, :1]
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    for b in range(B):
        x[b, :, :, n[b]:] = np.nan
        pt[b, :n[b]] = rng.choice(1 << 20, size=n[b], replace=False)
    return lens, n, x, pt


def _masses(x, b, h, n):
    return O.group_mass(O.head_mass(x[b, h, :, :n].astype(np.float64)))


def _check_offsets(st, counts):
    offs = st.buf.sel_offsets.cpu().numpy()
    U = len(counts)
    assert np.array_equal(offs[:U + 1], np.concatenate([[0], np.cumsum(counts)]))


@pytest.mark.parametrize("max_pages", [256, 257, 2048, 2049, 4096, 4097, 8192, 8193, 16384,
                                       16385])
def test_select_at_form_boundaries(gpu_lib, max_pages):
    lens, n, x, pt = _inputs(max_pages, 500 + max_pages)
    dims = lib.make_dims(B, HQ, HKV, max_pages)
    st = SparseDecodeStep(dims, 0.9, 16, scale=1.0)
    dev = torch.device("cuda")
    st.buf.logits.copy_(torch.from_numpy(x).to(dev))
    ctx = torch.from_numpy(lens).to(dev)
    table = torch.from_numpy(pt).to(dev)
    exact = total = 0
    for gamma in (0.5, 0.9, 0.99):
        lib.select_coverage(dims, st.buf.logits, ctx, table, gamma, st.buf.sel_counts,
                            st.buf.sel_offsets, st.buf.sel_pages, st.buf.sel_phys, st.buf.ws)
        torch.cuda.synchronize()
        counts = st.buf.sel_counts.cpu().numpy()[:B * HKV]
        pages = st.buf.sel_pages.cpu().numpy()
        phys = st.buf.sel_phys.cpu().numpy()
        for b in range(B):
            for h in range(HKV):
                u = b * HKV + h
                if n[b] == 0:
                    assert counts[u] == 0, (max_pages, gamma, u)
                    continue
                m = _masses(x, b, h, n[b])
                got = pages[u, :counts[u]]
                ok, why = O.list_accepted(got, m, gamma, 1e-5)
                assert ok, (max_pages, gamma, u, why)
                assert np.array_equal(phys[u, :counts[u]], pt[b, got])
                ref, k, _, _ = O.coverage_cut(m, gamma)
                exact += int(counts[u] == k and np.array_equal(got, ref))
                total += 1
        _check_offsets(st, counts)
    for kp in (1, 37, max_pages):
        lib.select_topk(dims, st.buf.logits, ctx, table, kp, st.buf.sel_counts,
                        st.buf.sel_offsets, st.buf.sel_pages, st.buf.sel_phys, st.buf.ws)
        torch.cuda.synchronize()
        counts = st.buf.sel_counts.cpu().numpy()[:B * HKV]
        pages = st.buf.sel_pages.cpu().numpy()
        for b in range(B):
            for h in range(HKV):
                u = b * HKV + h
                assert counts[u] == min(kp, n[b]), (max_pages, kp, u)
                if n[b] == 0:
                    continue
                m = _masses(x, b, h, n[b])
                got = pages[u, :counts[u]]
                assert np.all(np.diff(got) > 0)
                rest = np.setdiff1d(np.arange(n[b]), got)
                if rest.size:                  # a top set, up to 1e-5 relative mass ties
                    assert m[got].min() * (1 + 1e-5) >= m[rest].max() * (1 - 1e-5)
                exact += int(np.array_equal(got, O.topk_cut(m, kp)))
                total += 1
        _check_offsets(st, counts)
    say(f"  max_pages {max_pages}: exact-match {exact}/{total}")
    # every list passed the predicate above; exact agreement may fail only at
    # fp32 near-ties of the N(0, 3) logits
    assert exact >= 0.9 * total


def test_select_concentrated_mass(gpu_lib):
    """8192-page rows where 1 to 3 pages per unit hold nearly all the mass:
    their logits lie within a few units of each other, every other page's
    logit lies 100 to 160 below (fp32 exp underflows to 0, the fixed-point
    weight of every such page is 0).  The cut keeps k* = 1..3 pages; the lists
    must be the oracle's (fp64 masses of the same fp32 logits, where the cold
    pages keep tiny positive masses)."""
    max_pages = 8192
    rng = np.random.default_rng(8192)
    lens = np.array([16 * max_pages, 16 * max_pages - 3, 16 * 5000, 16 * max_pages],
                    dtype=np.int32)
    n = (lens + 15) // 16
    x = np.full((B, HKV, G, max_pages), np.nan, dtype=np.float32)
    hot = {}
    for b in range(B):
        for h in range(HKV):
            x[b, h, :, :n[b]] = rng.uniform(-160.0, -100.0, size=(G, n[b]))
            k0 = 1 + (b * HKV + h) % 3
            pages = rng.choice(n[b], size=k0, replace=False)
            # hot logits per head: a shared level plus small per-head offsets
            base = rng.uniform(-2.0, 2.0, size=k0)
            for g in range(G):
                x[b, h, g, pages] = base + rng.uniform(-0.3, 0.3, size=k0)
            hot[(b, h)] = np.sort(pages)
    pt = np.zeros((B, max_pages), dtype=np.int32)
    for b in range(B):
        pt[b, :n[b]] = rng.permutation(n[b])
    dims = lib.make_dims(B, HQ, HKV, max_pages)
    st = SparseDecodeStep(dims, 0.9, 16, scale=1.0)
    dev = torch.device("cuda")
    st.buf.logits.copy_(torch.from_numpy(x).to(dev))
    ctx = torch.from_numpy(lens).to(dev)
    table = torch.from_numpy(pt).to(dev)
    kept = []
    for gamma in (0.3, 0.6, 0.9, 0.99, 0.9999):
        lib.select_coverage(dims, st.buf.logits, ctx, table, gamma, st.buf.sel_counts,
                            st.buf.sel_offsets, st.buf.sel_pages, st.buf.sel_phys, st.buf.ws)
        torch.cuda.synchronize()
        counts = st.buf.sel_counts.cpu().numpy()
        pages = st.buf.sel_pages.cpu().numpy()
        for b in range(B):
            for h in range(HKV):
                u = b * HKV + h
                m = _masses(x, b, h, n[b])
                assert m.min() > 0.0           # fp64: no cold page's mass is zero
                got = pages[u, :counts[u]]
                ref, k, _, _ = O.coverage_cut(m, gamma)
                ok, why = O.list_accepted(got, m, gamma, 1e-5)
                assert ok, (gamma, u, why, counts[u], k)
                assert counts[u] == k and np.array_equal(got, ref), (gamma, u, counts[u], k)
                assert 1 <= k <= len(hot[(b, h)]) and set(ref) <= set(hot[(b, h)])
                kept.append(k)
    say(f"  concentrated rows: k* over units and gammas {sorted(set(kept))}")
