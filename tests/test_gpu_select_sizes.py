"""The selection at the page-row lengths where its workgroup size changes
(256 threads up to 2048 pages, 512 up to 4096, 1024 above), on seeded fp32
logits, against the oracle's cut of the same logits.  Each size runs ragged
contexts (the full row, a partial tail page, one page, no page) with NaN past
every context (the kernel must mask it) and a unit with exactly tied masses;
coverage lists at three gammas and fixed-budget lists at three budgets, plus
the physical ids and both whole-batch prefix sums."""

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
CHUNK = 16


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


def _check_offsets(st, counts, cap):
    offs = st.buf.sel_offsets.cpu().numpy()
    choffs = st.buf.chunk_offsets.cpu().numpy()
    U = len(counts)
    assert np.array_equal(offs[:U + 1], np.concatenate([[0], np.cumsum(counts)]))
    ch = (np.minimum(counts, cap) + CHUNK - 1) // CHUNK
    assert np.array_equal(choffs[:U + 1], np.concatenate([[0], np.cumsum(ch)]))


@pytest.mark.parametrize("max_pages", [256, 257, 2048, 2049, 4096, 4097])
def test_select_at_workgroup_size_boundaries(gpu_lib, max_pages):
    lens, n, x, pt = _inputs(max_pages, 500 + max_pages)
    dims = lib.make_dims(B, HQ, HKV, max_pages)
    st = SparseDecodeStep(dims, 0.9, CHUNK, scale=1.0)
    dev = torch.device("cuda")
    st.buf.logits.copy_(torch.from_numpy(x).to(dev))
    ctx = torch.from_numpy(lens).to(dev)
    table = torch.from_numpy(pt).to(dev)
    exact = total = 0
    for gamma in (0.5, 0.9, 0.99):
        lib.select_coverage(dims, st.buf.logits, ctx, table, gamma, CHUNK, st.buf.sel_counts,
                            st.buf.sel_offsets, st.buf.chunk_offsets, st.buf.sel_pages,
                            st.buf.sel_phys, st.buf.ws)
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
        _check_offsets(st, counts, max_pages)
    for kp in (1, 37, max_pages):
        lib.select_topk(dims, st.buf.logits, ctx, table, kp, CHUNK, st.buf.sel_counts,
                        st.buf.sel_offsets, st.buf.chunk_offsets, st.buf.sel_pages,
                        st.buf.sel_phys, st.buf.ws)
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
        _check_offsets(st, counts, max_pages)
    say(f"  max_pages {max_pages}: exact-match {exact}/{total}")
    assert exact >= 0.9 * total
