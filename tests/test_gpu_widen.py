"""GPU parity of the decode-time append (token write + summary refresh) and of
the fixed-budget top-k selection against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib

from _gpu_case import GpuLayer, check_unit, say

pytestmark = pytest.mark.gpu


def test_append_tokens_equals_rebuild(gpu_lib):
    w = I.custom_workload("append", 5, 8, 2, ("fixed", 100), index=130)
    L = np.array([1, 15, 16, 100, 47])           # slot 1, 15, 0 (new page), 4, 15
    say("[append] lengths before", L.tolist())
    full = I.build_layer(w, 0, "cuda", lens=L + 1)  # the pool already holds token L
    H, MP = w.kv_heads, full.max_pages
    dims = lib.make_dims(w.batch, w.q_heads, H, MP)
    sp_, sh_ = 2 * H * 2048, 4096
    pool = full.kv_pool.clone()
    k_new = torch.empty((w.batch, H, 128), dtype=torch.int16)
    v_new = torch.empty((w.batch, H, 128), dtype=torch.int16)
    valid_before = np.zeros(full.pool_pages, dtype=np.int32)
    table = full.page_table.cpu().numpy()
    for b in range(w.batch):
        n1 = I.pages_of(L[b] + 1)
        p, t = divmod(int(L[b]), 16)
        x = int(table[b, p])
        for h in range(H):
            k_new[b, h] = I.unit_kv_bits(w, 0, b, h, n1, 0)[p, t]
            v_new[b, h] = I.unit_kv_bits(w, 0, b, h, n1, 1)[p, t]
            pool[x, h, 0].view(16, 128)[t] = 0x7FC0            # token L unknown before the append
            pool[x, h, 1].view(128, 16)[:, t] = 0x7FC0
        nv = I.valid_tokens(L[b])
        valid_before[table[b, :len(nv)]] = nv
    summ = torch.full((full.pool_pages, H, 2, 128), 0x5A5A, dtype=torch.int16, device="cuda")
    lib.build_page_summaries(dims, pool, sp_, sh_, full.pool_pages,
                             torch.arange(full.pool_pages, dtype=torch.int32, device="cuda"),
                             torch.from_numpy(valid_before).cuda(), summ)
    ctx = torch.from_numpy(L.astype(np.int32)).cuda()
    lib.append_tokens(dims, k_new.cuda(), v_new.cuda(), pool, sp_, sh_, full.pool_pages,
                      full.page_table, ctx, summ)
    torch.cuda.synchronize()
    assert ctx.cpu().tolist() == (L + 1).tolist()
    assert torch.equal(pool, full.kv_pool)                      # bit-exact K and V tiles
    ref = torch.zeros_like(summ)
    lib.build_page_summaries(dims, full.kv_pool, sp_, sh_, full.pool_pages,
                             torch.arange(full.pool_pages, dtype=torch.int32, device="cuda"),
                             full.page_valid, ref)
    torch.cuda.synchronize()
    for b in range(w.batch):
        n1 = I.pages_of(L[b] + 1)
        x = table[b, :n1]
        assert torch.equal(summ[torch.from_numpy(x).long().cuda()],
                           ref[torch.from_numpy(x).long().cuda()])
        for h in range(H):      # and against the oracle's summaries
            k = I.unit_kv_bits(w, 0, b, h, n1, 0).numpy()
            lo, hi = O.summaries(k, I.valid_tokens(L[b] + 1))
            got = summ[torch.from_numpy(x).long().cuda(), h].cpu().numpy().astype(np.int64) & 0xFFFF
            assert np.array_equal(got[:, 0], lo.astype(np.int64))
            assert np.array_equal(got[:, 1], hi.astype(np.int64))


def test_append_then_step_matches_oracle(gpu_lib):
    """The step after an append attends the new token: parity on L + 1."""
    w = I.custom_workload("append2", 3, 8, 2, ("uniform", 200, 900), index=131)
    layer = GpuLayer(w)
    L1 = layer.lens.copy()
    li = layer.li
    H = w.kv_heads
    table = li.page_table.cpu().numpy()
    ctx = torch.from_numpy((L1 - 1).astype(np.int32)).cuda()
    k_new = torch.empty((w.batch, H, 128), dtype=torch.int16)
    v_new = torch.empty((w.batch, H, 128), dtype=torch.int16)
    for b in range(w.batch):
        p, t = divmod(int(L1[b]) - 1, 16)
        n1 = I.pages_of(L1[b])
        for h in range(H):
            k_new[b, h] = I.unit_kv_bits(w, 0, b, h, n1, 0)[p, t]
            v_new[b, h] = I.unit_kv_bits(w, 0, b, h, n1, 1)[p, t]
    lib.append_tokens(layer.dims, k_new.cuda(), v_new.cuda(), li.kv_pool, layer.stride_page,
                      layer.stride_head, li.pool_pages, li.page_table, ctx, layer.summ)
    torch.cuda.synchronize()
    assert torch.equal(ctx.cpu(), li.ctx_lens.cpu())
    st = layer.step(0.95, 8)
    layer.run(st)
    for b in range(w.batch):
        for h in range(H):
            check_unit(layer, st, b, h, 0.95)


def test_topk_select_matches_oracle(gpu_lib):
    w = I.custom_workload("topk", 3, 8, 2, ("uniform", 100, 20000), alpha=("uniform", 0.5, 6),
                          index=132)
    say("[topk] ragged lengths, k in 1, 7, 50, 10000")
    layer = GpuLayer(w)
    li = layer.li
    st = layer.step(0.9, 16)
    layer.run(st)        # logits and the coverage lists
    b_ = st.buf
    oracle = {}
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = layer.unit_oracle(b, h)
            oracle[(b, h)] = O.select_unit(un["q"], un["kmin"], un["kmax"], un["nv"], w.scale, 0.9)
    cov_counts = b_.sel_counts.cpu().numpy().copy()
    cov_pages = b_.sel_pages.cpu().numpy().copy()
    exact = total = 0
    for k in (1, 7, 50, 10000):
        lib.select_topk(layer.dims, b_.logits, li.ctx_lens, li.page_table, k, b_.sel_counts,
                        b_.sel_offsets, b_.sel_pages, b_.sel_phys, b_.ws)
        torch.cuda.synchronize()
        counts = b_.sel_counts.cpu().numpy()
        for (b, h), sel in oracle.items():
            u = b * w.kv_heads + h
            n = len(sel["m"])
            assert counts[u] == min(k, n)
            got = b_.sel_pages[u, :counts[u]].cpu().numpy()
            m = sel["m"]
            assert np.all(np.diff(got) > 0)
            rest = np.setdiff1d(np.arange(n), got)
            if rest.size:                      # a top set, up to 1e-5 relative mass ties
                assert m[got].min() * (1 + 1e-5) >= m[rest].max() * (1 - 1e-5)
            ref = O.topk_cut(m, k)
            exact += int(np.array_equal(got, ref))
            total += 1
    say(f"  top-k exact-match {exact}/{total}")
    # top-k with k = the coverage count reproduces the coverage list
    ks = cov_counts
    for u in range(len(ks)):
        b, h = divmod(u, w.kv_heads)
        lib.select_topk(layer.dims, b_.logits, li.ctx_lens, li.page_table, int(ks[u]),
                        b_.sel_counts, b_.sel_offsets, b_.sel_pages, b_.sel_phys, b_.ws)
        torch.cuda.synchronize()
        got = b_.sel_pages[u, :ks[u]].cpu().numpy()
        assert np.array_equal(got, cov_pages[u, :ks[u]])
