"""The coverage cut with several cooperating workgroups per unit
(sparse_select_coverage_coop) and scoring + cut in one cooperative kernel
(sparse_score_select_coverage), against the fp64 oracle on every unit, and
against the one-workgroup selection.  Also: requests shorter than one
member's share of the row (members with no pages), an empty request,
concentrated masses whose fp32 values underflow, gamma = 1, repeated calls
(the workspace is left zeroed, its error word 0), and a graph replay."""

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.step import SparseDecodeStep, capture

from _gpu_case import GpuLayer, check_unit, say
from _oracle_pool import check_every_unit, summarize

pytestmark = pytest.mark.gpu


def _coop_step(layer, gamma, mode):
    return SparseDecodeStep(layer.dims, gamma, scale=layer.w.scale, offsets=False, select=mode)


def _run_select(layer, st):
    li = layer.li
    if st.select == "fused":
        # the fused kernel writes no logits: fill them for the score check
        lib.score_pages(layer.dims, li.q, layer.summ, li.pool_pages, li.page_table,
                        li.ctx_lens, st.scale, st.buf.logits)
    st.score_select(li.q, layer.summ, li.pool_pages, li.page_table, li.ctx_lens)
    torch.cuda.synchronize()


def _ws_clean(st):
    ws = st.coop_ws
    assert int(ws[:4].view(torch.int32)[0].item()) == 0, "a cooperative wait timed out"
    assert int(ws.count_nonzero().item()) == 0, "workspace not left zeroed"


def _lists(st, U):
    c = st.buf.sel_counts.cpu().numpy()[:U].copy()
    p = st.buf.sel_pages.cpu().numpy()
    x = st.buf.sel_phys.cpu().numpy()
    return c, [p[u, :c[u]].copy() for u in range(U)], [x[u, :c[u]].copy() for u in range(U)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,gamma", [("long_128k", 0.99), ("llama8b_32k", 0.99),
                                        ("long_128k", 0.9)])
def test_coop_every_unit_against_oracle_and_single(gpu_lib, name, gamma):
    w = I.WORKLOADS[name]
    say(f"[coop] {name} gamma {gamma}")
    layer = GpuLayer(w)
    U = w.batch * w.kv_heads
    ref = SparseDecodeStep(layer.dims, gamma, scale=w.scale, offsets=False)
    _run_select(layer, ref)
    rc, rp, rx = _lists(ref, U)
    for mode in ("coop", "fused"):
        st = _coop_step(layer, gamma, mode)
        _run_select(layer, st)
        _ws_clean(st)
        c, p, x = _lists(st, U)
        table = layer.li.page_table.cpu().numpy()
        for u in range(U):
            assert np.array_equal(x[u], table[u // w.kv_heads, p[u]])
        same = sum(int(np.array_equal(p[u], rp[u])) for u in range(U))
        s = summarize(check_every_unit(layer, st, gamma))
        say(f"  {mode}: accepted {s['accepted']}/{s['units']}, exact {s['exact']}, "
            f"same lists as the one-workgroup cut {same}/{U}")
        assert not s["bad"], s["bad"]
        assert s["exact"] >= 0.99 * s["units"]
        # attention on the cooperative lists, a sample of units
        st.attend(layer.li.q, layer.li.kv_pool, layer.stride_page, layer.stride_head,
                  layer.li.pool_pages, layer.li.ctx_lens)
        torch.cuda.synchronize()
        for b, h in [(0, 0), (w.batch - 1, w.kv_heads - 1)]:
            check_unit(layer, st, b, h, gamma)


def test_coop_ragged_rows_empty_members_and_empty_request(gpu_lib):
    """Rows of 1875 pages over 8 members of 256 pages: a 63-page request
    leaves seven members without pages, a zero-length request none."""
    w = I.custom_workload("coop_ragged", 3, 8, 2, ("fixed", 30000), alpha=("uniform", 0.5, 6),
                          index=150)
    lens = np.array([30000, 1000, 0])
    layer = GpuLayer(w, lens=lens)
    for mode in ("coop", "fused"):
        st = _coop_step(layer, 0.95, mode)
        _run_select(layer, st)
        _ws_clean(st)
        for h in range(w.kv_heads):
            assert int(st.buf.sel_counts[2 * w.kv_heads + h]) == 0
        for b in (0, 1):
            for h in range(w.kv_heads):
                r = check_unit(layer, st, b, h, 0.95, full=False)
                say(f"  {mode} ({b},{h}) n={I.pages_of(lens[b])} exact={r['exact']}")


def test_coop_concentrated_masses_and_gamma_one(gpu_lib):
    """8192-page rows where 1-3 pages hold nearly all the mass (the others
    more than 100 below in logit, fp32 masses 0), and gamma = 1."""
    B, HQ, HKV, MP = 4, 8, 2, 8192
    G = HQ // HKV
    rng = np.random.default_rng(8193)
    lens = np.array([16 * MP, 16 * MP - 3, 16 * 5000, 16 * 2000], dtype=np.int32)
    n = (lens + 15) // 16
    x = np.full((B, HKV, G, MP), np.nan, dtype=np.float32)
    for b in range(B):
        for h in range(HKV):
            x[b, h, :, :n[b]] = rng.uniform(-160.0, -100.0, size=(G, n[b]))
            k0 = 1 + (b * HKV + h) % 3
            pages = rng.choice(n[b], size=k0, replace=False)
            base = rng.uniform(-2.0, 2.0, size=k0)
            for g in range(G):
                x[b, h, g, pages] = base + rng.uniform(-0.3, 0.3, size=k0)
    pt = np.zeros((B, MP), dtype=np.int32)
    for b in range(B):
        pt[b, :n[b]] = rng.permutation(n[b])
    dims = lib.make_dims(B, HQ, HKV, MP)
    st = SparseDecodeStep(dims, 0.9, scale=1.0, offsets=False, select="coop")
    dev = torch.device("cuda")
    st.buf.logits.copy_(torch.from_numpy(x).to(dev))
    ctx = torch.from_numpy(lens).to(dev)
    table = torch.from_numpy(pt).to(dev)
    for gamma in (0.3, 0.9, 0.9999, 1.0):
        assert lib.select_coverage_coop(dims, st.buf.logits, ctx, table, gamma, st.buf.sel_counts,
                                        st.buf.sel_pages, st.buf.sel_phys, st.coop_ws)
        torch.cuda.synchronize()
        _ws_clean(st)
        counts = st.buf.sel_counts.cpu().numpy()
        pages = st.buf.sel_pages.cpu().numpy()
        for b in range(B):
            for h in range(HKV):
                u = b * HKV + h
                m = O.group_mass(O.head_mass(x[b, h, :, :n[b]].astype(np.float64)))
                ref, k, _, _ = O.coverage_cut(m, gamma)
                got = pages[u, :counts[u]]
                assert counts[u] == k and np.array_equal(got, ref), (gamma, u, counts[u], k)
                assert np.array_equal(st.buf.sel_phys[u, :k].cpu().numpy(), pt[b, got])


def test_coop_repeated_calls_and_graph_replay(gpu_lib):
    """Three calls in a row give the same lists (the workspace is reused and
    left zeroed); the fused step captured in a graph replays the same."""
    w = I.custom_workload("coop_rep", 2, 32, 8, ("uniform", 20000, 40000),
                          alpha=("uniform", 0.5, 6), index=151)
    layer = GpuLayer(w)
    li = layer.li
    U = w.batch * w.kv_heads
    st = _coop_step(layer, 0.97, "fused")
    outs = []
    for _ in range(3):
        st.run(li.q, layer.summ, li.kv_pool, layer.stride_page, layer.stride_head,
               li.pool_pages, li.page_table, li.ctx_lens)
        torch.cuda.synchronize()
        _ws_clean(st)
        outs.append((_lists(st, U), st.buf.out.clone()))
    for o in outs[1:]:
        assert np.array_equal(o[0][0], outs[0][0][0])
        assert all(np.array_equal(a, b) for a, b in zip(o[0][1], outs[0][0][1]))
        assert torch.equal(o[1], outs[0][1])
    g = capture(lambda: st.run(li.q, layer.summ, li.kv_pool, layer.stride_page,
                               layer.stride_head, li.pool_pages, li.page_table, li.ctx_lens))
    for _ in range(3):
        st.buf.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        _ws_clean(st)
        assert torch.equal(st.buf.out, outs[0][1])
