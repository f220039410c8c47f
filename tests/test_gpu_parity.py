"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: summaries bit-exact; page logits within a bound derived from fp32
summation of 256 exact products; page lists accepted by the coverage-rule
predicate under 1e-5 relative mass perturbation (exact match rate reported);
attention outputs within 1e-2 max-abs of exact fp64 attention, both on the
GPU's own lists and on oracle-supplied lists."""


import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib
from adaptive_sparse_paged_amd.step import SparseDecodeStep, capture

from _gpu_case import ATTN_TOL, GpuLayer, check_unit, feed_lists, say

pytestmark = pytest.mark.gpu


def _all_units(layer, st, gamma, full=True):
    w = layer.w
    stats = []
    for b in range(w.batch):
        for h in range(w.kv_heads):
            if layer.lens[b] == 0:
                continue
            stats.append(check_unit(layer, st, b, h, gamma, full=full))
    return stats


SMALL = [
    # name, workload, gamma, attention workers (0 = one per compute unit)
    ("tiny_cfg", I.WORKLOADS["tiny"], 0.99, 0),
    ("ragged_g4", I.custom_workload("ragged_g4", 3, 8, 2, ("uniform", 1, 3000),
                                    alpha=("uniform", 0.5, 6.0), index=101), 0.9, 7),
    ("ragged_g1", I.custom_workload("ragged_g1", 2, 3, 3, ("uniform", 17, 2500),
                                    alpha=("fixed", 4.0), index=102), 0.95, 16),
    ("ragged_g8", I.custom_workload("ragged_g8", 2, 16, 2, ("uniform", 100, 5000),
                                    alpha=("fixed", 8.0), targets=("fixed", 2), index=103), 0.8, 64),
    ("g2_one_worker", I.custom_workload("g2_one_worker", 2, 4, 2, ("fixed", 1000),
                                    alpha=("fixed", 3.0), index=104), 0.5, 1),
    ("gamma1", I.custom_workload("gamma1", 2, 8, 2, ("uniform", 200, 900), index=105), 1.0, 16),
    # G = 16: every column of the matrix-core tiles live, rows of more than
    # 4096 pages (1024-thread selection, four rounds of logit loads)
    ("ragged_g16", I.custom_workload("ragged_g16", 3, 32, 2, ("uniform", 16 * 4097, 16 * 9000),
                                     alpha=("uniform", 1.0, 8.0), index=116), 0.9, 7),
]


@pytest.mark.parametrize("name,w,gamma,workers", SMALL, ids=[s[0] for s in SMALL])
def test_step_parity_small(gpu_lib, name, w, gamma, workers):
    say(f"[parity] {name} B={w.batch} Hq={w.q_heads} Hkv={w.kv_heads} gamma={gamma} "
        f"workers={workers}")
    layer = GpuLayer(w)
    st = layer.step(gamma, workers)
    layer.run(st)
    stats = _all_units(layer, st, gamma)
    ex = np.mean([s["exact"] for s in stats])
    say(f"  exact-match {ex:.3f}  max attn err {max(s['attn_err'] for s in stats):.2e}  "
        f"max score err {max(s['score_err'] for s in stats):.2e}  "
        f"frac {np.mean([s['frac'] for s in stats]):.3f}")
    if gamma >= 1.0:
        assert all(s["frac"] == 1.0 for s in stats)


def test_oracle_lists_through_attention(gpu_lib):
    w = I.custom_workload("olist", 3, 8, 2, ("uniform", 30, 4000), alpha=("uniform", 1, 6),
                          index=106)
    layer = GpuLayer(w)
    say("[oracle-lists] building lists")
    lists, refs = {}, {}
    rng = np.random.default_rng(5)
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = layer.unit_oracle(b, h)
            sel = O.select_unit(un["q"], un["kmin"], un["kmax"], un["nv"], w.scale, 0.9)
            lst = sel["list"]
            if (b + h) % 3 == 2:   # also arbitrary (non-top) lists: the kernel attends any list
                lst = np.sort(rng.choice(un["n"], size=max(1, un["n"] // 3), replace=False))
            u = b * w.kv_heads + h
            lists[u] = lst
            qf = O.bf16_bits_to_f64(un["q"])
            refs[u] = O.attend_pages(qf, O.bf16_bits_to_f64(un["k"]), O.bf16_bits_to_f64(un["v"]),
                                     un["nv"], lst, w.scale)
    for workers in (1, 5, 32, 0):
        st = layer.step(0.9, workers)
        feed_lists(st, layer, lists)
        li = layer.li
        st.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages,
                  li.ctx_lens)
        torch.cuda.synchronize()
        G = w.group
        worst = 0.0
        for u, (o_ref, lse_ref) in refs.items():
            b, h = divmod(u, w.kv_heads)
            o = st.buf.out[b, h * G:(h + 1) * G].double().cpu().numpy()
            lse = st.buf.out_lse[b, h * G:(h + 1) * G].double().cpu().numpy()
            worst = max(worst, float(np.abs(o - o_ref).max()))
            assert np.abs(lse - lse_ref).max() < 1e-3
        say(f"  workers {workers}: max attn err {worst:.2e}")
        assert worst <= ATTN_TOL


def test_summaries_signed_zero_and_tails(gpu_lib):
    say("[summaries] signed zeros, tails")
    rng = np.random.default_rng(9)
    Pp, H = 37, 3
    vals = rng.standard_normal((Pp, H, 16, 128))
    vals[0, 0, :, :4] = 0.0
    vals[0, 0, 5, :2] = -0.0
    vals[1, 1, :, 7] = -0.0
    tiles = O.f64_to_bf16_bits(vals).astype(np.int16)
    valid = rng.integers(0, 17, size=Pp).astype(np.int32)
    valid[:2] = 16
    pool = np.zeros((Pp, H, 2, 2048), dtype=np.int16)
    pool[:, :, 0] = tiles.reshape(Pp, H, 2048)
    pool[:, :, 1] = 0x7FC0          # V holds NaN patterns: summaries never read V
    d = lib.make_dims(1, H, H, 4)
    summ = torch.full((Pp, H, 2, 128), 0x1234, dtype=torch.int16, device="cuda")
    lib.build_page_summaries(d, torch.from_numpy(pool).cuda(), H * 4096, 4096, Pp,
                             torch.arange(Pp, dtype=torch.int32, device="cuda"),
                             torch.from_numpy(valid).cuda(), summ)
    torch.cuda.synchronize()
    got = summ.cpu().numpy().astype(np.int64) & 0xFFFF
    for x in range(Pp):
        for h in range(H):
            if valid[x] == 0:
                assert np.all(got[x, h] == 0x1234)
                continue
            lo, hi = O.summaries(tiles[x, h][None], [valid[x]])
            assert np.array_equal(got[x, h, 0], lo[0].astype(np.int64))
            assert np.array_equal(got[x, h, 1], hi[0].astype(np.int64))
    assert got[0, 0, 0, 0] == 0x8000 and got[0, 0, 1, 0] == 0x0000


def test_zero_length_request_and_single_token(gpu_lib):
    w = I.custom_workload("zl", 3, 8, 2, ("fixed", 100), index=107)
    lens = np.array([1, 0, 333])
    say("[edge] lengths", lens.tolist())
    layer = GpuLayer(w, lens=lens)
    st = layer.step(0.99, 4)
    layer.run(st)
    G = w.group
    for h in range(w.kv_heads):
        u = 1 * w.kv_heads + h
        assert st.buf.sel_counts[u].item() == 0
        assert torch.all(st.buf.out[1, h * G:(h + 1) * G] == 0)
        assert torch.all(torch.isneginf(st.buf.out_lse[1, h * G:(h + 1) * G]))
    for b in (0, 2):
        for h in range(w.kv_heads):
            check_unit(layer, st, b, h, 0.99)
    # one token: o = v_0 exactly up to rounding
    un = layer.unit_oracle(0, 0)
    v0 = O.bf16_bits_to_f64(un["v"][0, 0])
    assert np.abs(st.buf.out[0, 0].double().cpu().numpy() - v0).max() < 1e-6
    offs = st.buf.sel_offsets.cpu().numpy()
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(st.buf.sel_counts.cpu().numpy())]))


def test_request_without_valid_pages(gpu_lib):
    """A request whose page-table row holds no page of the pool: every one of
    its logits is -inf, its per-head normalisers are empty, and the selection
    must not turn that into NaN masses.  It keeps one (empty) page, its
    attention sees no token (output 0, lse -inf), and the other requests are
    unaffected."""
    w = I.custom_workload("nopages", 3, 8, 2, ("fixed", 700), index=110)
    say("[edge] request 1 with every page id out of range")
    layer = GpuLayer(w)
    li = layer.li
    li.page_table[1].fill_(-1)
    st = layer.step(0.95, 8)
    layer.run(st)
    G = w.group
    assert not torch.isnan(st.buf.out).any() and not torch.isnan(st.buf.out_lse).any()
    for h in range(w.kv_heads):
        u = 1 * w.kv_heads + h
        assert st.buf.sel_counts[u].item() == 1
        assert torch.all(st.buf.sel_phys[u, :1] == -1)
        assert torch.all(st.buf.out[1, h * G:(h + 1) * G] == 0)
        assert torch.all(torch.isneginf(st.buf.out_lse[1, h * G:(h + 1) * G]))
    for b in (0, 2):
        for h in range(w.kv_heads):
            check_unit(layer, st, b, h, 0.95)


def test_graph_replay_after_inputs_change(gpu_lib):
    """The whole step captured once, replayed after the queries and context
    lengths change in place: every replay equals the eager step bitwise, and
    the replayed lists and outputs match the oracle on the new inputs."""
    w = I.custom_workload("graph", 4, 8, 2, ("uniform", 500, 6000), alpha=("uniform", 1, 8),
                          index=108)
    say("[graph] capture and replay")
    layer = GpuLayer(w)
    st = layer.step(0.95, 16)
    li = layer.li
    g = capture(lambda: st.run(li.q, layer.summ, li.kv_pool, layer.stride_page,
                               layer.stride_head, li.pool_pages, li.page_table, li.ctx_lens))
    g.replay()
    torch.cuda.synchronize()
    ref1 = st.buf.out.clone()
    layer.run(st)
    assert torch.equal(st.buf.out, ref1)
    # new inputs in place: fresh queries and shorter contexts (shortened to
    # whole pages, so the summaries built for the original lengths still hold)
    other = I.custom_workload("graph", 4, 8, 2, ("uniform", 500, 6000), alpha=("uniform", 1, 8),
                              index=109)
    new_lens = np.minimum(layer.lens, np.array([4000, 304, 5984, 16]))
    for b in range(w.batch):
        for h in range(w.kv_heads):
            li.q[b, h * w.group:(h + 1) * w.group] = I.unit_query_bits(other, 0, b, h, int(new_lens[b])).cuda()
    li.ctx_lens.copy_(torch.from_numpy(new_lens.astype(np.int32)))
    for rep in range(3):
        st.buf.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        replay_out = st.buf.out.clone()
        replay_counts = st.buf.sel_counts.clone()
        layer.run(st)                          # eager on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(replay_out, st.buf.out)
        assert torch.equal(replay_counts, st.buf.sel_counts)
    assert not torch.equal(st.buf.out, ref1)
    # the replayed step against the oracle on the new inputs
    st.buf.out.zero_()
    g.replay()
    torch.cuda.synchronize()
    layer.lens = new_lens
    cache = {}
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = layer.unit_oracle(b, h)
            un["q"] = I.unit_query_bits(other, 0, b, h, int(new_lens[b])).numpy()
            cache[(b, h)] = un
    layer.oracle_cache = cache
    stats = _all_units(layer, st, 0.95)
    say(f"  replay vs oracle: exact {sum(r['exact'] for r in stats)}/{len(stats)}, "
        f"max attn err {max(r['attn_err'] for r in stats):.2e}")


def test_deterministic(gpu_lib):
    w = I.WORKLOADS["tiny"]
    layer = GpuLayer(w)
    st = layer.step(0.99, 8)
    layer.run(st)
    a = (st.buf.out.clone(), st.buf.sel_pages.clone(), st.buf.logits.clone())
    layer.run(st)
    assert torch.equal(a[0], st.buf.out) and torch.equal(a[1], st.buf.sel_pages)
    assert torch.equal(a[2], st.buf.logits)


@pytest.mark.parametrize("offsets", [True, False], ids=["offsets", "no_offsets"])
def test_grouped_streams_match_single_stream(gpu_lib, offsets):
    """Request groups on separate streams (selection of one group under the
    attention of another) give bitwise the same lists, and the same outputs
    up to the order of the log-sum-exp merge (each group's attention splits
    its own lists over the workgroups), eagerly and replayed from a graph;
    with and without the per-group prefix sums of the counts."""
    w = I.custom_workload("groups", 5, 8, 2, ("uniform", 300, 9000), alpha=("uniform", 1, 6),
                          index=111)
    say(f"[groups] 5 requests in 3 stream groups, offsets={offsets}")
    layer = GpuLayer(w)
    li = layer.li
    ref = layer.step(0.97, 16)
    layer.run(ref)
    grp = SparseDecodeStep(layer.dims, 0.97, 16, scale=w.scale, groups=3, offsets=offsets)
    args = (li.q, layer.summ, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages,
            li.page_table, li.ctx_lens)
    grp.run(*args)
    torch.cuda.synchronize()
    assert torch.equal(grp.buf.sel_counts, ref.buf.sel_counts)
    for u in range(w.batch * w.kv_heads):
        k = int(ref.buf.sel_counts[u])
        assert torch.equal(grp.buf.sel_pages[u, :k], ref.buf.sel_pages[u, :k])
    close = lambda a, b: float((a - b).abs().max()) <= 1e-5
    assert close(grp.buf.out, ref.buf.out) and close(grp.buf.out_lse, ref.buf.out_lse)
    eager = grp.buf.out.clone()
    g = capture(lambda: grp.run(*args))
    for _ in range(3):
        grp.buf.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(grp.buf.out, eager)


def test_list_bound_clamps_lists(gpu_lib):
    """dims' max_list_pages clamps every list: with a bound at the longest
    list the outputs are bitwise those without a bound; with a smaller bound
    each unit attends the first `bound` entries of its list only."""
    w = I.custom_workload("bound", 3, 8, 2, ("fixed", 20000), index=113)
    say("[bound] 3 x 20000 tokens (1250 pages per row), lists of up to 40 pages")
    layer = GpuLayer(w)
    rng = np.random.default_rng(17)
    n = I.pages_of(20000)
    lists = {u: np.sort(rng.choice(n, size=int(rng.integers(1, 41)), replace=False))
             for u in range(w.batch * w.kv_heads)}
    li = layer.li
    outs = {}
    for bound in (0, 40, 9):
        d = lib.make_dims(w.batch, w.q_heads, w.kv_heads, li.max_pages, max_list_pages=bound)
        st = SparseDecodeStep(d, 0.9, 8, scale=w.scale)
        feed_lists(st, layer, lists)
        st.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages,
                  li.ctx_lens)
        torch.cuda.synchronize()
        outs[bound] = (st.buf.out.clone(), st.buf.out_lse.clone())
    assert torch.equal(outs[0][0], outs[40][0]) and torch.equal(outs[0][1], outs[40][1])
    G = w.group
    for u, lst in lists.items():
        b, h = divmod(u, w.kv_heads)
        un = layer.unit_oracle(b, h)
        args = (O.bf16_bits_to_f64(un["q"]), O.bf16_bits_to_f64(un["k"]),
                O.bf16_bits_to_f64(un["v"]), un["nv"])
        for bound, part in ((40, lst), (9, lst[:9])):
            o_ref, _ = O.attend_pages(*args, part, w.scale)
            o = outs[bound][0][b, h * G:(h + 1) * G].double().cpu().numpy()
            assert np.abs(o - o_ref).max() <= ATTN_TOL, (u, bound)


def test_concentrated_query_end_to_end(gpu_lib):
    """The whole step where 1 to 3 pages of an 8192-page row hold nearly all
    the attention mass: every query head of a unit is the same +-1 pattern p,
    and the keys of the unit's hot pages are c_i * p with c_i = 16, 15.875,
    15.75 (exact in bf16), so the hot pages' logits sit about 160 above the
    others' (whose fp32 masses underflow) and about 1.4 apart from each other.
    Summaries are rebuilt for the changed pages; the oracle sees the same
    keys and queries.  Lists, scores and attention are checked per unit."""
    w = I.custom_workload("hot", 2, 8, 2, ("fixed", 16 * 8192 - 5), index=118)
    say("[concentrated] 2 x 8192 pages, 1-3 hot pages per unit")
    layer = GpuLayer(w)
    li = layer.li
    rng = np.random.default_rng(118)
    G, n = w.group, I.pages_of(16 * 8192 - 5)
    table = li.page_table.cpu().numpy()
    cache = {}
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = layer.unit_oracle(b, h)
            sign = rng.choice([-1.0, 1.0], size=128)
            pbits = O.f64_to_bf16_bits(sign).astype(np.int16)
            un["q"] = np.tile(pbits, (G, 1))
            li.q[b, h * G:(h + 1) * G] = torch.from_numpy(un["q"]).cuda()
            hot = rng.choice(n - 1, size=1 + (b * w.kv_heads + h) % 3, replace=False)
            for i, p in enumerate(hot):
                rows = O.f64_to_bf16_bits(np.tile((16.0 - 0.125 * i) * sign, (16, 1)))
                un["k"][p] = rows.astype(un["k"].dtype)
                li.kv_pool[int(table[b, p]), h, 0] = torch.from_numpy(
                    rows.astype(np.int16).reshape(-1)).cuda()
            un["kmin"], un["kmax"] = O.summaries(un["k"], un["nv"])
            cache[(b, h)] = un
    layer.oracle_cache = cache
    pages = torch.arange(li.pool_pages, dtype=torch.int32, device="cuda")
    lib.build_page_summaries(layer.dims, li.kv_pool, layer.stride_page, layer.stride_head,
                             li.pool_pages, pages, li.page_valid, layer.summ)
    for gamma in (0.5, 0.9, 0.99):
        st = layer.step(gamma)
        layer.run(st)
        stats = _all_units(layer, st, gamma)
        counts = [int(st.buf.sel_counts[u]) for u in range(w.batch * w.kv_heads)]
        say(f"  gamma {gamma}: k* {counts}, exact {sum(s['exact'] for s in stats)}/{len(stats)}, "
            f"max attn err {max(s['attn_err'] for s in stats):.2e}")
        assert all(s["exact"] for s in stats)
        assert 1 <= min(counts) and max(counts) <= 3


def test_attn_merge_in_one_call_equals_two_calls(gpu_lib):
    """sparse_decode_attn_merge runs the same kernels as sparse_decode_attn
    followed by sparse_merge_splits: bitwise the same outputs."""
    w = I.custom_workload("one_call", 3, 8, 2, ("uniform", 20, 9000), alpha=("uniform", 1, 6),
                          index=119)
    layer = GpuLayer(w)
    li = layer.li
    for workers in (1, 7, 0):
        st = layer.step(0.9, workers)
        st.score_select(li.q, layer.summ, li.pool_pages, li.page_table, li.ctx_lens)
        st.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages,
                  li.ctx_lens)                      # the one-call path
        torch.cuda.synchronize()
        one = (st.buf.out.clone(), st.buf.out_lse.clone())
        out2, lse2 = torch.empty_like(one[0]), torch.empty_like(one[1])
        lib.decode_attn(layer.dims, li.q, li.kv_pool, layer.stride_page, layer.stride_head,
                        li.pool_pages, li.ctx_lens, st.buf.sel_counts, st.buf.sel_pages,
                        st.buf.sel_phys, st.scale, workers, st.buf.part_o, st.buf.part_lse,
                        st.max_parts)
        lib.merge_splits(layer.dims, st.buf.part_o, st.buf.part_lse, st.buf.sel_counts, workers,
                         out2, lse2)
        torch.cuda.synchronize()
        assert torch.equal(one[0], out2) and torch.equal(one[1], lse2), workers


def test_out_of_range_ids_inside_lists(gpu_lib):
    """Physical ids outside the pool in the middle of otherwise valid lists
    (-1, a negative id, exactly pool_pages, far past it), and one unit whose
    every entry is out of range: each such entry reads as an empty page, so
    the outputs equal attention over the same lists with those entries
    removed, and nothing is NaN."""
    w = I.custom_workload("bad_ids", 3, 16, 4, ("uniform", 3000, 9000), index=117)
    say("[edge] out-of-range physical ids inside lists")
    layer = GpuLayer(w)
    li = layer.li
    H = w.kv_heads
    U = w.batch * H
    rng = np.random.default_rng(117)
    lens = li.ctx_lens.cpu().numpy()
    lists = {}
    for u in range(U):
        n = I.pages_of(int(lens[u // H]))
        lists[u] = np.sort(rng.choice(n, size=int(rng.integers(1, min(n, 150) + 1)),
                                      replace=False)).astype(np.int32)
    bad_vals = [-1, -12345, int(li.pool_pages), int(li.pool_pages) + 100000]
    st = layer.step(0.99, 12)
    ref = layer.step(0.99, 12)
    feed_lists(st, layer, lists)
    phys = st.buf.sel_phys.cpu().numpy()
    keep = {}
    for u in range(U):
        k = len(lists[u])
        if u == U - 2:
            bad = np.arange(k)                       # every entry out of range
        else:
            bad = rng.choice(k, size=min(k, int(rng.integers(0, 6))), replace=False)
        for i in bad:
            phys[u, i] = bad_vals[int(rng.integers(0, len(bad_vals)))]
        mask = np.ones(k, bool)
        mask[bad] = False
        keep[u] = lists[u][mask]
    st.buf.sel_phys.copy_(torch.from_numpy(phys))
    args = (li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages, li.ctx_lens)
    o, l = st.attend(*args)
    o, l = o.clone(), l.clone()
    feed_lists(ref, layer, keep)
    o_ref, l_ref = ref.attend(*args)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(l).any()
    fin = torch.isfinite(l_ref)
    assert torch.equal(fin, torch.isfinite(l))
    assert float((o - o_ref).abs().max()) <= 1e-5
    assert float((l[fin] - l_ref[fin]).abs().max()) <= 1e-5
    b, h = divmod(U - 2, H)
    G = w.group
    assert torch.all(o[b, h * G:(h + 1) * G] == 0)
    assert torch.all(torch.isneginf(l[b, h * G:(h + 1) * G]))
