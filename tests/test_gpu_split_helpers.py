"""The two stand-alone helpers of the host tier's split schedule, through the
C ABI: sparse_split_misses against its definition (the list entries placed
this step that were not resident before, in list order), and
sparse_lse_combine against the oracle's attention over the union of two
disjoint page sets (the merge identity of the self-planning attention,
"Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
Hierarchy", MOIRA abstract), with its one-sided and empty cases exact."""

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib

from _gpu_case import ATTN_TOL, GpuLayer, feed_lists, say

pytestmark = pytest.mark.gpu


def _expected_split(counts, pages, phys, hit, max_pages):
    U = counts.shape[0]
    mc = np.zeros(U, dtype=np.int32)
    mp = {}
    for u in range(U):
        n = min(max(int(counts[u]), 0), max_pages)
        keep = [i for i in range(n) if hit[u, i] < 0 and phys[u, i] >= 0]
        mc[u] = len(keep)
        mp[u] = (pages[u, keep], phys[u, keep])
    return mc, mp


@pytest.mark.parametrize("max_pages", [700, 4097])
def test_split_misses_matches_definition(gpu_lib, max_pages):
    say(f"split_misses: max_pages {max_pages}")
    B, HQ, HKV = 4, 8, 2
    U = B * HKV
    dims = lib.make_dims(B, HQ, HKV, max_pages)
    rng = np.random.default_rng(max_pages)
    # empty, one entry, a full row, ragged lengths across workgroup rounds,
    # and lengths outside [0, max_pages] (clamped)
    counts = np.array([0, 1, max_pages, 300, 257, 513, max_pages + 50, -7], dtype=np.int32)[:U]
    pages = rng.integers(0, max_pages, size=(U, max_pages), dtype=np.int32)
    phys = rng.integers(-1, 4096, size=(U, max_pages), dtype=np.int32)
    phys[rng.random((U, max_pages)) < 0.05] = -1
    hit = np.where(rng.random((U, max_pages)) < 0.6, rng.integers(0, 4096, size=(U, max_pages)), -1)
    hit = hit.astype(np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    mc = torch.full((U,), -3, dtype=torch.int32, device="cuda")
    mpg = torch.full((U, max_pages), -3, dtype=torch.int32, device="cuda")
    mph = torch.full((U, max_pages), -3, dtype=torch.int32, device="cuda")
    lib.split_misses(dims, dev(counts), dev(pages), dev(phys), dev(hit), mc, mpg, mph)
    torch.cuda.synchronize()
    exp_c, exp_l = _expected_split(counts, pages, phys, hit, max_pages)
    got_c = mc.cpu().numpy()
    assert np.array_equal(got_c, exp_c)
    gp, gx = mpg.cpu().numpy(), mph.cpu().numpy()
    for u in range(U):
        n = int(exp_c[u])
        assert np.array_equal(gp[u, :n], exp_l[u][0]), f"unit {u} pages"
        assert np.array_equal(gx[u, :n], exp_l[u][1]), f"unit {u} slots"
        # nothing past the count is written
        assert np.all(gp[u, n:] == -3) and np.all(gx[u, n:] == -3), f"unit {u} tail"


def test_lse_combine_against_oracle_union(gpu_lib):
    w = I.custom_workload("lse_combine", 2, 8, 2, ("uniform", 700, 1300), index=142)
    say("lse_combine: 2 requests, 2 KV heads, group 4")
    layer = GpuLayer(w)
    li, dims = layer.li, layer.dims
    B, H, G = w.batch, w.kv_heads, w.group
    rng = np.random.default_rng(7)
    n_of = [I.pages_of(int(L)) for L in layer.lens]
    # unit 0: both sides nonempty; unit 1: A empty; unit 2: B empty; unit 3:
    # both empty
    sides = {}
    for u in range(B * H):
        n = n_of[u // H]
        perm = rng.permutation(n)
        a = np.sort(perm[: n // 3])
        b = np.sort(perm[n // 3: n // 3 + n // 4])
        if u == 1:
            a = a[:0]
        if u == 2:
            b = b[:0]
        if u == 3:
            a, b = a[:0], b[:0]
        sides[u] = (a, b)
    st = layer.step(0.99, workers=16)
    res = {}
    for key, pick in (("a", lambda s: s[0]), ("b", lambda s: s[1]),
                      ("ab", lambda s: np.sort(np.concatenate(s)))):
        feed_lists(st, layer, {u: pick(s) for u, s in sides.items()})
        o, l = st.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages,
                         li.ctx_lens)
        res[key] = (o.clone(), l.clone())
    out = torch.full_like(res["a"][0], 5.0)
    out_lse = torch.full_like(res["a"][1], 5.0)
    lib.lse_combine(dims, res["a"][0], res["a"][1], res["b"][0], res["b"][1], out, out_lse)
    # out may alias out_a
    alias_o, alias_l = res["a"][0].clone(), torch.empty_like(out_lse)
    lib.lse_combine(dims, alias_o, res["a"][1], res["b"][0], res["b"][1], alias_o, alias_l)
    torch.cuda.synchronize()
    assert torch.equal(alias_o, out) and torch.equal(alias_l, out_lse)
    o_gpu, l_gpu = out.double().cpu().numpy(), out_lse.double().cpu().numpy()
    o_ab, l_ab = res["ab"][0].double().cpu().numpy(), res["ab"][1].double().cpu().numpy()
    for u, (a, b) in sides.items():
        bq, h = u // H, u % H
        rows = slice(h * G, (h + 1) * G)
        ra, rb = res["a"], res["b"]
        if len(a) == 0 and len(b) == 0:
            assert np.all(o_gpu[bq, rows] == 0.0) and np.all(np.isneginf(l_gpu[bq, rows]))
            continue
        if len(a) == 0 or len(b) == 0:
            one = rb if len(a) == 0 else ra
            assert torch.equal(out[bq, rows], one[0][bq, rows]), f"unit {u}: one-sided out"
            assert torch.equal(out_lse[bq, rows], one[1][bq, rows]), f"unit {u}: one-sided lse"
        un = layer.unit_oracle(bq, h)
        qf = O.bf16_bits_to_f64(un["q"])
        Kf, Vf = O.bf16_bits_to_f64(un["k"]), O.bf16_bits_to_f64(un["v"])
        o_ref, l_ref = O.attend_pages(qf, Kf, Vf, un["nv"], np.sort(np.concatenate((a, b))), w.scale)
        err = float(np.abs(o_gpu[bq, rows] - o_ref).max())
        lerr = float(np.abs(l_gpu[bq, rows] - l_ref).max())
        # the combined result and one attention over the union: the same
        # tokens, merged in another order
        uerr = float(np.abs(o_gpu[bq, rows] - o_ab[bq, rows]).max())
        say(f"  unit {u}: |A| {len(a)} |B| {len(b)}  vs oracle {err:.2e} (lse {lerr:.2e}), "
            f"vs union attention {uerr:.2e}")
        assert err <= ATTN_TOL and lerr <= ATTN_TOL
        assert uerr <= 1e-5 and float(np.abs(l_gpu[bq, rows] - l_ab[bq, rows]).max()) <= 1e-4
