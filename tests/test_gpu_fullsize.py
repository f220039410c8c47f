"""Parity at the full workload sizes, in the launch configuration bench.py
times (its per-workload attention chunk): sampled units against the fp64 oracle (regenerated on the
host from the seeded generator), structural properties on every unit, and the
select kernel fed with oracle logits."""

import gc

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I

from _gpu_case import GpuLayer, check_unit, say
from bench import DEFAULT_CHUNK

pytestmark = pytest.mark.gpu


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _structural(layer, st):
    """Properties every unit's list must have, whatever the masses."""
    w = layer.w
    U = w.batch * w.kv_heads
    counts = st.buf.sel_counts.cpu().numpy().astype(np.int64)
    pages = st.buf.sel_pages.cpu().numpy()
    phys = st.buf.sel_phys.cpu().numpy()
    table = layer.li.page_table.cpu().numpy()
    for u in range(U):
        b = u // w.kv_heads
        n = I.pages_of(layer.lens[b])
        k = counts[u]
        assert 1 <= k <= n
        lst = pages[u, :k]
        assert lst[0] >= 0 and lst[-1] < n and np.all(np.diff(lst) > 0)
        assert np.array_equal(phys[u, :k], table[b, lst])
    offs = st.buf.sel_offsets.cpu().numpy()
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)]))
    ch = st.buf.chunk_offsets.cpu().numpy()
    assert np.array_equal(ch, np.concatenate([[0], np.cumsum(-(-counts // st.chunk_pages))]))
    return counts


CASES = [
    ("tiny", 0, 0.99, 0),
    ("llama8b_32k", 0, 0.99, 4),
    ("long_128k", 0, 0.99, 3),
    ("long_128k", 31, 0.98, 2),
    ("serving_b64", 0, 0.99, 4),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,layer_idx,gamma,samples", CASES,
                         ids=[f"{c[0]}_L{c[1]}_g{c[2]}" for c in CASES])
def test_fullsize_sampled(gpu_lib, name, layer_idx, gamma, samples):
    w = I.WORKLOADS[name]
    say(f"[fullsize] {name} layer {layer_idx} gamma {gamma}: generating")
    layer = GpuLayer(w, layer=layer_idx)
    st = layer.step(gamma, DEFAULT_CHUNK.get(name, 256))
    layer.run(st)
    counts = _structural(layer, st)
    say(f"  structural ok; mean kept fraction "
        f"{np.mean(counts / np.repeat([I.pages_of(L) for L in layer.lens], w.kv_heads)):.4f}")
    rng = np.random.default_rng(hash((name, layer_idx)) % 2**32)
    units = [(int(b), int(h)) for b, h in zip(rng.integers(0, w.batch, samples),
                                                  rng.integers(0, w.kv_heads, samples))]
    if name == "serving_b64":   # the shortest and the longest request too
        units += [(int(np.argmin(layer.lens)), 0), (int(np.argmax(layer.lens)), 7)]
    if name == "tiny":          # every unit
        units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    for b, h in units:
        r = check_unit(layer, st, b, h, gamma)
        say(f"  unit ({b},{h}) n={I.pages_of(layer.lens[b])} exact={r['exact']} "
            f"frac={r['frac']:.4f} attn_err={r['attn_err']:.2e} score_err={r['score_err']:.2e}")
    del st, layer
    _free()


@pytest.mark.timeout(400)
def test_host_tier_context_score_select(gpu_lib):
    """524288-token contexts (32768 pages per list): score + select parity."""
    w = I.WORKLOADS["host_tier_512k"]
    say("[fullsize] host_tier_512k: generating 16 x 524288 tokens")
    layer = GpuLayer(w)
    st = layer.step(0.99, 256)          # the whole HBM step at this context, library default
    layer.run(st)
    _structural(layer, st)
    for b, h in [(3, 5), (15, 0)]:
        r = check_unit(layer, st, b, h, 0.99, full=(b == 15))
        say(f"  unit ({b},{h}) exact={r['exact']} frac={r['frac']:.4f} score_err={r['score_err']:.2e}")
    del st, layer
    _free()


def test_select_on_oracle_logits(gpu_lib):
    """The select kernel alone, fed with the oracle's logits rounded to fp32:
    its lists must be the oracle's cut of those same fp32 logits."""
    w = I.custom_workload("sel", 4, 16, 4, ("uniform", 2000, 60000),
                          alpha=("loguniform", 0.25, 8.0), targets=("uniform", 1, 64), index=110)
    layer = GpuLayer(w)
    st = layer.step(0.95, 16)
    li = layer.li
    G = w.group
    xs = {}
    logits = torch.full_like(st.buf.logits, float("nan"))
    for b in range(w.batch):
        for h in range(w.kv_heads):
            un = layer.unit_oracle(b, h)
            sel = O.select_unit(un["q"], un["kmin"], un["kmax"], un["nv"], w.scale, 0.95)
            x32 = sel["x"].astype(np.float32)
            xs[(b, h)] = x32.astype(np.float64)
            logits[b, h, :, :un["n"]] = torch.from_numpy(x32)
    exact = 0
    for gamma in (0.5, 0.9, 0.99, 0.999):
        st.gamma = gamma
        st.buf.logits.copy_(logits)
        from adaptive_sparse_paged_amd import lib
        lib.select_coverage(layer.dims, st.buf.logits, li.ctx_lens, li.page_table, gamma,
                            st.chunk_pages, st.buf.sel_counts, st.buf.sel_offsets,
                            st.buf.chunk_offsets, st.buf.sel_pages, st.buf.sel_phys, st.buf.ws)
        torch.cuda.synchronize()
        for (b, h), x in xs.items():
            m = O.group_mass(O.head_mass(x))
            ref, k, _, _ = O.coverage_cut(m, gamma)
            u = b * w.kv_heads + h
            cnt = int(st.buf.sel_counts[u].item())
            got = st.buf.sel_pages[u, :cnt].cpu().numpy()
            ok, why = O.list_accepted(got, m, gamma, 1e-5)
            assert ok, (b, h, gamma, why, cnt, k)
            exact += int(cnt == k and np.array_equal(got, ref))
    say(f"  exact-match {exact}/{4 * len(xs)}")
    assert exact >= 0.9 * 4 * len(xs)
