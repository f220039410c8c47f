"""Parity at the full workload sizes, in the launch configuration bench.py
times (the attention's default grid, one workgroup per compute unit).

Every unit of the layer is checked against the fp64 oracle, regenerated on the
host from the seeded generator (a process pool): summaries bit-exact, logits
within the fp32 summation bound, the page list accepted by the coverage
predicate, and the rate of lists equal to the oracle's at least 99%.  The
attention output is compared with exact fp64 attention on the GPU's own list
for a fixed, seeded sample of units (and the shortest and longest requests of
the ragged workload).  Plus structural properties of every list, and the
select kernel fed with the oracle's own logits."""

import gc
import zlib

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib

from _gpu_case import GpuLayer, check_unit, say
from _oracle_pool import check_every_unit, summarize

pytestmark = pytest.mark.gpu

EXACT_RATE = 0.99


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
    return counts


def _every_unit(layer, st, gamma, tag):
    res = check_every_unit(layer, st, gamma)
    s = summarize(res)
    frac = np.mean([r["count"] / r["n"] for r in res])
    say(f"  {tag}: {s['units']} units, accepted {s['accepted']}, exact {s['exact']} "
        f"({s['exact'] / s['units']:.4f}), max score err {s['max_score_err']:.2e}, "
        f"mean kept fraction {frac:.4f}")
    assert not s["bad"], s["bad"]
    assert s["exact"] >= EXACT_RATE * s["units"], s
    return res


def _sample(name, layer_idx, w, k):
    """k units drawn with a seed fixed by the case's name (stable across runs)."""
    rng = np.random.default_rng(zlib.crc32(f"{name}:{layer_idx}".encode()))
    return [(int(b), int(h)) for b, h in zip(rng.integers(0, w.batch, k),
                                               rng.integers(0, w.kv_heads, k))]


CASES = [
    # name, layer, gamma, attention samples (None = every unit)
    ("tiny", 0, 0.99, None),
    ("llama8b_32k", 0, 0.99, 4),
    ("long_128k", 0, 0.99, 3),
    ("long_128k", 31, 0.98, 3),
    ("serving_b64", 0, 0.99, 4),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,layer_idx,gamma,samples", CASES,
                         ids=[f"{c[0]}_L{c[1]}_g{c[2]}" for c in CASES])
def test_fullsize_every_unit(gpu_lib, name, layer_idx, gamma, samples):
    w = I.WORKLOADS[name]
    say(f"[fullsize] {name} layer {layer_idx} gamma {gamma}: generating")
    layer = GpuLayer(w, layer=layer_idx)
    st = layer.step(gamma)                  # workers = 0: one per compute unit, as timed
    layer.run(st)
    _structural(layer, st)
    _every_unit(layer, st, gamma, "every unit")
    if samples is None:
        units = [(b, h) for b in range(w.batch) for h in range(w.kv_heads)]
    else:
        units = _sample(name, layer_idx, w, samples)
    if name == "serving_b64":   # the shortest and the longest request too
        units += [(int(np.argmin(layer.lens)), 0), (int(np.argmax(layer.lens)), 7)]
    for b, h in units:
        r = check_unit(layer, st, b, h, gamma)
        say(f"  attention ({b},{h}) n={I.pages_of(layer.lens[b])} err={r['attn_err']:.2e}")
    del st, layer
    _free()


@pytest.mark.timeout(600)
def test_host_tier_context_every_unit(gpu_lib):
    """524288-token contexts (32768 pages per list, the 32-pages-per-thread
    select form): the whole HBM step, every unit's list against the oracle."""
    w = I.WORKLOADS["host_tier_512k"]
    say("[fullsize] host_tier_512k: generating 16 x 524288 tokens")
    layer = GpuLayer(w)
    st = layer.step(0.99)
    layer.run(st)
    _structural(layer, st)
    _every_unit(layer, st, 0.99, "every unit")
    for b, h in _sample("host_tier_512k", 0, w, 1):
        r = check_unit(layer, st, b, h, 0.99)
        say(f"  attention ({b},{h}) err={r['attn_err']:.2e}")
    del st, layer
    _free()


def test_select_on_oracle_logits(gpu_lib):
    """The select kernel alone, fed with the oracle's logits rounded to fp32:
    its lists must be the oracle's cut of those same fp32 logits."""
    w = I.custom_workload("sel", 4, 16, 4, ("uniform", 2000, 60000),
                          alpha=("loguniform", 0.25, 8.0), targets=("uniform", 1, 64), index=110)
    layer = GpuLayer(w)
    st = layer.step(0.95)
    li = layer.li
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
        st.buf.logits.copy_(logits)
        lib.select_coverage(layer.dims, st.buf.logits, li.ctx_lens, li.page_table, gamma,
                            st.buf.sel_counts, st.buf.sel_offsets, st.buf.sel_pages,
                            st.buf.sel_phys, st.buf.ws)
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
    assert exact >= EXACT_RATE * 4 * len(xs)
