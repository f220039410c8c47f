"""The coverage rule against a fixed budget at equal bytes ("Adaptive
DHiSparse: Speculative Decoding over a Load-Adaptive KV Hierarchy", MOIRA
abstract: fixed budgets against the coverage rule; "HiSparse", abstract).

One layer of a workload, either with near-uniform estimated masses (query
strength alpha log-uniform in [0.25, 8]) or with units that range from
concentrated to spread attention (alpha 0.25 or 64 per unit): the coverage
cut at gamma, then the top-k cut with k = the mean of
the coverage counts (the same total pages, so the same KV bytes), both on the
GPU from the same logits, with attention over each list.  Per unit, against
the fp64 oracle:
  - the estimated mass each list keeps (the oracle's page masses),
  - the true attention mass it keeps, exp(lse over the list - dense lse),
    per query head,
  - the output's max-abs distance from dense attention.
Asserted: every coverage list keeps at least gamma of the estimated mass;
the top-k lists read the same total pages up to rounding; and, where the
coverage counts differ between units, some top-k list keeps less than gamma
(a unit whose coverage count exceeds k cannot reach gamma with k pages, the
coverage count being the smallest that does)."""

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib

from _gpu_case import GpuLayer, LIST_EPS, say

pytestmark = pytest.mark.gpu


ALPHAS = {"spread": ("loguniform", 0.25, 8.0), "mixed": ("choice", (0.25, 64.0))}


@pytest.mark.parametrize("gamma", [0.9, 0.99])
@pytest.mark.parametrize("kind", ["spread", "mixed"])
def test_coverage_against_fixed_budget_at_equal_bytes(gpu_lib, kind, gamma):
    w = I.custom_workload("budgets", 4, 16, 4, ("fixed", 8192), alpha=ALPHAS[kind],
                          targets=("uniform", 1, 32), index=144)
    say(f"[budgets] {kind}, gamma {gamma}: 4 requests x 4 KV heads, 512 pages each")
    layer = GpuLayer(w)
    li = layer.li
    B, H, G = w.batch, w.kv_heads, w.group
    U = B * H
    st = layer.step(gamma, 16)
    layer.run(st)
    bf = st.buf
    cov_counts = bf.sel_counts.cpu().numpy().copy()
    cov_pages = bf.sel_pages.cpu().numpy().copy()
    cov_out = bf.out.double().cpu().numpy().copy()
    cov_lse = bf.out_lse.double().cpu().numpy().copy()
    K = int(cov_counts.sum())
    k = max(1, int(round(K / U)))
    lib.select_topk(layer.dims, bf.logits, li.ctx_lens, li.page_table, k, bf.sel_counts,
                    bf.sel_offsets, bf.sel_pages, bf.sel_phys, bf.ws)
    top_out, top_lse = st.attend(li.q, li.kv_pool, layer.stride_page, layer.stride_head,
                                 li.pool_pages, li.ctx_lens)
    torch.cuda.synchronize()
    top_counts = bf.sel_counts.cpu().numpy()
    top_pages = bf.sel_pages.cpu().numpy()
    top_out = top_out.double().cpu().numpy()
    top_lse = top_lse.double().cpu().numpy()
    assert abs(int(top_counts.sum()) - K) <= U // 2 + 1, "not equal bytes"

    rows = []
    for u in range(U):
        b, h = divmod(u, H)
        un = layer.unit_oracle(b, h)
        sel = O.select_unit(un["q"], un["kmin"], un["kmax"], un["nv"], w.scale, gamma)
        m = sel["m"]
        qf = O.bf16_bits_to_f64(un["q"])
        Kf, Vf = O.bf16_bits_to_f64(un["k"]), O.bf16_bits_to_f64(un["v"])
        o_d, l_d = O.dense_unit(qf, Kf, Vf, un["nv"], w.scale)
        r = slice(h * G, (h + 1) * G)
        lc = cov_pages[u, :cov_counts[u]]
        lt = top_pages[u, :top_counts[u]]
        rows.append(dict(
            k_cov=int(cov_counts[u]),
            est_cov=float(m[lc].sum() / m.sum()), est_top=float(m[lt].sum() / m.sum()),
            true_cov=float(np.exp(cov_lse[b, r] - l_d).min()),
            true_top=float(np.exp(top_lse[b, r] - l_d).min()),
            err_cov=float(np.abs(cov_out[b, r] - o_d).max()),
            err_top=float(np.abs(top_out[b, r] - o_d).max())))
    f = lambda key: np.array([x[key] for x in rows])
    say(f"  coverage counts {f('k_cov').min()}..{f('k_cov').max()} (total {K}); top-k k = {k} "
        f"(total {int(top_counts.sum())})")
    for name in ("est", "true", "err"):
        c, t = f(f"{name}_cov"), f(f"{name}_top")
        say(f"  {name:4s}  coverage min {c.min():.4f} mean {c.mean():.4f} max {c.max():.4f} | "
            f"top-k min {t.min():.4f} mean {t.mean():.4f} max {t.max():.4f}")
    below = int((f("est_top") < gamma).sum())
    say(f"  top-k units below gamma (estimated mass): {below} of {U}")
    # the coverage guarantee, within the list acceptance's relative mass bar
    assert np.all(f("est_cov") >= gamma * (1 - LIST_EPS)), "a coverage list below gamma"
    if f("k_cov").min() < f("k_cov").max():
        assert below >= 1, "counts differ but every top-k list reaches gamma"
