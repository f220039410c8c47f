"""Every (request, KV head) unit of a full-size layer against the fp64 oracle,
in a pool of host processes.

The GPU test copies, per unit, what the step produced (the summaries of the
unit's pages, its logits, its page list) to the host; a worker regenerates
the unit's keys and queries from the seeded generator, runs the oracle's
summaries, bound and cut, and reports:
  - summaries bit-exact,
  - every logit within the fp32 summation bound of its oracle value,
  - the list accepted by the coverage predicate (1e-5 relative mass),
  - the list equal to the oracle's (the exact-match rate is aggregated by
    the caller).

Workers are forked (they never touch the GPU) and limited to one thread."""

import multiprocessing as mp
import os

import numpy as np

import oracle as O
from adaptive_sparse_paged_amd import inputs as I

LIST_EPS = 1e-5
POOL_PROCS = 8      # few enough that the test and its workers stay a small process group


def score_tolerance(q_bits, kmin_bits, kmax_bits, scale):
    """Bound on |fp32 logit - exact logit| per (head, page): s * 300 * 2^-24 *
    sum_d |q_d| max(|kmin_d|, |kmax_d|) + 1e-6 -- fp32 summation of 256
    exact bf16 products (two per channel) plus the ln(n_valid) term."""
    qf = np.abs(O.bf16_bits_to_f64(q_bits))
    mag = np.maximum(np.abs(O.bf16_bits_to_f64(kmin_bits)),
                     np.abs(O.bf16_bits_to_f64(kmax_bits)))
    return scale * 300 * 2.0 ** -24 * (qf[:, None, :] * mag[None]).sum(-1) + 1e-6


def _limit_threads():
    import torch
    torch.set_num_threads(1)
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass


def _check(task):
    (w, layer, seed, b, h, L, gamma, summ_gpu, x_gpu, lst) = task
    n = I.pages_of(L)
    k = I.unit_kv_bits(w, layer, b, h, n, 0, seed=seed).numpy()
    q = I.unit_query_bits(w, layer, b, h, L, seed).numpy()
    nv = I.valid_tokens(L)
    kmin, kmax = O.summaries(k, nv)
    del k
    res = {"unit": (b, h), "n": n, "count": int(len(lst))}
    g = summ_gpu.astype(np.int64) & 0xFFFF
    res["summ_ok"] = bool(np.array_equal(g[:, 0], kmin.astype(np.int64)) and
                          np.array_equal(g[:, 1], kmax.astype(np.int64)))
    sel = O.select_unit(q, kmin, kmax, nv, w.scale, gamma)
    err = np.abs(x_gpu.astype(np.float64) - sel["x"])
    res["score_err"] = float(err.max())
    res["score_ok"] = bool(np.all(err <= score_tolerance(q, kmin, kmax, w.scale)))
    ok, why = O.list_accepted(lst, sel["m"], gamma, LIST_EPS)
    res["accepted"], res["why"] = bool(ok), why
    res["oracle_count"] = int(sel["count"])
    res["exact"] = bool(len(lst) == sel["count"] and np.array_equal(lst, sel["list"]))
    return res


def _tasks(layer, st, gamma):
    """One task per unit with a nonempty context, built lazily on the host."""
    w = layer.w
    summ = layer.summ
    table = layer.li.page_table
    counts = st.buf.sel_counts.cpu().numpy()
    for b in range(w.batch):
        L = int(layer.lens[b])
        if L == 0:
            continue
        n = I.pages_of(L)
        phys = table[b, :n].long()
        for h in range(w.kv_heads):
            u = b * w.kv_heads + h
            yield (w, layer.layer, layer.seed, b, h, L, gamma,
                   summ[phys, h].cpu().numpy(),
                   st.buf.logits[b, h, :, :n].cpu().numpy(),
                   st.buf.sel_pages[u, :int(counts[u])].cpu().numpy())


def check_every_unit(layer, st, gamma, procs=POOL_PROCS):
    """Run the per-unit checks over the pool; returns the list of results
    (one dict per unit, in unit order)."""
    ctx = mp.get_context("fork")
    procs = max(1, min(procs, os.cpu_count() or 1))
    with ctx.Pool(procs, initializer=_limit_threads) as pool:
        return list(pool.imap(_check, _tasks(layer, st, gamma), chunksize=1))


def summarize(results):
    """Counts of the checks and the units that failed any of them."""
    bad = [r for r in results
           if not (r["summ_ok"] and r["score_ok"] and r["accepted"])]
    return {
        "units": len(results),
        "exact": sum(r["exact"] for r in results),
        "accepted": sum(r["accepted"] for r in results),
        "max_score_err": max((r["score_err"] for r in results), default=0.0),
        "bad": [(r["unit"], r["why"], r["summ_ok"], r["score_ok"]) for r in bad][:10],
    }
