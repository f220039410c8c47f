"""Pins of the fp64 oracle against things other than itself: hand-derived
closed forms (tests/golden), brute force over tiny inputs, invariants, special
cases that reduce to textbook results, and library routines."""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261202)


def _bits(x):
    return O.f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


# ---------------------------------------------------------------- bf16 codec

def test_bf16_roundtrip_all_patterns():
    b = np.arange(65536, dtype=np.int64)
    with np.errstate(invalid="ignore"):      # the NaN patterns (signalling ones warn on cast)
        f = O.bf16_bits_to_f64(b)
    ok = ~np.isnan(f)
    assert np.array_equal(O.f64_to_bf16_bits(f[ok]).astype(np.int64), b[ok])


def test_bf16_ties_to_even_and_torch():
    import torch
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert O.f64_to_bf16_bits(1 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6 -> even mantissa (0x3F82)
    assert O.f64_to_bf16_bits(1 + 3 * 2.0 ** -8) == 0x3F82
    x = RNG.standard_normal(100000).astype(np.float32)   # exact in fp32
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    assert np.array_equal(O.f64_to_bf16_bits(x.astype(np.float64)).astype(np.int64), ref)


# ---------------------------------------------------------------- summaries

def _brute_summary(tile, nv):
    P, D = tile.shape
    vals = O.bf16_bits_to_f64(tile)
    kmin = np.zeros(D, dtype=np.int64)
    kmax = np.zeros(D, dtype=np.int64)
    for d in range(D):
        best_lo = best_hi = None
        for t in range(nv):
            v = vals[t, d]
            b = int(tile[t, d]) & 0xFFFF
            key = (v, math.copysign(1.0, v))      # -0 sorts below +0
            if best_lo is None or key < best_lo[0]:
                best_lo = (key, b)
            if best_hi is None or key > best_hi[0]:
                best_hi = (key, b)
        kmin[d], kmax[d] = best_lo[1], best_hi[1]
    return kmin, kmax


def test_summaries_brute_force_with_tail_and_signed_zero():
    n, P, D = 6, 16, 8
    vals = RNG.standard_normal((n, P, D))
    vals[0, :, 0] = 0.0
    vals[0, 3, 0] = -0.0                 # signed zero decides kmin
    vals[1, :, 1] = 1.5                  # all equal
    tiles = _bits(vals)
    nv = np.array([16, 16, 1, 7, 16, 3])
    tiles[3, 7:] = _bits(1e30)           # garbage beyond the valid tokens
    tiles[5, 3:] = _bits(-1e30)
    lo, hi = O.summaries(tiles, nv)
    for p in range(n):
        blo, bhi = _brute_summary(tiles[p], nv[p])
        assert np.array_equal(lo[p].astype(np.int64), blo)
        assert np.array_equal(hi[p].astype(np.int64), bhi)
    assert lo[0, 0] == 0x8000 and hi[0, 0] == 0x0000


# ---------------------------------------------------------------- bound

def test_bound_dominates_true_max_logit():
    n, P, D, G = 40, 16, 128, 4
    K = O.bf16_bits_to_f64(_bits(RNG.standard_normal((n, P, D))))
    q = O.bf16_bits_to_f64(_bits(RNG.standard_normal((G, D))))
    nv = RNG.integers(1, P + 1, size=n)
    lo, hi = O.summaries(_bits(K), nv)
    u = O.bound(q, O.bf16_bits_to_f64(lo), O.bf16_bits_to_f64(hi))
    for p in range(n):
        true = q @ K[p, :nv[p]].T                      # [G][nv]
        slack = 1e-12 * np.abs(q[:, None, :] * K[p, None, :nv[p], :]).sum(-1).max()
        assert np.all(u[:, p] >= true.max(axis=1) - slack)


def test_bound_brute_force_loops():
    G, n, D = 2, 3, 5
    q = RNG.standard_normal((G, D))
    a = RNG.standard_normal((n, D))
    b = a + np.abs(RNG.standard_normal((n, D)))
    u = O.bound(q, a, b)
    for g in range(G):
        for p in range(n):
            s = 0.0
            for d in range(D):
                s += max(q[g, d] * a[p, d], q[g, d] * b[p, d])
            assert abs(u[g, p] - s) <= 1e-12


def test_bound_special_cases():
    D, n = 16, 7
    k = RNG.standard_normal((n, D))
    q = RNG.standard_normal((3, D))
    # identical keys: kmin = kmax = k -> u = q.k exactly
    assert np.allclose(O.bound(q, k, k), q @ k.T, rtol=0, atol=1e-12)
    lo = k - np.abs(RNG.standard_normal((n, D)))
    hi = k + np.abs(RNG.standard_normal((n, D)))
    qp = np.abs(q)
    assert np.allclose(O.bound(qp, lo, hi), qp @ hi.T, atol=1e-12)      # q >= 0
    assert np.allclose(O.bound(-qp, lo, hi), -qp @ lo.T, atol=1e-12)    # q <= 0


# ---------------------------------------------------------------- masses

def test_mass_sums_to_one_and_is_exact_for_constant_pages():
    G, D, n, P = 4, 32, 24, 16
    keys = O.bf16_bits_to_f64(_bits(RNG.standard_normal((n, D))))
    q = O.bf16_bits_to_f64(_bits(RNG.standard_normal((G, D)) * 2))
    nv = RNG.integers(1, P + 1, size=n)
    s = 1 / math.sqrt(D)
    u = O.bound(q, keys, keys)
    x = O.page_logits(u, nv, s)
    pi = O.head_mass(x)
    m = O.group_mass(pi)
    assert abs(m.sum() - 1) < 1e-12
    # exact attention over every token; every token of page p has key keys[p]
    tok_keys = np.repeat(keys, nv, axis=0)
    tok_page = np.repeat(np.arange(n), nv)
    logits = s * q @ tok_keys.T
    w = np.exp(logits - logsumexp(logits, axis=1, keepdims=True))
    exact = np.stack([np.bincount(tok_page, weights=w[g], minlength=n) for g in range(G)])
    assert np.allclose(pi, exact, rtol=1e-12, atol=1e-15)
    assert np.allclose(m, exact.mean(0), rtol=1e-12, atol=1e-15)


def test_golden_worked_example_masses_cuts_attention():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    s = math.log(2.0)
    q = np.array(ex["q"])
    nv = np.array([p["valid"] for p in ex["pages"]])
    key = np.array([p["key"] for p in ex["pages"]])
    val = np.array([p["value"] for p in ex["pages"]])
    n, D = key.shape
    K = np.zeros((n, 16, D))
    V = np.zeros((n, 16, D))
    for p in range(n):
        K[p, :] = key[p]
        V[p, :] = val[p]
        K[p, nv[p]:] = 99.0            # invalid tokens must be ignored
        V[p, nv[p]:] = -99.0
    lo, hi = O.summaries(_bits(K), nv)
    u = O.bound(q, O.bf16_bits_to_f64(lo), O.bf16_bits_to_f64(hi))
    m = O.group_mass(O.head_mass(O.page_logits(u, nv, s)))
    expect = np.array(ex["mass_num"]) / ex["mass_den"]
    assert np.allclose(m, expect, rtol=1e-13, atol=0)
    for g_str, lst in ex["cuts"].items():
        got, k, _, _ = O.coverage_cut(m, float(g_str))
        assert got.tolist() == lst and k == len(lst)
    o, lse = O.dense_unit(q, K, V, nv, s)
    eo = np.array([[a / b for a, b in row] for row in ex["dense"]["o"]])
    assert np.allclose(o, eo, atol=1e-13)
    assert np.allclose(lse, np.log(ex["dense"]["lse_of"]), atol=1e-13)
    o, lse = O.attend_pages(q, K, V, nv, [0, 1, 3], s)
    eo = np.array([[a / b for a, b in row] for row in ex["subset_013"]["o"]])
    assert np.allclose(o, eo, atol=1e-13)
    assert np.allclose(lse, np.log(ex["subset_013"]["lse_of"]), atol=1e-13)


def test_select_unit_on_the_worked_example():
    """select_unit (bound, page logits, masses, cut in one call, from bf16
    bits) gives the hand-derived masses and cuts of the worked example."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    s = math.log(2.0)
    q = np.array(ex["q"], dtype=np.float64)
    nv = np.array([p["valid"] for p in ex["pages"]])
    key = np.array([p["key"] for p in ex["pages"]], dtype=np.float64)
    expect = np.array(ex["mass_num"]) / ex["mass_den"]
    for g_str, lst in ex["cuts"].items():
        sel = O.select_unit(_bits(q), _bits(key), _bits(key), nv, s, float(g_str))
        assert sel["list"].tolist() == lst and sel["count"] == len(lst)
        assert np.allclose(sel["m"], expect, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- the cut

def test_golden_dyadic_cuts():
    with open(os.path.join(GOLDEN, "coverage_dyadic.json")) as f:
        ex = json.load(f)
    m = np.array(ex["mass_num"], dtype=np.float64) / ex["mass_den"]
    for g_str, lst in ex["cuts"].items():
        got, k, _, _ = O.coverage_cut(m, float(g_str))
        assert got.tolist() == lst


@pytest.mark.parametrize("n", [1, 2, 5, 9, 12])
def test_cut_brute_force_minimal_and_reaching(n):
    for trial in range(6):
        m = RNG.dirichlet(np.full(n, 0.5))
        if trial == 0 and n > 2:
            m[1] = m[2]                      # an exact tie
        for gamma in (0.3, 0.5, 0.9, 0.98, 0.99, 1.0):
            lst, k, _, _ = O.coverage_cut(m, gamma)
            Z = m.sum()
            best = None
            for r in range(1, n + 1):
                for sub in itertools.combinations(range(n), r):
                    if gamma >= 1.0:
                        if r == n:
                            best = r
                    elif m[list(sub)].sum() >= gamma * Z * (1 - 1e-12):
                        best = r
                    if best is not None:
                        break
                if best is not None:
                    break
            assert k == best
            assert len(lst) == k
            if gamma < 1:
                assert m[lst].sum() >= gamma * Z * (1 - 1e-12)
                out = np.setdiff1d(np.arange(n), lst)
                if out.size:
                    assert m[lst].min() >= m[out].max()


def test_cut_monotone_nested_and_degenerate():
    m = RNG.dirichlet(np.ones(300))
    prev = set()
    for gamma in np.linspace(0.05, 1.0, 40):
        lst, k, _, _ = O.coverage_cut(m, gamma)
        cur = set(lst.tolist())
        assert prev <= cur
        prev = cur
    assert len(prev) == 300
    assert O.coverage_cut(np.array([0.7]), 0.5)[0].tolist() == [0]
    dup = np.full(8, 1 / 8)                  # all tied: lowest indices first
    assert O.coverage_cut(dup, 0.5)[0].tolist() == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        O.coverage_cut(m, 0.0)


# ---------------------------------------------------------------- attention

def test_attention_brute_force_loops():
    G, T, D = 2, 7, 4
    q, K, V = RNG.standard_normal((G, D)), RNG.standard_normal((T, D)), RNG.standard_normal((T, D))
    s = 0.37
    o, lse = O.attend_tokens(q, K, V, s)
    for g in range(G):
        ls = [s * sum(q[g, d] * K[t, d] for d in range(D)) for t in range(T)]
        z = sum(math.exp(v) for v in ls)
        assert abs(lse[g] - math.log(z)) < 1e-12
        for d in range(D):
            ref = sum(math.exp(ls[t]) * V[t, d] for t in range(T)) / z
            assert abs(o[g, d] - ref) < 1e-12
    assert np.allclose(lse, logsumexp(s * q @ K.T, axis=1), atol=1e-12)


def test_attention_special_cases_and_permutation():
    D = 16
    q = RNG.standard_normal((3, D))
    k = RNG.standard_normal((1, D))
    v = RNG.standard_normal((1, D))
    o, lse = O.attend_tokens(q, k, v, 0.5)
    assert np.allclose(o, np.repeat(v, 3, 0), atol=1e-15)
    assert np.allclose(lse, 0.5 * q @ k[0], atol=1e-14)
    K = np.repeat(k, 10, 0)
    V = RNG.standard_normal((10, D))
    o, lse = O.attend_tokens(q, K, V, 0.5)
    assert np.allclose(o, V.mean(0)[None].repeat(3, 0), atol=1e-14)
    n, P = 9, 16
    Kp, Vp = RNG.standard_normal((n, P, D)), RNG.standard_normal((n, P, D))
    nv = RNG.integers(1, P + 1, size=n)
    a = O.attend_pages(q, Kp, Vp, nv, [0, 3, 5, 8], 0.3)
    b = O.attend_pages(q, Kp, Vp, nv, [8, 5, 0, 3], 0.3)
    assert np.allclose(a[0], b[0], atol=1e-13) and np.allclose(a[1], b[1], atol=1e-13)


def test_gamma_one_equals_dense_brute_force():
    n, P, D, G = 12, 16, 32, 4
    K = O.bf16_bits_to_f64(_bits(RNG.standard_normal((n, P, D))))
    V = O.bf16_bits_to_f64(_bits(RNG.standard_normal((n, P, D))))
    q = _bits(RNG.standard_normal((G, D)))
    nv = np.full(n, P)
    nv[-1] = 5
    lo, hi = O.summaries(_bits(K), nv)
    sel = O.select_unit(q, lo, hi, nv, 1 / math.sqrt(D), 1.0)
    assert sel["list"].tolist() == list(range(n))
    qf = O.bf16_bits_to_f64(q)
    o, lse = O.attend_pages(qf, K, V, nv, sel["list"], 1 / math.sqrt(D))
    toks = [(p, t) for p in range(n) for t in range(nv[p])]
    for g in range(G):
        ls = np.array([qf[g] @ K[p, t] / math.sqrt(D) for p, t in toks])
        w = np.exp(ls - ls.max())
        ref = sum(w[i] * V[p, t] for i, (p, t) in enumerate(toks)) / w.sum()
        assert np.allclose(o[g], ref, atol=1e-12)


def test_merge_partition_identity():
    T, D, G = 200, 16, 4
    q, K, V = RNG.standard_normal((G, D)), RNG.standard_normal((T, D)), RNG.standard_normal((T, D))
    o, lse = O.attend_tokens(q, K, V, 0.25)
    cuts = np.sort(RNG.choice(np.arange(1, T), size=6, replace=False))
    parts = np.split(np.arange(T), cuts)
    po, pl = zip(*[O.attend_tokens(q, K[ix], V[ix], 0.25) for ix in parts])
    mo, ml = O.merge_partials(np.stack(po), np.stack(pl))
    assert np.allclose(mo, o, atol=1e-12) and np.allclose(ml, lse, atol=1e-12)


# ---------------------------------------------------------------- acceptance

def test_list_acceptance_predicate():
    m = RNG.dirichlet(np.ones(200))
    gamma = 0.9
    lst, k, order, _ = O.coverage_cut(m, gamma)
    assert O.list_accepted(lst, m, gamma)[0]
    assert not O.list_accepted(lst[:-1], m, gamma)[0] or k == 1
    bigger = np.sort(np.append(lst, order[k]))
    assert not O.list_accepted(bigger, m, gamma)[0]
    swapped = np.sort(np.append(np.setdiff1d(lst, [order[0]]), order[-1]))
    assert not O.list_accepted(swapped, m, gamma)[0]
    assert not O.list_accepted(lst[::-1], m, gamma)[0] or k == 1
    assert O.list_accepted(np.arange(200), m, 1.0)[0]
    # a swap across an exact tie at the cut is accepted
    m2 = m.copy()
    m2[order[k]] = m2[order[k - 1]]
    lst2, k2, order2, _ = O.coverage_cut(m2, gamma)
    last_in = order2[k2 - 1]
    tie = [p for p in order2[k2:] if m2[p] == m2[last_in]]
    if tie:
        alt = np.sort(np.append(np.setdiff1d(lst2, [last_in]), tie[0]))
        assert O.list_accepted(alt, m2, gamma)[0]


# ---------------------------------------------------------------- LRU

def test_lru_matches_textbook_trace():
    C, n_units = 64, 400
    st = O.LRUState(C, n_units)
    steps = []
    cur = RNG.choice(n_units, size=50, replace=False)
    for t in range(40):
        steps.append(cur.copy())
        keep = RNG.choice(cur, size=45, replace=False)
        fresh = RNG.choice(np.setdiff1d(np.arange(n_units), keep), size=5, replace=False)
        cur = np.concatenate([keep, fresh])
    ref = O.textbook_lru_trace(C, steps)
    for t, units in enumerate(steps):
        r = O.resolve_step(st, units, t)
        hits, misses, ev, resident = ref[t]
        assert (r["hits"], r["misses"], r["evictions"], r["overflow"]) == (hits, misses, ev, 0)
        assert set(st.tag[st.tag >= 0].tolist()) == set(resident)
        for u in set(units.tolist()):
            assert st.tag[st.slot_of[u]] == u
        # placement rule: misses ascending <-> slots ascending
        placed = r["placed"]
        assert [u for u, _ in placed] == sorted(u for u, _ in placed)
        assert [s for _, s in placed] == sorted(s for _, s in placed)


@pytest.mark.parametrize("shift", [0, 1, 2, 3])
def test_bucketed_lru_matches_bucket_model(shift):
    """Victims ordered by (stamp >> s, unit id) against a model that keeps
    recency buckets explicitly; s = 0 is also the textbook LRU."""
    C, n_units = 40, 300
    rng = np.random.default_rng(11 + shift)
    steps = []
    cur = rng.choice(n_units, size=30, replace=False)
    for t in range(50):
        steps.append(cur.copy())
        keep = rng.choice(cur, size=24, replace=False)
        fresh = rng.choice(np.setdiff1d(np.arange(n_units), keep), size=6, replace=False)
        cur = np.concatenate([keep, fresh])
    ref = O.textbook_bucketed_trace(C, steps, shift)
    if shift == 0:
        assert [r[:3] for r in ref] == [r[:3] for r in O.textbook_lru_trace(C, steps)]
    st = O.LRUState(C, n_units)
    for t, units in enumerate(steps):
        r = O.resolve_step(st, units, t, recency_shift=shift)
        hits, misses, ev, resident = ref[t]
        assert (r["hits"], r["misses"], r["evictions"], r["overflow"]) == (hits, misses, ev, 0)
        assert set(st.tag[st.tag >= 0].tolist()) == set(resident)


def test_bucketed_lru_worked_case():
    """Three slots; units 2, 1, 3 used at steps 0, 1, 2, then unit 4 misses.
    Exact LRU evicts unit 2 (oldest); with buckets of 2 steps, units 2 and 1
    share the oldest bucket and the lower id, 1, goes."""
    steps = [[2], [1], [3], [4]]
    for shift, victim in ((0, 2), (1, 1)):
        st = O.LRUState(3, 10)
        for t, units in enumerate(steps):
            O.resolve_step(st, units, t, recency_shift=shift)
        assert set(st.tag.tolist()) == {1, 2, 3, 4} - {victim}


def test_pooled_cache_without_pressure_equals_per_request_caches():
    """A pool large enough never to evict gives every request the hits and
    misses it would have in a cache of its own; under pressure the pool is
    one LRU over pooled ids, matching the textbook trace on those ids."""
    B, H, MP = 3, 2, 50
    space = H * MP
    rng = np.random.default_rng(21)
    steps = []
    for t in range(12):
        steps.append([sorted(set(O.pooled_unit(b, h, int(p), H, MP)
                                 for h in range(H)
                                 for p in rng.choice(MP, size=6, replace=False)))
                      for b in range(B)])
    big = O.LRUState(B * space, B * space)
    own = [O.LRUState(space, space) for _ in range(B)]
    for t, per_req in enumerate(steps):
        r = O.resolve_pooled_step(big, per_req, t, space)
        assert r["evictions"] == 0
        for b in range(B):
            rb = O.resolve_step(own[b], [u - b * space for u in per_req[b]], t)
            assert r["per_request"][b].tolist() == [rb["hits"], rb["misses"], 0, 0]
    small = O.LRUState(40, B * space)
    ref = O.textbook_lru_trace(40, [[u for us in pr for u in us] for pr in steps])
    for t, per_req in enumerate(steps):
        r = O.resolve_pooled_step(small, per_req, t, space)
        hits, misses, ev, resident = ref[t]
        assert (r["hits"], r["misses"], r["evictions"]) == (hits, misses, ev)
        assert r["per_request"][:, :3].sum(0).tolist() == [hits, misses, ev]
        assert set(small.tag[small.tag >= 0].tolist()) == set(resident)


def test_lru_overflow_flagged():
    st = O.LRUState(8, 100)
    r = O.resolve_step(st, range(12), 0)
    assert r["overflow"] == 1 and r["misses"] == 12
    assert sum(1 for _, s in r["placed"] if s < 0) == 4
    with pytest.raises(OverflowError):
        O.textbook_lru_trace(8, [range(12)])


def test_topk_brute_force_and_agrees_with_coverage():
    for n in (1, 4, 9):
        m = RNG.dirichlet(np.ones(n))
        if n > 2:
            m[0] = m[2]                      # a tie: lower index first
        for k in range(1, n + 2):
            got = O.topk_cut(m, k).tolist()
            best = sorted(range(n), key=lambda p: (-m[p], p))[:min(k, n)]
            assert got == sorted(best)
    m = RNG.dirichlet(np.full(500, 0.3))
    for gamma in (0.5, 0.9, 0.99):
        lst, k, _, _ = O.coverage_cut(m, gamma)
        assert O.topk_cut(m, k).tolist() == lst.tolist()
