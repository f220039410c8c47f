"""bench.py's CPU-side pieces: the oracle timing legs (one thread and a
process pool) and the parity summary it reports for the timed run (fed here
with the oracle's own lists and outputs, then with a corrupted output and a
corrupted list), the attention plan's partial count and the byte accounting."""

import numpy as np

import bench
import oracle as O
from adaptive_sparse_paged_amd import inputs as I


def _oracle_results(w, lens, gamma):
    U = w.batch * w.kv_heads
    n_max = max(I.pages_of(int(L)) for L in lens)
    counts = np.zeros(U, dtype=np.int32)
    pages = np.full((U, n_max), -1, dtype=np.int32)
    out = np.zeros((w.batch, w.q_heads, 128), dtype=np.float32)
    for b in range(w.batch):
        for h in range(w.kv_heads):
            k, v, q, nv = I.unit_host(w, 0, b, h, int(lens[b]))
            lo, hi = O.summaries(k, nv)
            sel = O.select_unit(q, lo, hi, nv, w.scale, gamma)
            u = b * w.kv_heads + h
            counts[u] = sel["count"]
            pages[u, :sel["count"]] = sel["list"]
            o, _ = O.attend_pages(O.bf16_bits_to_f64(q), O.bf16_bits_to_f64(k),
                                  O.bf16_bits_to_f64(v), nv, sel["list"], w.scale)
            out[b, h * w.group:(h + 1) * w.group] = o
    return counts, pages, out


def test_cpu_baselines_and_parity_report():
    w = I.custom_workload("bench_cpu", 2, 8, 2, ("uniform", 300, 900), index=120)
    lens = I.context_lengths(w)
    counts, pages, out = _oracle_results(w, lens, 0.9)
    chk = bench.oracle_check(w, lens, 0.9, (counts, pages, out))
    assert chk["units"] == w.batch * w.kv_heads
    assert chk["accepted"] == chk["units"] and chk["exact"] == chk["units"]
    assert chk["max_abs_err"] < 1e-6
    out_bad = out.copy()
    out_bad[1, 3, 7] += 0.5
    chk_bad = bench.oracle_check(w, lens, 0.9, (counts, pages, out_bad))
    assert abs(chk_bad["max_abs_err"] - 0.5) < 1e-3
    pages_bad = pages.copy()
    pages_bad[0, 0] = pages[0, 1]          # a repeated page: not ascending
    assert bench.oracle_check(w, lens, 0.9, (counts, pages_bad, out))["accepted"] < chk["units"]
    base = bench.cpu_baseline(w, lens, 0.9, 0.2)
    assert base["kind"] == "oracle" and base["cores"] == 1 and base["value"] > 0
    pool = bench.cpu_baseline_pool(w, lens, 0.9, 0.2, 2)
    assert pool["kind"] == "oracle" and pool["cores"] == 2 and pool["value"] > 0
    assert pool["unit"] == base["unit"] == "us/layer"
    assert 1 <= bench.host_cores() <= 16


def _plan_brute(counts, workers, min_pages, unit_cost):
    """Workers whose range meets each unit's entries, by walking every
    position: a nonempty unit's unit_cost leading positions (marked -1) hold
    no entry."""
    k = np.asarray(counts, dtype=np.int64)
    unit = []
    for u, n in enumerate(k):
        if n > 0:
            unit += [-1] * unit_cost + [u] * int(n)
    unit = np.array(unit, dtype=np.int64)
    T = len(unit)
    if T == 0:
        return np.zeros(len(k), dtype=np.int64)
    W = min(workers, -(-T // min_pages))
    owner = np.zeros(T, dtype=np.int64)
    for w in range(W):
        owner[w * T // W:(w + 1) * T // W] = w
    return np.array([len(set(owner[unit == u])) for u in range(len(k))], dtype=np.int64)


def test_plan_segments_match_a_walk_over_positions():
    rng = np.random.default_rng(3)
    for trial in range(200):
        U = int(rng.integers(1, 40))
        counts = rng.integers(0, 300, size=U) * (rng.random(U) < 0.8)
        workers = int(rng.integers(1, 80))
        minp = int(rng.choice([1, 7, 32]))
        c = int(rng.choice([0, 5, 12]))
        assert np.array_equal(bench.plan_segments(counts, workers, minp, c),
                              _plan_brute(counts, workers, minp, c)), (trial, counts, workers,
                                                                       minp, c)
    assert bench.plan_segments([0, 0], 4, 32, 12).tolist() == [0, 0]
    # cap clamps every list before the plan
    assert np.array_equal(bench.plan_segments([500, 10], 8, 1, 12, cap=100),
                          _plan_brute([100, 10], 8, 1, 12))


def test_byte_accounting():
    # one unit: 8192 pages, all kept and full, split into 16 partials, G = 4, Hkv = 8
    n, k, t = 8192, 8192, 8192 * 16
    got = bench.counted_bytes(n, k, t, 4, 8, 16)
    parts = 2 * 16 * 4 * 129 * 4
    assert got == 512 * n + 32 * n + 4 * n / 8 + 512 * t + 16 * k + parts + 2 * 4 * 128 * 2 + 4 * 128 * 4 + 16
    assert bench.attn_bytes(k, t, 4, 16) == 512 * t + 8 * k + 4 * 128 * 2 + 16 * 4 * 129 * 4
