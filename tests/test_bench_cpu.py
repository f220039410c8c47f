"""bench.py's CPU-side pieces: the oracle timing leg and the parity summary it
reports for the timed run (fed here with the oracle's own lists and outputs,
then with a corrupted output), the chunk table and the byte accounting."""

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


def test_cpu_baseline_reports_parity_of_the_run():
    w = I.custom_workload("bench_cpu", 2, 8, 2, ("uniform", 300, 900), index=120)
    lens = I.context_lengths(w)
    counts, pages, out = _oracle_results(w, lens, 0.9)
    base, chk = bench.cpu_baseline(w, lens, 0.9, 0.2, gpu=(counts, pages, out))
    assert base["kind"] == "oracle" and base["cores"] == 1 and base["value"] > 0
    assert chk["units"] == w.batch * w.kv_heads
    assert chk["accepted"] == chk["units"] and chk["exact"] == chk["units"]
    assert chk["max_abs_err"] < 1e-6
    out_bad = out.copy()
    out_bad[1, 3, 7] += 0.5
    _, chk_bad = bench.cpu_baseline(w, lens, 0.9, 0.2, gpu=(counts, pages, out_bad))
    assert abs(chk_bad["max_abs_err"] - 0.5) < 1e-3
    base2, none = bench.cpu_baseline(w, lens, 0.9, 0.2)
    assert none is None and base2["unit"] == "us/layer"


def test_chunk_table_and_byte_accounting():
    for name in bench.DEFAULT_CHUNK:
        assert name in I.WORKLOADS
    # one unit: 8192 pages, all kept and full, chunk 512, G = 4, Hkv = 8
    n, k, t = 8192, 8192, 8192 * 16
    got = bench.counted_bytes(n, k, t, 4, 8, 512)
    parts = 2 * 16 * 4 * 129 * 4
    assert got == 512 * n + 32 * n + 4 * n / 8 + 512 * t + 16 * k + parts + 2 * 4 * 128 * 2 + 4 * 128 * 4 + 16
    assert bench.attn_bytes(k, t, 4, 512) == 512 * t + 8 * k + 4 * 128 * 2 + 16 * 4 * 129 * 4
