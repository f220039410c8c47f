"""The seeded input generator: published known answers, determinism, and
per-unit / per-page regeneration."""

import numpy as np
import torch

from adaptive_sparse_paged_amd import inputs as I


def test_splitmix64_known_answers():
    # First outputs of splitmix64 seeded with 1234567 (the reference sequence
    # published with Vigna's splitmix64.c test harness).
    z = I.splitmix64_stream(1234567, 0, 5)
    got = [int(x) & ((1 << 64) - 1) for x in z]
    assert got == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                   4593380528125082431, 16408922859458223821]
    assert I.mix64_int(1234567 + 0x9E3779B97F4A7C15) == got[0]


def test_normal_table_symmetric_and_standard():
    t = I.bf16_bits_to_float(I.normal_table()).double().numpy()
    assert np.all(np.diff(t) >= 0)
    assert np.array_equal(t, -t[::-1])
    assert abs(t.mean()) < 1e-12 and abs(t.std() - 1) < 2e-3


def test_stream_slices_regenerate():
    key = I.stream_key(3, 1, 4)
    full = I.normal_bf16(key, 0, 5000)
    for s, c in [(0, 1), (1, 3), (7, 129), (4095, 900)]:
        assert torch.equal(I.normal_bf16(key, s, c), full[s:s + c])


def test_unit_tiles_regenerate_and_queries_deterministic():
    w = I.WORKLOADS["serving_b64"]
    lens = I.context_lengths(w)
    assert lens.min() >= 4096 and lens.max() <= 131072 and (lens % 16 != 0).any()
    n = I.pages_of(lens[0])
    full = I.unit_kv_bits(w, 0, 0, 3, n, 1)
    some = I.unit_kv_bits(w, 0, 0, 3, n, 1, pages=[0, 5, n - 1])
    assert torch.equal(some[1], full[5]) and torch.equal(some[2], full[n - 1])
    q1 = I.unit_query_bits(w, 0, 0, 3, lens[0])
    q2 = I.unit_query_bits(w, 0, 0, 3, lens[0])
    assert torch.equal(q1, q2) and q1.shape == (4, 128)
    nv = I.valid_tokens(lens[0])
    assert nv.sum() == lens[0] and nv[:-1].min() == 16


def test_build_layer_layout():
    w = I.custom_workload("t", 2, 8, 2, ("uniform", 40, 100))
    li = I.build_layer(w, 0, "cpu")
    lens = li.ctx_lens.numpy()
    for b in range(2):
        n = I.pages_of(lens[b])
        phys = li.page_table[b, :n].long()
        k = I.unit_kv_bits(w, 0, b, 1, n, 0)
        v = I.unit_kv_bits(w, 0, b, 1, n, 1)
        assert torch.equal(li.kv_pool[phys, 1, 0].view(n, 16, 128), k)
        assert torch.equal(li.kv_pool[phys, 1, 1].view(n, 128, 16).transpose(1, 2), v)
        assert (li.page_table[b, n:] == -1).all()
    assert sorted(li.page_table[li.page_table >= 0].tolist()) == list(range(li.pool_pages))
