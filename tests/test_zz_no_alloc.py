"""The allocation-free attention entry point, sparse_decode_attn_merge_noalloc,
through the C ABI: its outputs must equal those of sparse_decode_attn_merge
(same kernels, partials in a caller workspace) bitwise, on two calls in a
row, the second with a smaller step, and agree with the fp64 oracle.  It
rejects a step whose partials exceed its device array, with no launch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from adaptive_sparse_paged_amd import inputs as I
from adaptive_sparse_paged_amd import lib

from _gpu_case import ATTN_TOL, GpuLayer, say

pytestmark = pytest.mark.gpu


def _both(layer, st, workers):
    """Outputs of the workspace entry point and of the allocation-free one."""
    li = layer.li
    st.score_select(li.q, layer.summ, li.pool_pages, li.page_table, li.ctx_lens)
    args = (layer.dims, li.q, li.kv_pool, layer.stride_page, layer.stride_head, li.pool_pages,
            li.ctx_lens, st.buf.sel_counts, st.buf.sel_pages, st.buf.sel_phys, st.scale, workers)
    ref = (torch.full_like(st.buf.out, 7.0), torch.full_like(st.buf.out_lse, 7.0))
    lib.decode_attn_merge(*args, st.buf.part_o, st.buf.part_lse, st.max_parts, *ref)
    got = (torch.full_like(st.buf.out, -7.0), torch.full_like(st.buf.out_lse, -7.0))
    lib.decode_attn_merge_noalloc(*args, *got)
    torch.cuda.synchronize()
    return ref, got


def _oracle_check(layer, st, out, units):
    w = layer.w
    G = w.group
    worst = 0.0
    for b, h in units:
        un = layer.unit_oracle(b, h)
        u = b * w.kv_heads + h
        lst = st.buf.sel_pages[u, :int(st.buf.sel_counts[u])].cpu().numpy()
        o_ref, _ = O.attend_pages(O.bf16_bits_to_f64(un["q"]), O.bf16_bits_to_f64(un["k"]),
                                  O.bf16_bits_to_f64(un["v"]), un["nv"], lst, w.scale)
        o = out[b, h * G:(h + 1) * G].double().cpu().numpy()
        worst = max(worst, float(np.abs(o - o_ref).max()))
    assert worst <= ATTN_TOL
    return worst


def test_noalloc_equals_workspace_entry_point_twice(gpu_lib):
    big = I.custom_workload("noalloc_big", 6, 32, 8, ("uniform", 2000, 40000),
                            alpha=("uniform", 0.5, 6), index=140)
    small = I.custom_workload("noalloc_small", 2, 8, 2, ("uniform", 100, 3000),
                              alpha=("uniform", 0.5, 6), index=141)
    for w, workers in ((big, 0), (small, 5)):        # the second call is the smaller step
        say(f"[noalloc] B={w.batch} Hq={w.q_heads} Hkv={w.kv_heads} workers={workers}")
        layer = GpuLayer(w)
        st = layer.step(0.95, workers)
        ref, got = _both(layer, st, workers)
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
        worst = _oracle_check(layer, st, got[0], [(0, 0), (w.batch - 1, w.kv_heads - 1)])
        say(f"  bitwise equal to the workspace entry point; max err vs oracle {worst:.1e}")


def test_noalloc_rejects_a_step_beyond_its_array(gpu_lib):
    # (U + W) * G * 129 * 4 bytes of partials: 16384 units of G = 4 need 33 MiB
    d = lib.make_dims(2048, 32, 8, 64)
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: the size check fails first
    L = lib.load()
    r = L.sparse_decode_attn_merge_noalloc(ctypes.byref(d), fake, fake, 8192, 4096, 100, fake,
                                           fake, fake, fake, 0.1, 16, fake, fake, None)
    assert r == lib.ERR_WORKSPACE
    assert (2048 * 8 + 16) * 4 * 129 * 4 > lib.NOALLOC_SCRATCH_BYTES
