"""Python binding of the C ABI in include/sparse_paged.h (ctypes).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libsparse_paged.so.  torch supplies device memory and the stream.
The library is looked for next to this file; when it is missing, ``load()``
raises -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_paged.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)

EXPORTS = (
    "sparse_version",
    "sparse_status_string",
    "sparse_build_page_summaries",
    "sparse_score_pages",
    "sparse_select_workspace_bytes",
    "sparse_select_coverage",
    "sparse_decode_max_parts",
    "sparse_decode_attn",
    "sparse_merge_splits",
    "sparse_merge_splits_pair",
    "sparse_cache_workspace_bytes",
    "sparse_hbm_cache_resolve",
    "sparse_select_topk",
    "sparse_append_tokens",
    "sparse_cache_policy_workspace_bytes",
    "sparse_hbm_cache_resolve_policy",
    "sparse_read_blocks",
    "sparse_hbm_cache_resolve_split",
    "sparse_hbm_cache_fetch",
    "sparse_hbm_cache_fetch_attn",
    "sparse_split_misses",
    "sparse_lse_combine",
    "sparse_decode_attn_merge",
    "sparse_decode_attn_merge_noalloc",
)


class SparseError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} returned {code} ({msg})")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("max_list_pages", ctypes.c_int32),
    ]


def make_dims(batch, q_heads, kv_heads, max_pages, head_dim=128, page_size=16,
              max_list_pages=0):
    """max_list_pages: 0, or a bound on every page list's length (the
    attention and merge clamp each list's count to it)."""
    return Dims(batch, q_heads, kv_heads, head_dim, page_size, max_pages, max_list_pages)


class CachePolicy(ctypes.Structure):
    _fields_ = [
        ("recency_shift", ctypes.c_int32),
        ("pooled", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_D = ctypes.POINTER(Dims)
_CP = ctypes.POINTER(CachePolicy)

_SIGS = {
    "sparse_version": (ctypes.c_char_p, []),
    "sparse_status_string": (ctypes.c_char_p, [_I32]),
    "sparse_build_page_summaries": (_I32, [_D, _P, _I64, _I64, _I64, _P, _P, _I32, _P, _P]),
    "sparse_score_pages": (_I32, [_D, _P, _P, _I64, _P, _P, _F, _P, _P]),
    "sparse_select_workspace_bytes": (ctypes.c_size_t, [_D]),
    "sparse_select_coverage": (_I32, [_D, _P, _P, _P, _F, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]),
    "sparse_decode_max_parts": (_I64, [_D, _I32]),
    "sparse_decode_attn": (_I32, [_D, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _F, _I32,
                                  _P, _P, _I64, _P]),
    "sparse_merge_splits": (_I32, [_D, _P, _P, _P, _I32, _P, _P, _P]),
    "sparse_merge_splits_pair": (_I32, [_D, _P, _P, _P, _I32, _P, _P, _P, _I32, _P, _P, _P]),
    "sparse_cache_workspace_bytes": (ctypes.c_size_t, [_D, _I32]),
    "sparse_select_topk": (_I32, [_D, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
    "sparse_append_tokens": (_I32, [_D, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "sparse_hbm_cache_resolve": (_I32, [_D, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "sparse_cache_policy_workspace_bytes": (ctypes.c_size_t, [_D, _CP, _I32]),
    "sparse_hbm_cache_resolve_policy": (_I32, [_D, _CP, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                                               _P, _P, ctypes.c_size_t, _P]),
    "sparse_read_blocks": (_I32, [_P, _I64, _P, _I64, _P, _P]),
    "sparse_hbm_cache_resolve_split": (_I32, [_D, _CP, _P, _P, _I32, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "sparse_hbm_cache_fetch": (_I32, [_D, _CP, _P, _P, _I32, _P, _P, ctypes.c_size_t, _P]),
    "sparse_hbm_cache_fetch_attn": (_I32, [_D, _CP, _P, _P, _I32, _P, _P, _P, _P, _P, _P, _P,
                                           _P, _P, _F, _I32, _P, _P, _I64, _P, _P, _P]),
    "sparse_split_misses": (_I32, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sparse_lse_combine": (_I32, [_D, _P, _P, _P, _P, _P, _P, _P]),
    "sparse_decode_attn_merge": (_I32, [_D, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _F, _I32,
                                        _P, _P, _I64, _P, _P, _P]),
    "sparse_decode_attn_merge_noalloc": (_I32, [_D, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _F,
                                                _I32, _P, _P, _P]),
}

_lib = None


def load(path=LIB_PATH):
    """Load libsparse_paged.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m adaptive_sparse_paged_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, code):
    if code != OK:
        msg = load().sparse_status_string(code).decode()
        raise SparseError(fn, code, msg)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def version():
    return load().sparse_version().decode()


def build_page_summaries(dims, kv, stride_page, stride_head, pool_pages, pages, valid, summ,
                         stream=None):
    _dev(kv, pages, valid, summ)
    n = pages.numel()
    _check("sparse_build_page_summaries", load().sparse_build_page_summaries(
        ctypes.byref(dims), _ptr(kv), stride_page, stride_head, pool_pages, _ptr(pages),
        _ptr(valid), n, _ptr(summ), _stream(stream)))


def score_pages(dims, q, summ, pool_pages, page_table, ctx_lens, scale, logits, stream=None):
    _dev(q, summ, page_table, ctx_lens, logits)
    _check("sparse_score_pages", load().sparse_score_pages(
        ctypes.byref(dims), _ptr(q), _ptr(summ), pool_pages, _ptr(page_table), _ptr(ctx_lens),
        scale, _ptr(logits), _stream(stream)))


def select_workspace_bytes(dims):
    return int(load().sparse_select_workspace_bytes(ctypes.byref(dims)))


def select_coverage(dims, logits, ctx_lens, page_table, gamma, sel_counts, sel_offsets,
                    sel_pages, sel_phys, ws, stream=None):
    """sel_offsets / ws may both be None (no whole-batch prefix sum)."""
    _dev(logits, ctx_lens, page_table, sel_counts, sel_offsets, sel_pages, sel_phys, ws)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("sparse_select_coverage", load().sparse_select_coverage(
        ctypes.byref(dims), _ptr(logits), _ptr(ctx_lens), _ptr(page_table), gamma,
        _ptr(sel_counts), _ptr(sel_offsets), _ptr(sel_pages), _ptr(sel_phys), _ptr(ws), nbytes,
        _stream(stream)))


ATTN_MIN_WORKER_PAGES = 32   # SPARSE_ATTN_MIN_WORKER_PAGES
ATTN_UNIT_COST_PAGES = 12    # SPARSE_ATTN_UNIT_COST_PAGES


def decode_max_parts(dims, workers=0):
    """Partial slots of one attention step: U + W (W = workers, or the current
    device's compute units when 0); -1 when invalid."""
    return int(load().sparse_decode_max_parts(ctypes.byref(dims), workers))


def decode_attn(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens, sel_counts,
                sel_pages, sel_phys, scale, workers, part_o, part_lse, max_parts, stream=None):
    _dev(q, kv, ctx_lens, sel_counts, sel_pages, sel_phys, part_o, part_lse)
    _check("sparse_decode_attn", load().sparse_decode_attn(
        ctypes.byref(dims), _ptr(q), _ptr(kv), stride_page, stride_head, pool_pages,
        _ptr(ctx_lens), _ptr(sel_counts), _ptr(sel_pages), _ptr(sel_phys), scale, workers,
        _ptr(part_o), _ptr(part_lse), max_parts, _stream(stream)))


def decode_attn_merge(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens, sel_counts,
                      sel_pages, sel_phys, scale, workers, part_o, part_lse, max_parts, out,
                      out_lse, stream=None):
    """decode_attn then merge_splits in one call (the partials in part_o / part_lse)."""
    _dev(q, kv, ctx_lens, sel_counts, sel_pages, sel_phys, part_o, part_lse, out, out_lse)
    _check("sparse_decode_attn_merge", load().sparse_decode_attn_merge(
        ctypes.byref(dims), _ptr(q), _ptr(kv), stride_page, stride_head, pool_pages,
        _ptr(ctx_lens), _ptr(sel_counts), _ptr(sel_pages), _ptr(sel_phys), scale, workers,
        _ptr(part_o), _ptr(part_lse), max_parts, _ptr(out), _ptr(out_lse), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20   # SPARSE_NOALLOC_SCRATCH_BYTES
FETCH_ATTN_COPY_GROUPS = 64         # SPARSE_FETCH_ATTN_COPY_GROUPS
FETCH_ATTN_COPY_WAVES = 4 * FETCH_ATTN_COPY_GROUPS   # SPARSE_FETCH_ATTN_COPY_WAVES
FETCH_GROUPS = 32                   # SPARSE_FETCH_GROUPS


def decode_attn_merge_noalloc(dims, q, kv, stride_page, stride_head, pool_pages, ctx_lens,
                              sel_counts, sel_pages, sel_phys, scale, workers, out, out_lse,
                              stream=None):
    """decode_attn_merge with the partials in the library's own device array
    (no allocation; steps up to NOALLOC_SCRATCH_BYTES of partials)."""
    _dev(q, kv, ctx_lens, sel_counts, sel_pages, sel_phys, out, out_lse)
    _check("sparse_decode_attn_merge_noalloc", load().sparse_decode_attn_merge_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(kv), stride_page, stride_head, pool_pages,
        _ptr(ctx_lens), _ptr(sel_counts), _ptr(sel_pages), _ptr(sel_phys), scale, workers,
        _ptr(out), _ptr(out_lse), _stream(stream)))


def merge_splits(dims, part_o, part_lse, sel_counts, workers, out, out_lse, stream=None):
    _dev(part_o, part_lse, sel_counts, out, out_lse)
    _check("sparse_merge_splits", load().sparse_merge_splits(
        ctypes.byref(dims), _ptr(part_o), _ptr(part_lse), _ptr(sel_counts), workers,
        _ptr(out), _ptr(out_lse), _stream(stream)))


def merge_splits_pair(dims, part_o_a, part_lse_a, sel_counts_a, workers_a, part_o_b, part_lse_b,
                      sel_counts_b, workers_b, out, out_lse, stream=None):
    """One merge over the partials of two disjoint sets of lists."""
    _dev(part_o_a, part_lse_a, sel_counts_a, part_o_b, part_lse_b, sel_counts_b, out, out_lse)
    _check("sparse_merge_splits_pair", load().sparse_merge_splits_pair(
        ctypes.byref(dims), _ptr(part_o_a), _ptr(part_lse_a), _ptr(sel_counts_a), workers_a,
        _ptr(part_o_b), _ptr(part_lse_b), _ptr(sel_counts_b), workers_b, _ptr(out),
        _ptr(out_lse), _stream(stream)))


def cache_workspace_bytes(dims, capacity):
    return int(load().sparse_cache_workspace_bytes(ctypes.byref(dims), capacity))


def hbm_cache_resolve(dims, sel_counts, sel_pages, host_kv, cache_kv, capacity, slot_tag,
                      slot_stamp, unit_slot, step_counter, sel_phys, stats, ws, stream=None):
    """host_kv must be pinned host memory (torch pin_memory) addressable by the GPU;
    step_counter is a 1-element int32 device tensor the call reads and advances."""
    _dev(sel_counts, sel_pages, cache_kv, slot_tag, slot_stamp, unit_slot, step_counter,
         sel_phys, stats, ws)
    if not host_kv.is_pinned():
        raise ValueError("host_kv must be pinned host memory")
    nbytes = ws.numel() * ws.element_size()
    _check("sparse_hbm_cache_resolve", load().sparse_hbm_cache_resolve(
        ctypes.byref(dims), _ptr(sel_counts), _ptr(sel_pages), _ptr(host_kv), _ptr(cache_kv),
        capacity, _ptr(slot_tag), _ptr(slot_stamp), _ptr(unit_slot), _ptr(step_counter),
        _ptr(sel_phys),
        _ptr(stats), _ptr(ws), nbytes, _stream(stream)))


def cache_policy_workspace_bytes(dims, policy, capacity):
    return int(load().sparse_cache_policy_workspace_bytes(ctypes.byref(dims),
                                                          ctypes.byref(policy), capacity))


def hbm_cache_resolve_policy(dims, policy, sel_counts, sel_pages, host_kv, cache_kv, capacity,
                             slot_tag, slot_stamp, unit_slot, step_counter, sel_phys, stats, ws,
                             stream=None):
    """hbm_cache_resolve under a CachePolicy (bucketed recency, pooled slots)."""
    _dev(sel_counts, sel_pages, cache_kv, slot_tag, slot_stamp, unit_slot, step_counter,
         sel_phys, stats, ws)
    if not host_kv.is_pinned():
        raise ValueError("host_kv must be pinned host memory")
    nbytes = ws.numel() * ws.element_size()
    _check("sparse_hbm_cache_resolve_policy", load().sparse_hbm_cache_resolve_policy(
        ctypes.byref(dims), ctypes.byref(policy), _ptr(sel_counts), _ptr(sel_pages),
        _ptr(host_kv), _ptr(cache_kv), capacity, _ptr(slot_tag), _ptr(slot_stamp),
        _ptr(unit_slot), _ptr(step_counter), _ptr(sel_phys), _ptr(stats), _ptr(ws), nbytes,
        _stream(stream)))


def select_topk(dims, logits, ctx_lens, page_table, k_pages, sel_counts, sel_offsets,
                sel_pages, sel_phys, ws, stream=None):
    _dev(logits, ctx_lens, page_table, sel_counts, sel_offsets, sel_pages, sel_phys, ws)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("sparse_select_topk", load().sparse_select_topk(
        ctypes.byref(dims), _ptr(logits), _ptr(ctx_lens), _ptr(page_table), k_pages,
        _ptr(sel_counts), _ptr(sel_offsets), _ptr(sel_pages), _ptr(sel_phys), _ptr(ws), nbytes,
        _stream(stream)))


def append_tokens(dims, k_new, v_new, kv, stride_page, stride_head, pool_pages, page_table,
                  ctx_lens, summ, stream=None):
    _dev(k_new, v_new, kv, page_table, ctx_lens, summ)
    _check("sparse_append_tokens", load().sparse_append_tokens(
        ctypes.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(kv), stride_page, stride_head,
        pool_pages, _ptr(page_table), _ptr(ctx_lens), _ptr(summ), _stream(stream)))


READ_BLOCKS_GROUPS = 4096   # SPARSE_READ_BLOCKS_GROUPS


def read_blocks(pool, pool_blocks, order, xor_out, stream=None):
    """Measurement helper: read the 8 KiB blocks order[:] of pool.  xor_out
    (int32 [READ_BLOCKS_GROUPS]) receives one XOR fold per workgroup; their
    XOR is the XOR of every 32-bit word of the listed blocks."""
    _dev(pool, order, xor_out)
    if xor_out.numel() * xor_out.element_size() < 4 * READ_BLOCKS_GROUPS:
        raise ValueError(f"xor_out must hold {READ_BLOCKS_GROUPS} 32-bit words")
    _check("sparse_read_blocks", load().sparse_read_blocks(
        _ptr(pool), int(pool_blocks), _ptr(order), order.numel(), _ptr(xor_out),
        _stream(stream)))


def hbm_cache_resolve_split(dims, policy, sel_counts, sel_pages, capacity, slot_tag, slot_stamp,
                            unit_slot, step_counter, sel_phys, hit_phys, stats, ws,
                            miss_lists=None, stream=None):
    """miss_lists: None, or (miss_counts, miss_pages, miss_phys) to receive each
    unit's placed misses."""
    _dev(sel_counts, sel_pages, slot_tag, slot_stamp, unit_slot, step_counter, sel_phys,
         hit_phys, stats, ws)
    mc = mp = mph = None
    if miss_lists is not None:
        mc, mp, mph = miss_lists
        _dev(mc, mp, mph)
    _check("sparse_hbm_cache_resolve_split", load().sparse_hbm_cache_resolve_split(
        ctypes.byref(dims), ctypes.byref(policy), _ptr(sel_counts), _ptr(sel_pages), capacity,
        _ptr(slot_tag), _ptr(slot_stamp), _ptr(unit_slot), _ptr(step_counter), _ptr(sel_phys),
        _ptr(hit_phys), _ptr(stats), _ptr(mc), _ptr(mp), _ptr(mph), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def hbm_cache_fetch(dims, policy, host_kv, cache_kv, capacity, step_counter, ws, stream=None):
    _dev(cache_kv, step_counter, ws)
    if not host_kv.is_pinned():
        raise ValueError("host_kv must be pinned host memory")
    _check("sparse_hbm_cache_fetch", load().sparse_hbm_cache_fetch(
        ctypes.byref(dims), ctypes.byref(policy), _ptr(host_kv), _ptr(cache_kv), capacity,
        _ptr(step_counter), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def hbm_cache_fetch_attn(dims, policy, host_kv, cache_kv, capacity, step_counter, q, ctx_lens,
                         sel_counts, sel_pages, hit_phys, miss_counts, miss_pages, miss_phys,
                         scale, workers, part_o, part_lse, max_parts, miss_part_o, miss_part_lse,
                         stream=None):
    """The copies of the miss lists, attended in the copying waves (partials
    miss_part_o / miss_part_lse, FETCH_ATTN_COPY_WAVES workers), and
    decode_attn over (sel_counts, sel_pages, hit_phys) on the cache pool, in
    one launch."""
    _dev(cache_kv, step_counter, q, ctx_lens, sel_counts, sel_pages, hit_phys, miss_counts,
         miss_pages, miss_phys, part_o, part_lse, miss_part_o, miss_part_lse)
    if not host_kv.is_pinned():
        raise ValueError("host_kv must be pinned host memory")
    U = dims.batch * dims.num_kv_heads
    G = dims.num_q_heads // dims.num_kv_heads
    if (miss_part_o.numel() < (U + FETCH_ATTN_COPY_WAVES) * G * 128
            or miss_part_lse.numel() < (U + FETCH_ATTN_COPY_WAVES) * G):
        raise ValueError("miss partials hold U + FETCH_ATTN_COPY_WAVES slots")
    _check("sparse_hbm_cache_fetch_attn", load().sparse_hbm_cache_fetch_attn(
        ctypes.byref(dims), ctypes.byref(policy), _ptr(host_kv), _ptr(cache_kv), capacity,
        _ptr(step_counter), _ptr(q), _ptr(ctx_lens), _ptr(sel_counts), _ptr(sel_pages),
        _ptr(hit_phys), _ptr(miss_counts), _ptr(miss_pages), _ptr(miss_phys), scale, workers,
        _ptr(part_o), _ptr(part_lse), max_parts, _ptr(miss_part_o), _ptr(miss_part_lse),
        _stream(stream)))


def split_misses(dims, sel_counts, sel_pages, sel_phys, hit_phys, miss_counts, miss_pages,
                 miss_phys, stream=None):
    _dev(sel_counts, sel_pages, sel_phys, hit_phys, miss_counts, miss_pages, miss_phys)
    _check("sparse_split_misses", load().sparse_split_misses(
        ctypes.byref(dims), _ptr(sel_counts), _ptr(sel_pages), _ptr(sel_phys), _ptr(hit_phys),
        _ptr(miss_counts), _ptr(miss_pages), _ptr(miss_phys), _stream(stream)))


def lse_combine(dims, out_a, lse_a, out_b, lse_b, out, out_lse, stream=None):
    _dev(out_a, lse_a, out_b, lse_b, out, out_lse)
    _check("sparse_lse_combine", load().sparse_lse_combine(
        ctypes.byref(dims), _ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out),
        _ptr(out_lse), _stream(stream)))
