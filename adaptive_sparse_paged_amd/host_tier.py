"""Host-resident KV tier with a fixed-size HBM page cache per request.

State and buffers for sparse_hbm_cache_resolve, all caller-owned (torch
memory); the resolve itself -- finding hits, choosing replacements and
fetching the misses from host memory -- runs in the library's kernels on the stream,
so it can sit inside the captured decode graph.
"""

import ctypes

import torch

from . import lib
from .step import SparseDecodeStep

UNIT_ELEMS = 2 * 16 * 128   # K tile + V tile of one (page, KV head)


def _hip():
    # the HIP runtime torch loaded (one copy per process, by its soname)
    return ctypes.CDLL("libamdhip64.so.7")


_HIP_EVENT_DISABLE_TIMING = 0x2
_HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000


class DeviceEvent:
    """A HIP event that orders work between two streams of one device.
    Recorded with a device-scope release: a default event's record writes
    back and invalidates the caches for the host's sake, which cost about
    7 us of GPU time per record or wait in the host tier's steps.  Neither
    stream's work is read by the host through it.  Works under graph capture
    (record and wait become graph edges)."""

    def __init__(self):
        self._hip = _hip()
        self._ev = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(
            ctypes.byref(self._ev),
            ctypes.c_uint(_HIP_EVENT_DISABLE_TIMING | _HIP_EVENT_RELEASE_TO_DEVICE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self._hip.hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def wait(self, stream):
        """Make `stream` wait for the last record."""
        rc = self._hip.hipStreamWaitEvent(ctypes.c_void_p(stream.cuda_stream), self._ev,
                                          ctypes.c_uint(0))
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent failed ({rc})")

    def __del__(self):
        if getattr(self, "_ev", None) and self._ev.value:
            self._hip.hipEventDestroy(self._ev)


def device_view_ok(host):
    """Check that pinned host memory is addressable by the GPU at its own
    address (unified addressing); raises otherwise."""
    if not host.is_pinned():
        raise ValueError("host KV must be pinned host memory")
    hip = _hip()
    dptr = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(host.data_ptr()), 0)
    if rc != 0 or dptr.value != host.data_ptr():
        raise RuntimeError(f"pinned host memory is not device-addressable at its host address "
                           f"(hipHostGetDevicePointer rc={rc})")
    return True


class HbmPageCache:
    """HBM page cache over a pinned host KV pool [B][max_pages][Hkv][2][2048]
    (bf16 bits): per request `capacity` units (pooled=False), or one pool of
    `capacity` units shared by all requests (pooled=True).  recency_shift > 0
    compares stamps in buckets of 2**recency_shift steps (bucketed LRU)."""

    def __init__(self, dims, host_kv, capacity, device="cuda", recency_shift=0, pooled=False):
        device_view_ok(host_kv)
        B, H, MP = dims.batch, dims.num_kv_heads, dims.max_pages
        if tuple(host_kv.shape[:3]) != (B, MP, H):
            raise ValueError("host_kv must be [B][max_pages][Hkv][2][2048]")
        self.dims, self.host_kv, self.capacity = dims, host_kv, int(capacity)
        self.policy = lib.CachePolicy(int(recency_shift), 1 if pooled else 0)
        self.pooled = bool(pooled)
        slots = capacity if pooled else B * capacity
        tag_shape = (capacity,) if pooled else (B, capacity)
        i32 = dict(dtype=torch.int32, device=device)
        self.cache_kv = torch.zeros((slots, UNIT_ELEMS), dtype=torch.int16, device=device)
        self.slot_tag = torch.full(tag_shape, -1, **i32)
        self.slot_stamp = torch.full(tag_shape, -1, **i32)
        self.unit_slot = torch.full((B, H * MP), -1, **i32)
        self.stats = torch.zeros((B, 4), **i32)
        self.step_counter = torch.zeros(1, **i32)
        self.ws = torch.zeros(lib.cache_policy_workspace_bytes(dims, self.policy, capacity),
                              dtype=torch.uint8, device=device)

    def resolve(self, sel_counts, sel_pages, sel_phys, stream=None):
        """Resolve one step's lists; the step number comes from (and advances)
        the device counter, so this can be captured and replayed."""
        lib.hbm_cache_resolve_policy(self.dims, self.policy, sel_counts, sel_pages,
                                     self.host_kv, self.cache_kv, self.capacity, self.slot_tag,
                                     self.slot_stamp, self.unit_slot, self.step_counter,
                                     sel_phys, self.stats, self.ws, stream)

    def resolve_split(self, sel_counts, sel_pages, sel_phys, hit_phys, miss_lists=None,
                      stream=None):
        """The resolve alone (no copy): sel_phys as resolve() writes it, and
        hit_phys -- the slot of every entry that was resident before this
        step, -1 for the others; with miss_lists = (counts, pages, phys), also
        each unit's placed misses as a list.  fetch() must follow."""
        lib.hbm_cache_resolve_split(self.dims, self.policy, sel_counts, sel_pages, self.capacity,
                                    self.slot_tag, self.slot_stamp, self.unit_slot,
                                    self.step_counter, sel_phys, hit_phys, self.stats, self.ws,
                                    miss_lists, stream)

    def fetch(self, stream=None):
        """Copy the misses placed by the last resolve_split; advances the step."""
        lib.hbm_cache_fetch(self.dims, self.policy, self.host_kv, self.cache_kv, self.capacity,
                            self.step_counter, self.ws, stream)

    def pool_args(self):
        """(kv, stride_page, stride_head, pool_pages) for sparse_decode_attn."""
        return self.cache_kv, UNIT_ELEMS, 0, self.cache_kv.shape[0]


class SplitHostTierStep:
    """One host-tier layer whose attention over the hits runs while the
    misses cross PCIe.  A hit's slot is never a victim of the same step, so
    the hits are final once the resolve has run; attention over a partition
    of a list, merged by log-sum-exp, is attention over the whole list.

    One stream, three launches: the resolve (no copy; it also writes each
    unit's placed misses as a list); one grid in which the copying waves
    fetch the misses and attend them as they arrive, beside the attention's
    workers over the lists with hit_phys (misses read as empty pages); one
    merge of both sets of partials into out.  With every access a hit the
    copying waves exit at once.  Cache state, statistics and slot ids equal
    those of HbmPageCache.resolve; outputs equal the one-pass attention up to
    the order of the log-sum-exp merge.  It can be captured whole."""

    def __init__(self, dims, cache, gamma, workers=0, scale=None, device="cuda"):
        """workers: the hit attention's grid (0 = one workgroup per compute
        unit).  It keeps every unit's worker although the copies take
        FETCH_ATTN_COPY_GROUPS units first: with fewer workers (units minus
        the copies) the launch took 87 us instead of 78 with every access a
        hit."""
        self.dims, self.cache = dims, cache
        self.hits = SparseDecodeStep(dims, gamma, workers, scale=scale, device=device,
                                     offsets=False, scoring=False)
        # the miss lists, and the copying waves' partials (one worker per wave)
        self.miss = SparseDecodeStep(dims, gamma, lib.FETCH_ATTN_COPY_WAVES, scale=scale,
                                     device=device, offsets=False, scoring=False)
        self.hit_phys = torch.zeros_like(self.hits.buf.sel_phys)

    @property
    def sel_counts(self):
        return self.hits.buf.sel_counts

    @property
    def sel_pages(self):
        return self.hits.buf.sel_pages

    @property
    def sel_phys(self):
        return self.hits.buf.sel_phys

    def run(self, q, ctx_lens, out, out_lse):
        """One step on the lists in sel_counts / sel_pages."""
        h, m, c = self.hits, self.miss, self.cache
        hb, mb = h.buf, m.buf
        c.resolve_split(hb.sel_counts, hb.sel_pages, hb.sel_phys, self.hit_phys,
                        miss_lists=(mb.sel_counts, mb.sel_pages, mb.sel_phys))
        lib.hbm_cache_fetch_attn(self.dims, c.policy, c.host_kv, c.cache_kv, c.capacity,
                                 c.step_counter, q, ctx_lens, hb.sel_counts, hb.sel_pages,
                                 self.hit_phys, mb.sel_counts, mb.sel_pages, mb.sel_phys,
                                 h.scale, h.workers, hb.part_o, hb.part_lse, h.max_parts,
                                 mb.part_o, mb.part_lse)
        lib.merge_splits_pair(self.dims, hb.part_o, hb.part_lse, hb.sel_counts, h.workers,
                              mb.part_o, mb.part_lse, mb.sel_counts, lib.FETCH_ATTN_COPY_WAVES,
                              out, out_lse)
        return out, out_lse


class LayeredHostTierStep:
    """Host-tier attention over several layers that share one set of page
    lists per step ("HiSparse: Scaling Sparse Attention Decoding with
    Hierarchical KV Cache", abstract: for models whose layers share their
    selections, layer-wise prefetching overlaps the fetch of later layers'
    misses with earlier layers' work; exact, since only placement changes).

    Each layer has its own pinned host pool and HBM cache.  With
    prefetch=False every layer runs resolve+fetch then attention+merge on the
    current stream.  With prefetch=True:
      - a resolve stream runs every layer's resolve (hits, LRU, placement; no
        copy) in layer order, up front: they depend on the shared lists
        only, so none of them waits for a fetch or runs beside an attention
        (a resolve beside an attention slowed both about twofold);
      - an IO stream runs the layers' fetches back to back, each after its
        layer's resolve;
      - the current stream runs layer l's attention + merge after layer l's
        fetch, so the PCIe fetch of layer l+1 runs under it.
    Given the same worker count, both modes leave the same cache state and
    outputs bitwise the same.  With workers=0 the pipelined attention runs on
    all compute units but FETCH_GROUPS (the next layer's fetch takes whole
    units), so its lists split differently and outputs agree up to the
    rounding of the merge.  The step joins the other streams before it
    returns, so it can be captured whole."""

    def __init__(self, dims, host_pools, capacity, gamma, workers=0, scale=None,
                 prefetch=True, device="cuda"):
        self.dims = dims
        self.prefetch = bool(prefetch)
        self.caches = [HbmPageCache(dims, h, capacity, device) for h in host_pools]
        if workers == 0 and self.prefetch:
            # leave the next layer's fetch its compute units: it needs whole
            # units, and attention workers on every unit would hold it off
            # until the attention drains
            cus = torch.cuda.get_device_properties(torch.device(device)).multi_processor_count
            workers = max(1, cus - lib.FETCH_GROUPS)
        self.attn = SparseDecodeStep(dims, gamma, workers, scale=scale, device=device,
                                     offsets=False, scoring=False)
        # per-layer slot lists: later layers' resolves write while layer l attends
        self.sel_phys = [torch.zeros_like(self.attn.buf.sel_phys) for _ in host_pools]
        # the split resolve's hit slots, unused here (one buffer: the resolves
        # run one after another)
        self.hit_phys = torch.zeros_like(self.attn.buf.sel_phys)
        self.rs = torch.cuda.Stream(device=device)
        self.io = torch.cuda.Stream(device=device)
        self.start = DeviceEvent()
        self.resolved = [DeviceEvent() for _ in host_pools]
        self.ready = [DeviceEvent() for _ in host_pools]

    @property
    def sel_counts(self):
        return self.attn.buf.sel_counts

    @property
    def sel_pages(self):
        return self.attn.buf.sel_pages

    def run(self, qs, ctx_lens, outs, lses):
        """One step over every layer on the lists in sel_counts / sel_pages;
        qs[l], outs[l], lses[l]: layer l's queries and outputs."""
        st = self.attn
        counts, pages = st.buf.sel_counts, st.buf.sel_pages
        if not self.prefetch:
            for l, cache in enumerate(self.caches):
                cache.resolve(counts, pages, self.sel_phys[l])
                kv, sp, sh, pp = cache.pool_args()
                st.attend(qs[l], kv, sp, sh, pp, ctx_lens, outs[l], lses[l],
                          sel_phys=self.sel_phys[l])
            return
        cur = torch.cuda.current_stream()
        self.start.record(cur)
        self.start.wait(self.rs)
        for l, cache in enumerate(self.caches):
            cache.resolve_split(counts, pages, self.sel_phys[l], self.hit_phys, stream=self.rs)
            self.resolved[l].record(self.rs)
        for l, cache in enumerate(self.caches):
            self.resolved[l].wait(self.io)
            cache.fetch(stream=self.io)
            self.ready[l].record(self.io)
        # waiting for the last layer's fetch joins both other streams (the IO
        # stream waited for every resolve)
        for l, cache in enumerate(self.caches):
            self.ready[l].wait(cur)
            kv, sp, sh, pp = cache.pool_args()
            st.attend(qs[l], kv, sp, sh, pp, ctx_lens, outs[l], lses[l],
                      sel_phys=self.sel_phys[l])
