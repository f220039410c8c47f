"""Host-resident KV tier with a fixed-size HBM page cache per request.

State and buffers for sparse_hbm_cache_resolve, all caller-owned (torch
memory); the resolve itself -- hit detection, LRU replacement and the
host-to-device fetch of misses -- runs in the library's kernels on the stream,
so it can sit inside the captured decode graph.
"""

import ctypes

import torch

from . import lib

UNIT_ELEMS = 2 * 16 * 128   # K tile + V tile of one (page, KV head)


def device_view_ok(host):
    """Check that pinned host memory is addressable by the GPU at its own
    address (unified addressing); raises otherwise."""
    if not host.is_pinned():
        raise ValueError("host KV must be pinned host memory")
    hip = ctypes.CDLL("libamdhip64.so.7")
    dptr = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(host.data_ptr()), 0)
    if rc != 0 or dptr.value != host.data_ptr():
        raise RuntimeError(f"pinned host memory is not device-addressable at its host address "
                           f"(hipHostGetDevicePointer rc={rc})")
    return True


class HbmPageCache:
    """Per-request HBM caches of `capacity` units over a pinned host KV pool
    [B][max_pages][Hkv][2][2048] (bf16 bits)."""

    def __init__(self, dims, host_kv, capacity, device="cuda"):
        device_view_ok(host_kv)
        B, H, MP = dims.batch, dims.num_kv_heads, dims.max_pages
        if tuple(host_kv.shape[:3]) != (B, MP, H):
            raise ValueError("host_kv must be [B][max_pages][Hkv][2][2048]")
        self.dims, self.host_kv, self.capacity = dims, host_kv, int(capacity)
        i32 = dict(dtype=torch.int32, device=device)
        self.cache_kv = torch.zeros((B * capacity, UNIT_ELEMS), dtype=torch.int16, device=device)
        self.slot_tag = torch.full((B, capacity), -1, **i32)
        self.slot_stamp = torch.full((B, capacity), -1, **i32)
        self.unit_slot = torch.full((B, H * MP), -1, **i32)
        self.stats = torch.zeros((B, 4), **i32)
        self.step_counter = torch.zeros(1, **i32)
        self.ws = torch.zeros(lib.cache_workspace_bytes(dims, capacity), dtype=torch.uint8,
                              device=device)

    def resolve(self, sel_counts, sel_pages, sel_phys, stream=None):
        """Resolve one step's lists; the step number comes from (and advances)
        the device counter, so this can be captured and replayed."""
        lib.hbm_cache_resolve(self.dims, sel_counts, sel_pages, self.host_kv, self.cache_kv,
                              self.capacity, self.slot_tag, self.slot_stamp, self.unit_slot,
                              self.step_counter, sel_phys, self.stats, self.ws, stream)

    def pool_args(self):
        """(kv, stride_page, stride_head, pool_pages) for sparse_decode_attn."""
        return self.cache_kv, UNIT_ELEMS, 0, self.cache_kv.shape[0]
